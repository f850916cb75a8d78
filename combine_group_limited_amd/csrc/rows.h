// rows.h -- per-piece row work shared by the dispatch kernels: one lane's
// piece of a token's row is read once and stored to each of the token's k
// receive rows.  The receive-row index of pick j lives in lane j of
// `my_slot` (broadcast with v_readlane, so row addresses are wave-uniform and
// each row gets its own buffer resource); rows outside [0, nrows) are
// skipped.
#pragma once

#include "device.h"

namespace ep {

// FP8: a lane owns 16 consecutive channels (`chunk` counts 16-channel
// pieces), so a 128-channel scale block is 8 adjacent lanes and its amax a
// 3-step butterfly.  All 8 lanes of a block must store together.
// Per block: a = max(amax, 1e-4), inv = 448 / a, scale = a / 448,
// code = e4m3_rne(x * inv).  x is read with default caching, the codes are
// streamed (nt).  Loading and storing are separate steps so that a caller
// can issue the loads before work the stores depend on.
//
// Every lane of the wave calls these, also lanes whose piece lies past the
// end of the row: their loads read zeros and their payload stores are
// dropped by the per-row buffer resources, and the one plain store (the
// scale) is guarded per lane.  So the v_readlane of the row indices never
// runs under a partial exec mask.
struct Fp8Piece {
    i32x4 a, b;
};

__device__ __forceinline__ Fp8Piece fp8_load(const uint16_t* __restrict__ xrow, int chunk, int H) {
    const auto xr = buffer_rsrc(xrow, (uint32_t)H * 2u);
    Fp8Piece v;
    v.a = __builtin_amdgcn_raw_buffer_load_b128(xr, chunk * 32, 0, kCached);
    v.b = __builtin_amdgcn_raw_buffer_load_b128(xr, chunk * 32 + 16, 0, kCached);
    return v;
}

__device__ __forceinline__ void fp8_store(const Fp8Piece& v, int chunk, int H, int k, int my_slot, int nrows,
                                          uint8_t* __restrict__ recv, float* __restrict__ recv_sc) {
    const int lane = threadIdx.x & 63;
    const i32x4 a = v.a, b = v.b;
    float f[16];
    f[0] = bf16_lo(a.x);  f[1] = bf16_hi(a.x);  f[2] = bf16_lo(a.y);  f[3] = bf16_hi(a.y);
    f[4] = bf16_lo(a.z);  f[5] = bf16_hi(a.z);  f[6] = bf16_lo(a.w);  f[7] = bf16_hi(a.w);
    f[8] = bf16_lo(b.x);  f[9] = bf16_hi(b.x);  f[10] = bf16_lo(b.y); f[11] = bf16_hi(b.y);
    f[12] = bf16_lo(b.z); f[13] = bf16_hi(b.z); f[14] = bf16_lo(b.w); f[15] = bf16_hi(b.w);

    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 4, kWave));
    const float ac = fmaxf(amax, 1e-4f);
    const float inv = 448.0f / ac;
    const float sc = ac / 448.0f;

    i32x4 q;
    q.x = (int)pack_e4m3x4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
    q.y = (int)pack_e4m3x4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
    q.z = (int)pack_e4m3x4(f[8] * inv, f[9] * inv, f[10] * inv, f[11] * inv);
    q.w = (int)pack_e4m3x4(f[12] * inv, f[13] * inv, f[14] * inv, f[15] * inv);

    const int nblk = H >> 7;
    const bool sc_lane = (lane & 7) == 0 && chunk * 16 < H;  // first lane of a block inside the row
    for (int j = 0; j < k; ++j) {
        const int r = __builtin_amdgcn_readlane(my_slot, j);
        if ((unsigned)r < (unsigned)nrows) {
            const auto rr = buffer_rsrc(recv + (size_t)r * H, (uint32_t)H);
            __builtin_amdgcn_raw_buffer_store_b128(q, rr, chunk * 16, 0, kStream);
            if (sc_lane) recv_sc[(size_t)r * nblk + (chunk >> 3)] = sc;
        }
    }
}

__device__ __forceinline__ void fp8_piece(const uint16_t* __restrict__ xrow, int chunk, int H, int k,
                                          int my_slot, int nrows, uint8_t* __restrict__ recv,
                                          float* __restrict__ recv_sc) {
    fp8_store(fp8_load(xrow, chunk, H), chunk, H, k, my_slot, nrows, recv, recv_sc);
}

// BF16: a lane owns 8 channels (`chunk` counts 8-channel pieces): one 16-byte
// load, one 16-byte streamed store per receive row.
__device__ __forceinline__ i32x4 bf16_load(const uint16_t* __restrict__ xrow, int chunk, int H) {
    return __builtin_amdgcn_raw_buffer_load_b128(buffer_rsrc(xrow, (uint32_t)H * 2u), chunk * 16, 0, kCached);
}

__device__ __forceinline__ void bf16_store(i32x4 v, int chunk, int H, int k, int my_slot, int nrows,
                                           uint16_t* __restrict__ recv) {
    for (int j = 0; j < k; ++j) {
        const int r = __builtin_amdgcn_readlane(my_slot, j);
        if ((unsigned)r < (unsigned)nrows) {
            const auto rr = buffer_rsrc(recv + (size_t)r * H, (uint32_t)H * 2u);
            __builtin_amdgcn_raw_buffer_store_b128(v, rr, chunk * 16, 0, kStream);
        }
    }
}

__device__ __forceinline__ void bf16_piece(const uint16_t* __restrict__ xrow, int chunk, int H, int k,
                                           int my_slot, int nrows, uint16_t* __restrict__ recv) {
    bf16_store(bf16_load(xrow, chunk, H), chunk, H, k, my_slot, nrows, recv);
}

}  // namespace ep
