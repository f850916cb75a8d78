// combine.hip -- gather of each token's k expert outputs and their
// gate-weighted sum in fp32, rounded once to bf16.
//
// Combine brings the experts' outputs back to their token and accumulates
// them (DeepEP blog "【Day2】DeepEP ...", sections "DeepEP是什么" and
// "All-to-All通信"), in BF16 (news report on the release, "具体性能方面").
// Reading: acc = +0; acc = fma(w_j, y_j, acc) for j = 0..k-1 in pick order;
// out = bf16_rne(acc).
//
// A lane owns 8 channels: it issues up to 8 of its 16-byte row loads before
// the first multiply-add, so that 128 bytes per lane are in flight, then
// stores one 16-byte bf16 result.  Row indices and weights are loaded once
// per wavefront and broadcast with v_readlane, so row addresses are
// wave-uniform (one buffer resource per row, in scalar registers).  Loads
// and the store are streaming (nt): nothing is read twice.  Measured on
// MI355X at 4096 tokens x 7168 channels, top-8: 91 us with nt loads, 99 us
// with cached loads.
#include "device.h"
#include "launch.h"

namespace ep {

namespace {

// k rows are gathered in batches of B: all B loads of a batch are issued
// before its multiply-adds, which keep the pick order j = 0, 1, ...
template <int B, bool UNIT = false>
__global__ __launch_bounds__(64, 8) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ slot,
                                                      const float* __restrict__ w,
                                                      uint16_t* __restrict__ out, int H, int k, int nrows,
                                                      int segs, int items) {
    const int lane = threadIdx.x;
    const uint32_t row_bytes = (uint32_t)H * 2u;
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int t = item / segs;
        const int chunk = (item - t * segs) * 64 + lane;  // 8-channel piece of row t

        int my_slot = -1;
        float my_w = 1.0f;  // UNIT: every weight is 1, so fma(1, y, acc) = acc + y
        if (lane < k) {
            my_slot = slot[(size_t)t * k + lane];
            if (!UNIT) my_w = w[(size_t)t * k + lane];
        }

        // every lane takes part, also past the row end (its loads read zeros
        // and its store is dropped by the row's buffer resource), so the
        // v_readlane broadcasts below never run under a partial exec mask
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += B) {
            i32x4 v[B];
#pragma unroll
            for (int j = 0; j < B; ++j) {
                v[j] = i32x4{0, 0, 0, 0};
                if (j0 + j < k) {
                    const int r = __builtin_amdgcn_readlane(my_slot, j0 + j);
                    if ((unsigned)r < (unsigned)nrows) {
                        const auto yr = buffer_rsrc(y + (size_t)r * H, row_bytes);
                        v[j] = __builtin_amdgcn_raw_buffer_load_b128(yr, chunk * 16, 0, kStream);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < B; ++j) {
                if (j0 + j < k) {
                    const int r = __builtin_amdgcn_readlane(my_slot, j0 + j);
                    if ((unsigned)r < (unsigned)nrows) {
                        const float wj =
                            __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_w), j0 + j));
                        acc[0] = __builtin_fmaf(wj, bf16_lo(v[j].x), acc[0]);
                        acc[1] = __builtin_fmaf(wj, bf16_hi(v[j].x), acc[1]);
                        acc[2] = __builtin_fmaf(wj, bf16_lo(v[j].y), acc[2]);
                        acc[3] = __builtin_fmaf(wj, bf16_hi(v[j].y), acc[3]);
                        acc[4] = __builtin_fmaf(wj, bf16_lo(v[j].z), acc[4]);
                        acc[5] = __builtin_fmaf(wj, bf16_hi(v[j].z), acc[5]);
                        acc[6] = __builtin_fmaf(wj, bf16_lo(v[j].w), acc[6]);
                        acc[7] = __builtin_fmaf(wj, bf16_hi(v[j].w), acc[7]);
                    }
                }
            }
        }
        i32x4 o;
        o.x = (int)pack_bf16x2(acc[0], acc[1]);
        o.y = (int)pack_bf16x2(acc[2], acc[3]);
        o.z = (int)pack_bf16x2(acc[4], acc[5]);
        o.w = (int)pack_bf16x2(acc[6], acc[7]);
        const auto orr = buffer_rsrc(out + (size_t)t * H, row_bytes);
        __builtin_amdgcn_raw_buffer_store_b128(o, orr, chunk * 16, 0, kStream);
    }
}

template <int B>
hipError_t launch(const Shape& s, int nrows, const uint16_t* y, const int32_t* slot, const float* w,
                  uint16_t* out, hipStream_t st) {
    const RowGrid g = row_grid(s.T, s.H >> 3);
    hipLaunchKernelGGL(combine_kernel<B>, dim3(g.blocks), dim3(64), 0, st, y, slot, w, out, s.H, s.k, nrows,
                       g.segs, g.items);
    return hipGetLastError();
}

// In-rank partial combine.  A wave holds one 64-lane piece of token t's
// output: it loads the rows of all k picks first (KB >= k rows in
// registers), then, for each pick j that is the token's first pick on its
// rank, sums the picks on that rank in pick order (fp32 fma chain) and
// stores the bf16 partial row rank_slot[t, j].  Lane j < k holds the mask of
// the picks on pick j's rank (built with every lane active), so the sums
// test uniform bits.
template <int KB>
__global__ __launch_bounds__(64, (KB <= 8 ? 8 : (KB <= 16 ? 4 : 2))) void combine_rank_partial_kernel(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ idx, const int32_t* __restrict__ slot,
    const float* __restrict__ w, const int32_t* __restrict__ rank_slot, uint16_t* __restrict__ partial, int H, int k,
    int E, int EPR, int nrows, int segs, int items) {
    const int lane = threadIdx.x;
    const uint32_t row_bytes = (uint32_t)H * 2u;
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int t = item / segs;
        const int chunk = (item - t * segs) * 64 + lane;

        int my_slot = -1, my_rank = -1, my_rs = -1;
        float my_w = 0.0f;
        if (lane < k) {
            const size_t p = (size_t)t * k + lane;
            my_slot = slot[p];
            my_w = w[p];
            const int e = idx[p];
            my_rank = (unsigned)e < (unsigned)E ? e / EPR : -1;
            my_rs = rank_slot[p];
        }
        uint32_t my_mask = 0u;  // picks on the same rank as pick `lane`, with a valid row
        for (int j = 0; j < k; ++j) {
            const int rj = __builtin_amdgcn_readlane(my_rank, j);
            const int sj = __builtin_amdgcn_readlane(my_slot, j);
            if (rj >= 0 && rj == my_rank && (unsigned)sj < (unsigned)nrows) my_mask |= 1u << j;
        }

        // every lane takes part (see combine_kernel)
        i32x4 v[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            v[j] = i32x4{0, 0, 0, 0};
            if (j < k) {
                const int r = __builtin_amdgcn_readlane(my_slot, j);
                if ((unsigned)r < (unsigned)nrows) {
                    const auto yr = buffer_rsrc(y + (size_t)r * H, row_bytes);
                    v[j] = __builtin_amdgcn_raw_buffer_load_b128(yr, chunk * 16, 0, kStream);
                }
            }
        }
        for (int jr = 0; jr < k; ++jr) {
            const int prow = __builtin_amdgcn_readlane(my_rs, jr);
            if ((unsigned)prow >= (unsigned)nrows) continue;  // not a first pick on its rank
            const uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)my_mask, jr);
            // keep the rows packed across the jr loop: unpacking all KB rows
            // to fp32 once (hoisted out of the loop) would need 8*KB registers
#pragma unroll
            for (int j = 0; j < KB; ++j) asm volatile("" : "+v"(v[j]));
            float acc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                if ((m >> j) & 1u) {
                    const float wj = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_w), j));
                    acc[0] = __builtin_fmaf(wj, bf16_lo(v[j].x), acc[0]);
                    acc[1] = __builtin_fmaf(wj, bf16_hi(v[j].x), acc[1]);
                    acc[2] = __builtin_fmaf(wj, bf16_lo(v[j].y), acc[2]);
                    acc[3] = __builtin_fmaf(wj, bf16_hi(v[j].y), acc[3]);
                    acc[4] = __builtin_fmaf(wj, bf16_lo(v[j].z), acc[4]);
                    acc[5] = __builtin_fmaf(wj, bf16_hi(v[j].z), acc[5]);
                    acc[6] = __builtin_fmaf(wj, bf16_lo(v[j].w), acc[6]);
                    acc[7] = __builtin_fmaf(wj, bf16_hi(v[j].w), acc[7]);
                }
            }
            i32x4 o;
            o.x = (int)pack_bf16x2(acc[0], acc[1]);
            o.y = (int)pack_bf16x2(acc[2], acc[3]);
            o.z = (int)pack_bf16x2(acc[4], acc[5]);
            o.w = (int)pack_bf16x2(acc[6], acc[7]);
            const auto pr = buffer_rsrc(partial + (size_t)prow * H, row_bytes);
            __builtin_amdgcn_raw_buffer_store_b128(o, pr, chunk * 16, 0, kStream);
        }
    }
}

template <int KB>
hipError_t launch_partial(const Shape& s, const uint16_t* y, const int32_t* idx, const int32_t* slot, const float* w,
                          const int32_t* rank_slot, uint16_t* partial, hipStream_t st) {
    const RowGrid g = row_grid(s.T, s.H >> 3);
    hipLaunchKernelGGL(combine_rank_partial_kernel<KB>, dim3(g.blocks), dim3(64), 0, st, y, idx, slot, w, rank_slot,
                       partial, s.H, s.k, s.E, s.E / s.R, s.T * s.k, g.segs, g.items);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine_rank_partial(const Shape& s, const uint16_t* y, const int32_t* topk_idx,
                                       const int32_t* slot, const float* w, const int32_t* rank_slot,
                                       uint16_t* partial, hipStream_t stream) {
    if (s.T == 0) return hipSuccess;
    if (s.k <= 8) return launch_partial<8>(s, y, topk_idx, slot, w, rank_slot, partial, stream);
    if (s.k <= 16) return launch_partial<16>(s, y, topk_idx, slot, w, rank_slot, partial, stream);
    return launch_partial<32>(s, y, topk_idx, slot, w, rank_slot, partial, stream);
}

hipError_t launch_combine_ranks(const Shape& s, const uint16_t* partial, const int32_t* rank_slot, uint16_t* out,
                                hipStream_t stream) {
    if (s.T == 0) return hipSuccess;
    const RowGrid g = row_grid(s.T, s.H >> 3);
    if (s.k <= 4)
        hipLaunchKernelGGL((combine_kernel<4, true>), dim3(g.blocks), dim3(64), 0, stream, partial, rank_slot, nullptr,
                           out, s.H, s.k, s.T * s.k, g.segs, g.items);
    else
        hipLaunchKernelGGL((combine_kernel<8, true>), dim3(g.blocks), dim3(64), 0, stream, partial, rank_slot, nullptr,
                           out, s.H, s.k, s.T * s.k, g.segs, g.items);
    return hipGetLastError();
}

hipError_t launch_combine(const Shape& s, int nrows, const uint16_t* y, const int32_t* slot, const float* w,
                          uint16_t* out, hipStream_t stream) {
    if (s.T == 0) return hipSuccess;
    if (s.k <= 4) return launch<4>(s, nrows, y, slot, w, out, stream);
    return launch<8>(s, nrows, y, slot, w, out, stream);
}

}  // namespace ep
