// dispatch.hip -- scatter of each token's hidden row to its k receive rows,
// as FP8 E4M3 with one fp32 scale per 128 channels, or as BF16.
//
// Dispatch sends each token to the experts its gate chose (DeepEP blog
// "【Day2】DeepEP ...", section "DeepEP是什么"); the DeepEP test setting uses an
// FP8 payload for dispatch (news report on the release, "具体性能方面").  The
// scaling rule is this library's reading: per token and 128-channel block,
// amax = max |x|, a = max(amax, 1e-4), inv = 448 / a, scale = a / 448,
// code = e4m3_rne(x * inv).
//
// One-wave workgroups stride over the (token, 64-lane piece of its row)
// items (in XCD-contiguous order for large batches, launch.h); a lane's piece is read once and written to the token's k receive
// rows (rows.h: 16 channels per lane for FP8, 8 for BF16).  Receive-row
// indices are loaded once per wavefront and broadcast with v_readlane.
//
// Cache policy, measured on MI355X at 4096 tokens x 7168 channels, top-8:
// streaming (nt) stores of the receive rows (cached stores: 65 us), and
// default-cached loads of x.  With x still in the 256 MB Infinity Cache
// (written or read shortly before) the cached loads take 49.5 us against
// 62 us for nt loads; with x cold in HBM both take 62-63 us.
#include "launch.h"
#include "rows.h"

namespace ep {

namespace {

__global__ __launch_bounds__(64, 8) void dispatch_fp8_kernel(const uint16_t* __restrict__ x,
                                                             const int32_t* __restrict__ slot,
                                                             uint8_t* __restrict__ recv,
                                                             float* __restrict__ recv_sc, int H, int k,
                                                             int nrows, int segs, int items, bool xcd_order) {
    const int lane = threadIdx.x;
    for (int v = blockIdx.x; v < items; v += gridDim.x) {
        const int item = xcd_order ? xcd_item(v, items) : v;
        const int t = item / segs;
        const int chunk = (item - t * segs) * 64 + lane;  // 16-channel piece of row t

        // receive rows of token t, one per lane j < k (loaded with all lanes on)
        int my_slot = -1;
        if (lane < k) my_slot = slot[(size_t)t * k + lane];

        // every lane takes part (pieces past the row end read zeros and
        // store nothing), so the row-index broadcasts run on a full wave
        fp8_piece(x + (size_t)t * H, chunk, H, k, my_slot, nrows, recv, recv_sc);
    }
}

__global__ __launch_bounds__(64, 8) void dispatch_bf16_kernel(const uint16_t* __restrict__ x,
                                                              const int32_t* __restrict__ slot,
                                                              uint16_t* __restrict__ recv, int H, int k,
                                                              int nrows, int segs, int items, bool xcd_order) {
    const int lane = threadIdx.x;
    for (int v = blockIdx.x; v < items; v += gridDim.x) {
        const int item = xcd_order ? xcd_item(v, items) : v;
        const int t = item / segs;
        const int chunk = (item - t * segs) * 64 + lane;  // 8-channel piece of row t

        int my_slot = -1;
        if (lane < k) my_slot = slot[(size_t)t * k + lane];

        bf16_piece(x + (size_t)t * H, chunk, H, k, my_slot, nrows, recv);
    }
}

}  // namespace

hipError_t launch_dispatch_fp8(const Shape& s, const uint16_t* x, const int32_t* slot, uint8_t* recv,
                               float* recv_scales, hipStream_t stream) {
    if (s.T == 0) return hipSuccess;
    const RowGrid g = row_grid(s.T, s.H >> 4);
    hipLaunchKernelGGL(dispatch_fp8_kernel, dim3(g.blocks), dim3(64), 0, stream, x, slot, recv, recv_scales,
                       s.H, s.k, s.T * s.k, g.segs, g.items, s.T >= kXcdOrderMinTokens);
    return hipGetLastError();
}

hipError_t launch_dispatch_bf16(const Shape& s, const uint16_t* x, const int32_t* slot, uint16_t* recv,
                                hipStream_t stream) {
    if (s.T == 0) return hipSuccess;
    const RowGrid g = row_grid(s.T, s.H >> 3);
    hipLaunchKernelGGL(dispatch_bf16_kernel, dim3(g.blocks), dim3(64), 0, stream, x, slot, recv, s.H, s.k,
                       s.T * s.k, g.segs, g.items, s.T >= kXcdOrderMinTokens);
    return hipGetLastError();
}

}  // namespace ep
