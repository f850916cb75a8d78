// ll.hip -- low-latency dispatch: each token goes straight into
// fixed-capacity receive rows of its experts, with no separate layout pass
// and nothing for the host to wait for.
//
// The DeepEP pages describe a second kernel family for latency-sensitive
// inference decoding (news report on the release, feature list; blog
// "【Day2】DeepEP ...", "DeepEP的关键技术" item 4 and "DeepEP 的性能表现",
// low-latency kernels at 128 tokens per batch, FP8 dispatch, BF16 combine).
// The reading implemented here: expert e owns receive rows
// [e * cap, (e + 1) * cap); pair (t, j) routed to e takes row e * cap + pos,
// where pos counts the routed pairs before it (row-major (t, j) order) with
// the same expert -- the same in-expert order as the normal layout -- and
// is dropped (slot -1) when pos >= cap.
//
// One workgroup per token: it counts the earlier routed pairs per expert in
// an LDS histogram, then stores the token's row pieces as the normal
// dispatch does (rows.h).  One extra
// workgroup writes the per-expert counts.  The work to find positions grows
// with T * k, so the path is limited to small batches (decode).
#include "launch.h"
#include "rows.h"

namespace ep {

namespace {

constexpr int kMaxBlockThreads = 1024;
// row pieces per thread: H/16 <= 1024 FP8 pieces, H/8 <= 2048 BF16 pieces
constexpr int kLLPieces = 2;

template <bool FP8>
__global__ __launch_bounds__(kMaxBlockThreads) void dispatch_ll_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ idx, void* __restrict__ recv,
    float* __restrict__ recv_sc, int32_t* __restrict__ recv_count, int32_t* __restrict__ recv_src,
    int32_t* __restrict__ slot_out, int T, int H, int E, int k, int cap) {
    __shared__ int s_cnt[kMaxExpertsLL];  // per-expert counts: of all pairs (last block) or of earlier pairs
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    if (blockIdx.x == (unsigned)T) {  // per-expert counts of routed pairs
        const int P = T * k;
        for (int i = tid; i < E; i += blockDim.x) s_cnt[i] = 0;
        __syncthreads();
        for (int p = tid; p < P; p += blockDim.x) {
            const int e = idx[p];
            if ((unsigned)e < (unsigned)E) atomicAdd(&s_cnt[e], 1);
        }
        __syncthreads();
        for (int i = tid; i < E; i += blockDim.x) recv_count[i] = s_cnt[i];
        return;
    }

    const int t = blockIdx.x;
    // position of pick j = routed pairs of earlier tokens with the same
    // expert (the entries [0, t*k) of idx), counted as a histogram over
    // experts in LDS.  The first pass's entries (four per thread) and the
    // token's own picks are loaded before the row pieces: loads complete in
    // issue order, so waiting for these small cache-resident reads does not
    // wait for the row pieces from HBM.  The loads are unconditional buffer
    // loads (out of range ones return 0 and are masked afterwards) so the
    // compiler can count what is still in flight.
    const int before = t * k;
    const int nt = blockDim.x;
    const auto er = buffer_rsrc(idx, (uint32_t)before * 4u);
    int v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = (int)__builtin_amdgcn_raw_buffer_load_b32(er, (tid + u * nt) * 4, 0, kCached);
    // lane j < k: expert of pick j, -1 if unrouted
    int my_e = (int)__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(idx + (size_t)before, (uint32_t)k * 4u),
                                                          lane * 4, 0, kCached);

    const uint16_t* xrow = x + (size_t)t * H;
    // the token's row pieces do not depend on the positions: load them now
    // so their latency overlaps the count (a thread owns at most kLLPieces
    // pieces: blockDim covers H/16 FP8 pieces, or half the H/8 BF16 pieces at
    // H = 16384)
    Fp8Piece pf[kLLPieces];
    i32x4 pb[kLLPieces];
#pragma unroll
    for (int u = 0; u < kLLPieces; ++u) {
        const int chunk = tid + u * nt;  // past the row: reads 0, never stored
        if (FP8) pf[u] = fp8_load(xrow, chunk, H);
        else pb[u] = bf16_load(xrow, chunk, H);
    }
    for (int i = tid; i < E; i += nt) s_cnt[i] = 0;
    my_e = (lane < k && (unsigned)my_e < (unsigned)E) ? my_e : -1;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u)
        if (tid + u * nt < before && (unsigned)v[u] < (unsigned)E) atomicAdd(&s_cnt[v[u]], 1);
    for (int p = tid + 4 * nt; p < before; p += nt) {
        const int e = idx[p];
        if ((unsigned)e < (unsigned)E) atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();
    int my_pos = my_e >= 0 ? s_cnt[my_e] : 0;
    // earlier picks of this token with the same expert (a repeated expert)
    for (int j = 0; j + 1 < k; ++j) {
        const int ej = __builtin_amdgcn_readlane(my_e, j);
        my_pos += (lane > j && lane < k && my_e >= 0 && my_e == ej) ? 1 : 0;
    }
    const int my_slot = (my_e >= 0 && my_pos < cap) ? my_e * cap + my_pos : -1;
    if (wave == 0 && lane < k) {
        slot_out[(size_t)t * k + lane] = my_slot;
        if (my_slot >= 0) recv_src[my_slot] = t;
    }

    const int nrows = E * cap;
    const int npieces = FP8 ? (H >> 4) : (H >> 3);
    // a pass runs when any of its pieces lies in the row (a condition uniform
    // over the workgroup); in it every lane stores (pieces past the row end
    // were read as zeros and are dropped by the row's buffer resource; the
    // scale store is guarded per lane), so the row-index broadcasts never
    // run under a partial exec mask
#pragma unroll
    for (int u = 0; u < kLLPieces; ++u) {
        if (u * nt >= npieces) break;
        const int chunk = tid + u * nt;
        if (FP8) fp8_store(pf[u], chunk, H, k, my_slot, nrows, static_cast<uint8_t*>(recv), recv_sc);
        else bf16_store(pb[u], chunk, H, k, my_slot, nrows, static_cast<uint16_t*>(recv));
    }
}

}  // namespace

hipError_t launch_dispatch_ll(const Shape& s, int cap, bool fp8, const uint16_t* x, const int32_t* topk_idx,
                              void* recv, float* recv_scales, int32_t* recv_count, int32_t* recv_src,
                              int32_t* slot, hipStream_t stream) {
    const int lanes = fp8 ? (s.H >> 4) : (s.H >> 3);
    int threads = (lanes + 63) / 64 * 64;
    if (threads > kMaxBlockThreads) threads = kMaxBlockThreads;
    if (fp8)
        hipLaunchKernelGGL(dispatch_ll_kernel<true>, dim3(s.T + 1), dim3(threads), 0, stream, x, topk_idx, recv,
                           recv_scales, recv_count, recv_src, slot, s.T, s.H, s.E, s.k, cap);
    else
        hipLaunchKernelGGL(dispatch_ll_kernel<false>, dim3(s.T + 1), dim3(threads), 0, stream, x, topk_idx, recv,
                           recv_scales, recv_count, recv_src, slot, s.T, s.H, s.E, s.k, cap);
    return hipGetLastError();
}

}  // namespace ep
