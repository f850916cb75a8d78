// gate.hip -- group-limited top-k gating, one 64-lane wavefront per token.
//
// Group-limited gating is named by the DeepEP pages (news report on the
// release, feature list; German summary page "DeepEP"); the pages give no
// formula.  These kernels compute: sigmoid scores; group score = sum of the
// group's m best scores, largest first; the TG best groups (score desc,
// index asc); the k best experts in those groups (score desc, index asc);
// weights s_j / ((s_0 + s_1) + ... ).
//
// Lane l holds experts l, l + 64, l + 128, ... (EPL of them), so every
// logits load instruction of a wave reads 256 contiguous bytes.
//
// Two kernels compute the same result:
//  - gate_fast_kernel, when the group size GS = E/G divides 64 and m <= 2,
//    or when every group is kept (TG = G): a group is then an aligned run of
//    GS lanes inside one register, and its top-m is a butterfly merge of
//    sorted pairs across those lanes (DPP lane swaps).  The k picks are k
//    rounds of a 32-bit DPP wave maximum of the lanes' best candidate keys,
//    with a ballot to find the owning lane (the lowest expert index among
//    exact ties).  No LDS, no barriers.
//  - gate_kernel, any shape: scores staged in LDS, lane g ranks group g's
//    scores serially, k rounds of a 64-bit wave arg-max.
#include "device.h"
#include "launch.h"

namespace ep {

namespace {

constexpr int kGateWaves = 4;  // tokens per workgroup
constexpr int kMaxTopm = 8;

// Keys of candidate experts: score bits with the top bit set (scores are
// non-negative, so key order is score order and every candidate outranks the
// key 0 of non-candidates and of experts already picked).
constexpr uint32_t kCandidate = 0x80000000u;

// One butterfly step of a group's sorted best-MC list (a0 >= a1) over
// aligned runs of 2D lanes, when the runs of the group are longer than D.
template <int D, int MC>
__device__ __forceinline__ void merge_step(uint32_t& a0, uint32_t& a1, int gs_log2) {
    if ((1 << gs_log2) <= D) return;
    const uint32_t b0 = partner_u32<D>(a0);
    if (MC == 2) {
        const uint32_t b1 = partner_u32<D>(a1);
        const uint32_t lo = min(a0, b0);
        a0 = max(a0, b0);
        a1 = max(lo, max(a1, b1));
    } else {
        a0 = max(a0, b0);
    }
}

// MC: 0 = every group kept (no group step); 1 or 2 = capacity of the sorted
// list of a group's best scores (m <= MC).
template <int EPL, int MC>
__global__ __launch_bounds__(kGateWaves * kWave) void gate_fast_kernel(
    const float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int T, int E,
    int G, int TG, int k, int m, int gs_log2) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kGateWaves + wave;
    if (t >= T) return;  // the whole wave leaves; nothing below synchronises

    // 1. scores (lanes past E read expert 0 and are masked afterwards)
    uint32_t sb[EPL];
    const float* row = logits + (size_t)t * E;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = i * kWave + lane;
        const float sg = sigmoid(row[e < E ? e : 0]);
        sb[i] = e < E ? __float_as_uint(sg) : 0u;
    }

    // 2. kept groups (bit g of `kept`; groups hold GS = 2^gs_log2 <= 64 experts)
    uint64_t kept = ~0ull;
    if (MC > 0) {
        // group score of the group of expert i*64 + lane, in every lane of
        // that group's run: merge the sorted best-MC lists of the two halves
        // of ever larger aligned runs
        uint32_t gsc[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            uint32_t a0 = sb[i], a1 = 0u;
            merge_step<1, MC>(a0, a1, gs_log2);
            merge_step<2, MC>(a0, a1, gs_log2);
            merge_step<4, MC>(a0, a1, gs_log2);
            merge_step<8, MC>(a0, a1, gs_log2);
            merge_step<16, MC>(a0, a1, gs_log2);
            merge_step<32, MC>(a0, a1, gs_log2);
            float g = __uint_as_float(a0);
            if (MC == 2 && m == 2) g = g + __uint_as_float(a1);
            gsc[i] = __float_as_uint(g);
        }
        // lane g < G ranks group g: the number of groups that outrank it
        const int gi = (lane << gs_log2) >> 6;    // register holding group `lane`
        const int gsrc = (lane << gs_log2) & 63;  // first lane of its run
        uint32_t mine = 0u;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const uint32_t v = (uint32_t)__shfl((int)gsc[i], gsrc, kWave);
            if (i == gi) mine = v;
        }
        int rank = 0;
        for (int g = 0; g < G; ++g) {
            const int ri = (g << gs_log2) >> 6;
            uint32_t sel = 0u;
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (i == ri) sel = gsc[i];
            const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)sel, (g << gs_log2) & 63);
            rank += (o > mine || (o == mine && g < lane)) ? 1 : 0;
        }
        kept = __ballot(lane < G && rank < TG);
    }

    // 3. candidate keys
    uint32_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = i * kWave + lane;
        const bool cand = e < E && (MC == 0 || ((kept >> (e >> gs_log2)) & 1ull));
        key[i] = cand ? (sb[i] | kCandidate) : 0u;
    }

    // 4. k rounds: the best remaining key, lowest expert index among ties
    int my_e = 0;
    float my_s = 0.0f;
    float S = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint32_t bk = 0u;
        int bi = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (key[i] > bk) {
                bk = key[i];
                bi = i;
            }
        const uint32_t wm = wave_max_u32(bk);
        const uint64_t hit = __ballot(bk == wm);
        const int l0 = __ffsll((unsigned long long)hit) - 1;
        int e = __builtin_amdgcn_readlane(bi, l0) * kWave + l0;
        for (uint64_t rest = hit & (hit - 1); rest; rest &= rest - 1) {  // exact ties across lanes
            const int l = __ffsll((unsigned long long)rest) - 1;
            e = min(e, __builtin_amdgcn_readlane(bi, l) * kWave + l);
        }
        const float sv = __uint_as_float(wm & ~kCandidate);
        const bool owner = lane == (e & 63);
#pragma unroll
        for (int i = 0; i < EPL; ++i) key[i] = (owner && i == (e >> 6)) ? 0u : key[i];
        my_e = lane == j ? e : my_e;
        my_s = lane == j ? sv : my_s;
        S = S + sv;
    }

    // 5. weights
    if (lane < k) {
        topk_idx[(size_t)t * k + lane] = my_e;
        topk_w[(size_t)t * k + lane] = my_s / S;
    }
}

template <int EPL>
__global__ __launch_bounds__(kGateWaves * kWave) void gate_kernel(
    const float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int T, int E, int G, int TG, int k, int m) {
    __shared__ float s_lds[kGateWaves][EPL * kWave];
    __shared__ float g_lds[kGateWaves][64];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kGateWaves + wave;
    const bool active = t < T;
    const int GS = E / G;

    // 1. scores
    float s[EPL];
    const float* row = logits + (size_t)t * E;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = i * kWave + lane;
        s[i] = 0.0f;
        if (active && e < E) {
            s[i] = sigmoid(row[e]);
            s_lds[wave][e] = s[i];
        }
    }
    __syncthreads();

    // 2. group scores: lane g keeps its group's m largest scores (bit order)
    //    by compare-exchange insertion, then adds them largest first
    if (active && lane < G) {
        uint32_t top[kMaxTopm];
#pragma unroll
        for (int j = 0; j < kMaxTopm; ++j) top[j] = 0u;
        const float* gs = &s_lds[wave][lane * GS];
        for (int i = 0; i < GS; ++i) {
            uint32_t v = __float_as_uint(gs[i]);
#pragma unroll
            for (int j = 0; j < kMaxTopm; ++j) {
                if (j < m) {
                    const uint32_t hi = top[j] > v ? top[j] : v;
                    const uint32_t lo = top[j] > v ? v : top[j];
                    top[j] = hi;
                    v = lo;
                }
            }
        }
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < kMaxTopm; ++j)
            if (j < m) acc = acc + __uint_as_float(top[j]);
        g_lds[wave][lane] = acc;
    }
    __syncthreads();
    if (!active) return;  // no barriers below

    // 3. keep the TG best groups: a group's rank is the number of groups
    //    that outrank it
    bool kept = false;
    if (lane < G) {
        const uint32_t mine = __float_as_uint(g_lds[wave][lane]);
        int rank = 0;
        for (int g = 0; g < G; ++g) {
            const uint32_t o = __float_as_uint(g_lds[wave][g]);
            rank += (o > mine || (o == mine && g < lane)) ? 1 : 0;
        }
        kept = rank < TG;
    }
    const uint64_t kept_mask = __ballot(kept);

    // 4. candidate keys: score bits above, inverted index below, so the
    //    largest key is the best expert; non-candidates get 0
    uint64_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = i * kWave + lane;
        key[i] = 0;
        if (e < E && ((kept_mask >> (e / GS)) & 1ull))
            key[i] = ((uint64_t)__float_as_uint(s[i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
    }

    // 5. k rounds of wave-wide arg-max
    int my_e = 0;
    float my_s = 0.0f;
    float S = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
        const float sv = __uint_as_float((uint32_t)(best >> 32));
        if (lane == (e & 63)) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (i == (e >> 6)) key[i] = 0;
        }
        if (lane == j) {
            my_e = e;
            my_s = sv;
        }
        S = S + sv;
    }

    // 6. weights
    if (lane < k) {
        topk_idx[(size_t)t * k + lane] = my_e;
        topk_w[(size_t)t * k + lane] = my_s / S;
    }
}

template <int EPL>
hipError_t launch_gate(const Shape& s, const float* logits, int32_t* idx, float* w, hipStream_t st) {
    const int blocks = (s.T + kGateWaves - 1) / kGateWaves;
    hipLaunchKernelGGL(gate_kernel<EPL>, dim3(blocks), dim3(kGateWaves * kWave), 0, st, logits, idx, w,
                       s.T, s.E, s.G, s.TG, s.k, s.m);
    return hipGetLastError();
}

template <int EPL, int MC>
hipError_t launch_fast(const Shape& s, int gs_log2, const float* logits, int32_t* idx, float* w,
                       hipStream_t st) {
    const int blocks = (s.T + kGateWaves - 1) / kGateWaves;
    hipLaunchKernelGGL((gate_fast_kernel<EPL, MC>), dim3(blocks), dim3(kGateWaves * kWave), 0, st, logits, idx,
                       w, s.T, s.E, s.G, s.TG, s.k, s.m, gs_log2);
    return hipGetLastError();
}

template <int EPL>
hipError_t launch_fast_mc(const Shape& s, int mc, int gs_log2, const float* logits, int32_t* idx, float* w,
                          hipStream_t st) {
    if (mc == 0) return launch_fast<EPL, 0>(s, gs_log2, logits, idx, w, st);
    if (mc == 1) return launch_fast<EPL, 1>(s, gs_log2, logits, idx, w, st);
    return launch_fast<EPL, 2>(s, gs_log2, logits, idx, w, st);
}

// Elementwise gate scores, V consecutive values per lane per step (V = 4
// when both pointers are 16-byte aligned), grid-stride over the T*E values.
// No __restrict__: scores may alias logits.
template <int V>
__global__ __launch_bounds__(256) void scores_kernel(const float* logits, float* scores, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i * V < n; i += stride) {
        if (V == 4 && i * 4 + 4 <= n) {
            float4 v = reinterpret_cast<const float4*>(logits)[i];
            v.x = sigmoid(v.x);
            v.y = sigmoid(v.y);
            v.z = sigmoid(v.z);
            v.w = sigmoid(v.w);
            reinterpret_cast<float4*>(scores)[i] = v;
        } else {
#pragma unroll
            for (int u = 0; u < V; ++u) {
                const size_t j = i * V + u;
                if (j < n) scores[j] = sigmoid(logits[j]);
            }
        }
    }
}

}  // namespace

hipError_t launch_route(const Shape& s, const float* logits, int32_t* topk_idx, float* topk_w,
                        hipStream_t stream) {
    if (s.T == 0) return hipSuccess;
    const int epl = (s.E + kWave - 1) / kWave;
    const int GS = s.E / s.G;
    int gs_log2 = 0;
    while ((1 << gs_log2) < GS) ++gs_log2;
    const bool pow2 = (1 << gs_log2) == GS;
    if (s.TG == s.G || (pow2 && GS <= kWave && s.m <= 2)) {
        // with every group kept (mc = 0) the group size plays no part
        const int mc = s.TG == s.G ? 0 : s.m;
        if (epl <= 1) return launch_fast_mc<1>(s, mc, gs_log2, logits, topk_idx, topk_w, stream);
        if (epl <= 2) return launch_fast_mc<2>(s, mc, gs_log2, logits, topk_idx, topk_w, stream);
        if (epl <= 4) return launch_fast_mc<4>(s, mc, gs_log2, logits, topk_idx, topk_w, stream);
        if (epl <= 8) return launch_fast_mc<8>(s, mc, gs_log2, logits, topk_idx, topk_w, stream);
        return launch_fast_mc<16>(s, mc, gs_log2, logits, topk_idx, topk_w, stream);
    }
    if (epl <= 1) return launch_gate<1>(s, logits, topk_idx, topk_w, stream);
    if (epl <= 2) return launch_gate<2>(s, logits, topk_idx, topk_w, stream);
    if (epl <= 4) return launch_gate<4>(s, logits, topk_idx, topk_w, stream);
    if (epl <= 8) return launch_gate<8>(s, logits, topk_idx, topk_w, stream);
    return launch_gate<16>(s, logits, topk_idx, topk_w, stream);
}

hipError_t launch_scores(const Shape& s, const float* logits, float* scores, hipStream_t stream) {
    const size_t n = (size_t)s.T * (size_t)s.E;
    if (n == 0) return hipSuccess;
    const bool vec = ((reinterpret_cast<uintptr_t>(logits) | reinterpret_cast<uintptr_t>(scores)) & 15) == 0;
    const int V = vec ? 4 : 1;
    const size_t lanes = (n + V - 1) / V;
    const size_t want = (lanes + 255) / 256;
    const unsigned blocks = (unsigned)(want < (1u << 16) ? want : (1u << 16));
    if (vec)
        hipLaunchKernelGGL(scores_kernel<4>, dim3(blocks), dim3(256), 0, stream, logits, scores, n);
    else
        hipLaunchKernelGGL(scores_kernel<1>, dim3(blocks), dim3(256), 0, stream, logits, scores, n);
    return hipGetLastError();
}

}  // namespace ep
