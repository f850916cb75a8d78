// gate.hip -- group-limited top-k gating, one 64-lane wavefront per token.
//
// Group-limited gating is named by the DeepEP pages (news report on the
// release, feature list; German summary page "DeepEP"); the pages give no
// formula.  This kernel computes: sigmoid scores; group score = sum of the
// group's m best scores, largest first; the TG best groups (score desc,
// index asc); the k best experts in those groups (score desc, index asc);
// weights s_j / ((s_0 + s_1) + ... ).
//
// Lane l holds experts l, l + 64, l + 128, ... (EPL of them), so every
// logits load instruction of a wave reads 256 contiguous bytes.
#include "device.h"
#include "launch.h"

namespace ep {

namespace {

constexpr int kGateWaves = 4;  // tokens per workgroup
constexpr int kMaxTopm = 8;

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

}  // namespace

hipError_t launch_route(const Shape& s, const float* logits, int32_t* topk_idx, float* topk_w,
                        hipStream_t stream) {
    if (s.T == 0) return hipSuccess;
    const int epl = (s.E + kWave - 1) / kWave;
    if (epl <= 1) return launch_gate<1>(s, logits, topk_idx, topk_w, stream);
    if (epl <= 2) return launch_gate<2>(s, logits, topk_idx, topk_w, stream);
    if (epl <= 4) return launch_gate<4>(s, logits, topk_idx, topk_w, stream);
    if (epl <= 8) return launch_gate<8>(s, logits, topk_idx, topk_w, stream);
    return launch_gate<16>(s, logits, topk_idx, topk_w, stream);
}

}  // namespace ep
