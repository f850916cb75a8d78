// gate.hip -- group-limited top-k gating.
//
// Group-limited gating is named by the DeepEP pages (news report on the
// release, feature list; German summary page "DeepEP"); the pages give no
// formula.  These kernels compute: sigmoid scores; group score = sum of the
// group's m best scores, largest first; the TG best groups (score desc,
// index asc); the k best experts in those groups (score desc, index asc);
// weights s_j / ((s_0 + s_1) + ... ).
//
// Three kernels compute the same result:
//  - gate_pair_kernel, one or two tokens per wavefront (the token's 64 or 32
//    lanes each holding a run of 4, 8, 16 or 32 consecutive experts: E =
//    128, 256, 512 or 1024), when m <= 2 and a group is a power-of-two run
//    of whole lanes (or TG = G).  Group scores are mostly in-lane, and with two
//    tokens each cross-lane step serves both.  It can also count its picks
//    per workgroup for the routing layout (HIST).
//  - gate_fast_kernel, one wavefront per token, lane l holding experts l,
//    l + 64, ..., when the group size GS = E/G divides 64 and m <= 2, or
//    TG = G: a group is an aligned run of GS lanes inside one register, and
//    its top-m is a butterfly merge of sorted pairs across those lanes (DPP
//    lane swaps).  The k picks are k rounds of a 32-bit DPP wave maximum of
//    the lanes' best candidate keys, with a ballot to find the owning lane
//    (the lowest expert index among exact ties).  No LDS, no barriers.
//  - gate_kernel, any shape: scores staged in LDS, lane g ranks group g's
//    scores serially, k rounds of a 64-bit wave arg-max.
//
// Scores come from sigmoid_lane (device.h): the short exact form when every
// logit of the wavefront lies within +-80.
//
// Measured on MI355X, 256 experts in 8 groups, top-4 groups, top-8, back to
// back with the pick counts (HIP events): 128 tokens 5.3 us, 4096 tokens
// 5.7 us with one token per wavefront (6.5 us with two; gate_fast_kernel
// 8.9 us); 16384 tokens 14.5 us with two (18.9 us with one).  Without the
// counts, in 4-token workgroups, 128 tokens take 3.5 us.  One wave's
// dependency chain sets the time up to a few thousand tokens: the first
// load of its logits from HBM (~1.8 us), the k pick rounds (DPP steps with
// their wait states, lane reads, ballot) and, with counts, the workgroup
// barrier before they are written; at 4096 tokens four wavefronts share
// each SIMD and keep its VALU about half busy.
#include "device.h"
#include "launch.h"

namespace ep {

namespace {

constexpr int kGateWaves = 4;  // wavefronts per workgroup of the one-token-per-wavefront kernels
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
    float lg[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = i * kWave + lane;
        lg[i] = row[e < E ? e : 0];
    }
    sigmoid_lane(lg);
#pragma unroll
    for (int i = 0; i < EPL; ++i) sb[i] = i * kWave + lane < E ? __float_as_uint(lg[i]) : 0u;

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

// TPW tokens per wavefront (1 or 2), LPT = 64 / TPW lanes per token: lane l
// of the token's lanes holds the EPL = E / LPT consecutive experts
// [l*EPL, (l+1)*EPL).  Used when LPT divides E and a group is a
// power-of-two run of whole lanes (LPG = GS / EPL lanes, or every group
// kept), with m <= 2.  A group's top-m is then mostly in-lane; with two
// tokens, every cross-lane step (group merge, pick maximum, ballot) serves
// both with one instruction, which halves the per-token instruction count.
//
// Picks: each round takes the largest candidate key of each token (DPP
// maximum within its lanes, read from lane 31 and 63, or 63); the owner is
// the lowest lane holding it, and inside the owner the lowest of its
// experts with that key, which is the lowest expert index among exact ties
// since lanes hold ascending runs of experts.
constexpr uint64_t kHiHalf = 0xFFFFFFFF00000000ull;
constexpr int kPairTokens = 16;  // tokens per workgroup (one histogram column)
constexpr int kRouteTokens = 4;  // tokens per workgroup without counts, one per wavefront
constexpr int kMaxExpertsHist = 1024;
// One token per wavefront up to this many tokens, two above: one token per
// wave halves each lane's serial work (E/64 experts instead of E/32), which
// shortens every wavefront's dependency chain, while two tokens per wave
// issue fewer instructions per token, which wins once the SIMDs hold enough
// waves.
#ifndef GATE_ONE_TOKEN_MAX_T
#define GATE_ONE_TOKEN_MAX_T 4096
#endif

//
// With HIST, the workgroup (kPairTokens tokens, one "column") also counts
// its picks for the routing layout: column c = blockIdx.x gets hist[c][e]
// = picks of expert e and rank_hist[c][r] = tokens with at least one pick
// on virtual rank r (its first pick there), as bytes (at most kPairTokens
// each, since a token's picks are distinct experts).  The layout's assign
// step sums these columns instead of a separate counting launch.  With four
// experts per lane and R <= 64 each wavefront keeps its counts in registers
// (packed bytes per lane, ranks as a scalar mask) and the column sums one
// LDS row per wavefront after a single barrier; other shapes count with LDS
// atomics.
//
// KF, GF: k and G as compile-time constants for common shapes (0: the
// runtime values), so that the group ranking's lane reads and the pick
// rounds unroll.  With R <= 64 the picks' ranks are tracked in scalar
// registers during the rounds (the picks are wave-uniform per half), so
// first-on-rank needs no lane exchange afterwards; `epr_magic` =
// floor(2^32 / EPR) + 1 turns the division e / EPR into one high multiply,
// exact for e < 2^16 (EPR = 1 has magic 1 and the rank is e itself).

// Calls f(j) for j = 0 .. n-1: unrolled when N, the count known at compile
// time, is positive, else a loop over the runtime count n.
template <int N, typename F>
__device__ __forceinline__ void for_count(int n, F&& f) {
    if constexpr (N > 0) {
#pragma unroll
        for (int j = 0; j < N; ++j) f(j);
    } else {
        for (int j = 0; j < n; ++j) f(j);
    }
}

__device__ __forceinline__ uint32_t rank_of(uint32_t e, uint32_t epr_magic) {
    return __umulhi(e, epr_magic) + (epr_magic == 1u ? e : 0u);
}

template <int EPL, int MC, bool HIST, int KF, int GF, int TPW, int TPB>
__global__ __launch_bounds__(TPB / TPW * kWave) void gate_pair_kernel(
    const float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int T, int E,
    int G_rt, int TG, int k_rt, int m, int lpg_rt, uint8_t* __restrict__ hist, uint8_t* __restrict__ rank_hist,
    int R, uint32_t epr_magic) {
    static_assert(TPW == 1 || TPW == 2, "one or two tokens per wavefront");
    static_assert(!HIST || TPB == kPairTokens, "a workgroup with counts is one column");
    constexpr int LPT = kWave / TPW;  // lanes per token
    constexpr int LPT_LOG2 = TPW == 1 ? 6 : 5;
    // counts: E expert counts, then R rank counts (LDS atomics); or, with
    // four experts per lane and R <= 64, rows of per-wavefront counts
    __shared__ int cnt_lds[HIST ? 2 * kMaxExpertsHist : 1];
    static_assert(2 * (TPB / TPW) * kWave <= 2 * kMaxExpertsHist, "count rows fit the counters");
    const int k = KF > 0 ? KF : k_rt;
    const int G = GF > 0 ? GF : G_rt;
    // lanes per group: LPT / G when the groups are runs of whole lanes
    const int lpg_log2 = GF > 0 ? __builtin_ctz((unsigned)LPT / (GF > 0 ? GF : 1)) : lpg_rt;
    // the wave index is uniform across the wavefront: read it into a scalar
    // register so that the row resource below is uniform too
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int half = TPW == 2 ? lane >> 5 : 0;  // the wave's token of this lane
    const int hl = lane & (LPT - 1);             // lane within the token
    const int t0 = blockIdx.x * TPB + wave * TPW;
    if (!HIST && t0 >= T) return;  // the whole wave leaves; nothing below synchronises
    const bool track_ranks = HIST && R <= 64;
    // with four experts per lane and the ranks tracked, the counts need no
    // LDS atomics: each lane adds up the picks of its own four experts as
    // packed bytes during the pick rounds, and the column sums rows
    const bool row_counts = EPL == 4 && track_ranks;
    if (HIST && !row_counts)
        for (int i = threadIdx.x; i < E + R; i += blockDim.x) cnt_lds[i] = 0;
    const bool wlive = t0 < T;  // uniform: this wave has a token
    const int t = t0 + half;
    const bool live = t < T;  // the last wave's second half may have no token
    uint32_t cw = 0u;  // byte i: picks of the token's expert 4 * hl + i (four experts per lane)
    int my_e = 0;
    uint64_t first0 = 0, first1 = 0;  // bit j: pick j of the token is its first on that rank
    uint64_t seen0 = 0, seen1 = 0;  // ranks picked so far, per token
    if (wlive) {

    // 1. scores: EPL consecutive logits per lane, 16-byte loads through one
    //    resource over the wave's rows (every address is a multiple of 4
    //    bytes; a half with no token reads zeros and is masked below)
    uint32_t sb[EPL];
    {
        const int ntok = T - t0 < TPW ? T - t0 : TPW;
        const auto rr = buffer_rsrc(logits + (size_t)t0 * E, (uint32_t)(ntok * E) * 4u);
        const int base = (half * E + hl * EPL) * 4;
        float lg[EPL];
#pragma unroll
        for (int i = 0; i < EPL; i += 4) {
            const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rr, base + i * 4, 0, kCached);
            lg[i + 0] = __int_as_float(v.x);
            lg[i + 1] = __int_as_float(v.y);
            lg[i + 2] = __int_as_float(v.z);
            lg[i + 3] = __int_as_float(v.w);
        }
        sigmoid_lane(lg);
#pragma unroll
        for (int i = 0; i < EPL; ++i) sb[i] = __float_as_uint(lg[i]);
    }

    // 2. kept groups: the group of this lane is g = hl >> lpg_log2
    bool kept = true;
    if (MC > 0) {
        // sorted best-MC list of the lane's scores (bit order = value order
        // for these non-negative floats), then merged over the group's lanes
        uint32_t a0 = sb[0], a1 = 0u;
#pragma unroll
        for (int i = 1; i < EPL; ++i) {
            if (MC == 2) {
                const uint32_t lo = min(a0, sb[i]);
                a0 = max(a0, sb[i]);
                a1 = max(a1, lo);
            } else {
                a0 = max(a0, sb[i]);
            }
        }
        merge_step<1, MC>(a0, a1, lpg_log2);
        merge_step<2, MC>(a0, a1, lpg_log2);
        merge_step<4, MC>(a0, a1, lpg_log2);
        merge_step<8, MC>(a0, a1, lpg_log2);
        merge_step<16, MC>(a0, a1, lpg_log2);
        if (TPW == 1) merge_step<32, MC>(a0, a1, lpg_log2);
        float gf = __uint_as_float(a0);
        if (MC == 2 && m == 2) gf = gf + __uint_as_float(a1);
        const uint32_t mine = __float_as_uint(gf);
        // rank of this lane's group among the G groups of its token (with G
        // known at compile time every lane read is issued before the first
        // comparison)
        const int g = hl >> lpg_log2;
        int rank = 0;
        for_count<GF>(G, [&](int o) {
            const uint32_t v = (uint32_t)__shfl((int)mine, (half << LPT_LOG2) + (o << lpg_log2), kWave);
            rank += (v > mine || (v == mine && o < g)) ? 1 : 0;
        });
        kept = rank < TG;
    }

    uint32_t my_s = 0u;
    float S = 0.0f;
    if constexpr (EPL == 4) {
    // 3-4 with four experts per lane (256 experts at one token per
    // wavefront, 128 at two): each key carries its place in the lane, and the
    // lane's keys are sorted once, so a round reads the lane's best key
    // directly and the owner lane shifts its list.  Key = ((score bits + 1)
    // << 2) | (3 - i): score bits are at most those of 1.0f (a NaN score,
    // which the caller must not pass, is clamped there so that picks stay
    // distinct), so the shift loses nothing; candidates are >= 4,
    // non-candidates and a half with no token 0; within a lane equal scores
    // put the lower expert first.  Across lanes a larger low part must not
    // win an exact tie of scores, so a round's owner is the lowest lane of
    // the token whose best key has the round's best score (key >= that
    // score's lowest key).
    constexpr uint32_t kOneBits = 0x3F800000u;
    uint32_t q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        q[i] = (kept && live) ? (((min(sb[i], kOneBits) + 1u) << 2) | (uint32_t)(3 - i)) : 0u;
    {
        auto cx = [](uint32_t& a, uint32_t& b) {  // a >= b afterwards
            const uint32_t hi = max(a, b), lo = min(a, b);
            a = hi;
            b = lo;
        };
        cx(q[0], q[1]);
        cx(q[2], q[3]);
        cx(q[0], q[2]);
        cx(q[1], q[3]);
        cx(q[1], q[2]);
    }
    const uint32_t hsel = half ? ~0u : 0u;  // selects the upper half's value of a pair
    uint32_t pe0[KF > 0 ? KF : 1], ps0[KF > 0 ? KF : 1], pe1[KF > 0 ? KF : 1], ps1[KF > 0 ? KF : 1];
    for_count<KF>(k, [&](int j) {
        // each token's best key: row butterflies, then rows 0 -> 1 and
        // 2 -> 3 (and 1 -> 2, 3 for one token per wavefront)
        uint32_t v = q[0];
        v = max(v, dpp_u32<kDppXor1>(v));
        v = max(v, dpp_u32<kDppXor2>(v));
        v = max(v, dpp_u32<kDppHalfMirror>(v));
        v = max(v, dpp_u32<kDppMirror>(v));
        v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast15, 0xA, 0xF, false));
        // The owner of each token is the lowest lane of its ballot: a token's
        // lanes hold its maximum key, which passes the test, so neither half
        // is empty (a half without a token holds zero keys, which all pass).
        // The owner mask (x & -x per half) is formed on the scalar unit and
        // used as a lane mask, so no lane comparison waits for the index.
        uint32_t m0, m1 = 0u, hb1 = 0u;
        int o0, o1 = 32;
        uint64_t own;
        if constexpr (TPW == 2) {
            m0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
            m1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
            const uint32_t tgt = m0 ^ ((m0 ^ m1) & hsel);
            const uint64_t eq = __ballot(q[0] >= (tgt & ~3u));
            const uint64_t lo = eq & ~kHiHalf, hi = eq & kHiHalf;
            own = (lo & (0ull - lo)) | (hi & (0ull - hi));
            o0 = __builtin_ctzll(lo);
            o1 = __builtin_ctzll(hi);
            hb1 = (uint32_t)__builtin_amdgcn_readlane((int)q[0], o1);
        } else {
            v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast31, 0xC, 0xF, false));
            m0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
            const uint64_t eq = __ballot(q[0] >= (m0 & ~3u));
            own = eq & (0ull - eq);
            o0 = __builtin_ctzll(eq);
        }
        const uint32_t hb0 = (uint32_t)__builtin_amdgcn_readlane((int)q[0], o0);
        const bool owner = __builtin_amdgcn_inverse_ballot_w64(own);
        q[0] = owner ? q[1] : q[0];
        q[1] = owner ? q[2] : q[1];
        q[2] = owner ? q[3] : q[2];
        q[3] = owner ? 0u : q[3];
        // the picks (wave-uniform): expert and score bits of each token
        const uint32_t e0 = (uint32_t)o0 * 4u + (3u - (hb0 & 3u));
        const uint32_t s0 = (m0 >> 2) - 1u;
        const uint32_t e1 = (uint32_t)(o1 - 32) * 4u + (3u - (hb1 & 3u));
        const uint32_t s1 = (m1 >> 2) - 1u;
        const uint32_t sm = TPW == 2 ? (s0 ^ ((s0 ^ s1) & hsel)) : s0;
        S = S + __uint_as_float(sm);
        if constexpr (KF > 0) {
            pe0[j] = e0;
            ps0[j] = s0;
            pe1[j] = e1;
            ps1[j] = s1;
        } else {
            const bool mine = hl == j;
            const uint32_t em = TPW == 2 ? (e0 ^ ((e0 ^ e1) & hsel)) : e0;
            my_e = mine ? (int)em : my_e;
            my_s = mine ? sm : my_s;
        }
        if (HIST) {
            const uint32_t r0 = rank_of(e0, epr_magic) & 63u;
            first0 |= (uint64_t)(((seen0 >> r0) & 1ull) ^ 1ull) << j;
            seen0 |= 1ull << r0;
            // the owner lane holds the pick (expert e = 4 * hl + e % 4 of its
            // token, hl its lane within the token) and counts it in byte e % 4
            const uint32_t inc0 = 1u << ((e0 & 3u) << 3);
            uint32_t inc = inc0;
            if (TPW == 2) {
                const uint32_t r1 = rank_of(e1, epr_magic) & 63u;
                first1 |= (uint64_t)(((seen1 >> r1) & 1ull) ^ 1ull) << j;
                seen1 |= 1ull << r1;
                const uint32_t inc1 = 1u << ((e1 & 3u) << 3);
                inc = inc0 ^ ((inc0 ^ inc1) & hsel);
            }
            cw += owner ? inc : 0u;
        }
    });
    if constexpr (KF > 0) {
        // pick j to lane j of its token, after the rounds
        for_count<KF>(k, [&](int j) {
            const bool mine = hl == j;
            const uint32_t em = TPW == 2 ? (pe0[j] ^ ((pe0[j] ^ pe1[j]) & hsel)) : pe0[j];
            const uint32_t sm = TPW == 2 ? (ps0[j] ^ ((ps0[j] ^ ps1[j]) & hsel)) : ps0[j];
            my_e = mine ? (int)em : my_e;
            my_s = mine ? sm : my_s;
        });
    }
    } else {
    // 3. candidate keys (non-candidates, and a half with no token, hold 0)
    uint32_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) key[i] = (kept && live) ? (sb[i] | kCandidate) : 0u;

    // 4. k rounds
    const uint32_t hsel = half ? ~0u : 0u;  // selects the upper half's value of a pair
    for_count<KF>(k, [&](int j) {
        uint32_t bk = key[0];
#pragma unroll
        for (int i = 1; i < EPL; ++i) bk = max(bk, key[i]);
        // maximum of each token: row butterflies, then rows 0 -> 1 and
        // 2 -> 3 (and 1 -> 2, 3 for one token per wavefront)
        uint32_t v = bk;
        v = max(v, dpp_u32<kDppXor1>(v));
        v = max(v, dpp_u32<kDppXor2>(v));
        v = max(v, dpp_u32<kDppHalfMirror>(v));
        v = max(v, dpp_u32<kDppMirror>(v));
        v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast15, 0xA, 0xF, false));
        uint32_t tgt;
        uint64_t eq;
        int o0, o1 = 32;
        if constexpr (TPW == 2) {
            const uint32_t m0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
            const uint32_t m1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
            tgt = m0 ^ ((m0 ^ m1) & hsel);
            eq = __ballot(bk == tgt);
            o0 = __ffsll((unsigned long long)(eq & ~kHiHalf)) - 1;
            o1 = __ffsll((unsigned long long)(eq & kHiHalf)) - 1;
        } else {
            v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast31, 0xC, 0xF, false));
            tgt = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
            eq = __ballot(bk == tgt);
            o0 = __ffsll((unsigned long long)eq) - 1;
        }
        // the owner lanes take their first key equal to the maximum; `open`
        // and `hit` stay per-lane booleans (lane masks), so the clears are
        // selects on those masks
        bool open = lane == o0 || (TPW == 2 && lane == o1);
        uint32_t ii = 0u;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const bool hit = open && key[i] == bk;
            open = open && !hit;
            key[i] = hit ? 0u : key[i];
            ii = hit ? (uint32_t)i : ii;
        }
        const uint32_t e0 = (uint32_t)(o0 * EPL) + (uint32_t)__builtin_amdgcn_readlane((int)ii, o0);
        uint32_t e1 = 0u;
        int e = (int)e0;
        if constexpr (TPW == 2) {
            e1 = (uint32_t)((o1 - 32) * EPL) + (uint32_t)__builtin_amdgcn_readlane((int)ii, o1);
            e = (int)(e0 ^ ((e0 ^ e1) & hsel));
        }
        my_e = hl == j ? e : my_e;
        my_s = hl == j ? tgt : my_s;
        S = S + __uint_as_float(tgt & ~kCandidate);
        if (HIST) {
            // e0, e1 are wave-uniform: scalar bookkeeping (used when
            // R <= 64; the shifts are masked so other R stay defined)
            const uint32_t r0 = rank_of(e0, epr_magic) & 63u;
            first0 |= (uint64_t)(((seen0 >> r0) & 1ull) ^ 1ull) << j;
            seen0 |= 1ull << r0;
            if (TPW == 2) {
                const uint32_t r1 = rank_of(e1, epr_magic) & 63u;
                first1 |= (uint64_t)(((seen1 >> r1) & 1ull) ^ 1ull) << j;
                seen1 |= 1ull << r1;
            }
        }
    });
    }

    // 5. weights
    if (live && hl < k) {
        topk_idx[(size_t)t * k + hl] = my_e;
        topk_w[(size_t)t * k + hl] = __uint_as_float(my_s & ~kCandidate) / S;
    }
    }  // wlive

    if constexpr (HIST && EPL == 4) {
        if (row_counts) {
            // wavefront w writes row w: its lanes' packed expert counts, and
            // per rank r < R (lane r) its tokens with a pick on r; a second
            // half without a token counts nothing
            constexpr int NW = TPB / TPW;
            uint32_t rv = 0u;
            if (wlive) {
                rv = (uint32_t)((seen0 >> lane) & 1ull);
                if (TPW == 2 && t0 + 1 < T) rv += (uint32_t)((seen1 >> lane) & 1ull);
            }
            cnt_lds[wave * kWave + lane] = (int)(live ? cw : 0u);
            cnt_lds[(NW + wave) * kWave + lane] = (int)rv;
            __syncthreads();
            const size_t c = blockIdx.x;
            if (wave == 0 && lane < LPT) {
                // lane w sums word w (experts 4w .. 4w + 3) over the rows and
                // the halves: byte sums stay <= kPairTokens, so no carries
                uint32_t sum = 0u;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    sum += (uint32_t)cnt_lds[w * kWave + lane];
                    if (TPW == 2) sum += (uint32_t)cnt_lds[w * kWave + 32 + lane];
                }
                reinterpret_cast<uint32_t*>(hist + c * E)[lane] = sum;
            }
            if (wave == 1 && lane < R) {
                int sum = 0;
#pragma unroll
                for (int w = 0; w < NW; ++w) sum += cnt_lds[(NW + w) * kWave + lane];
                rank_hist[c * R + lane] = (uint8_t)sum;
            }
            return;
        }
    }
    if (HIST) {
        const bool pick = wlive && live && hl < k;
        const int r = pick ? (int)rank_of((uint32_t)my_e, epr_magic) : -1;
        bool first = pick;
        if (EPL != 4 && track_ranks) {  // (four experts per lane and R <= 64 took the rows above)
            first = pick && (((half ? first1 : first0) >> hl) & 1ull);
        } else {
            // a pick is the token's first on its rank when no earlier pick of
            // the token (lanes hl' < hl of its token) has the same rank; the
            // shuffles run with every lane active
            for (int jj = 0; jj + 1 < k; ++jj) {
                const int rj = __shfl(r, (half << LPT_LOG2) + jj, kWave);
                first = first && !(jj < hl && rj == r);
            }
        }
        __syncthreads();  // counters cleared
        if (pick) {
            atomicAdd(&cnt_lds[my_e], 1);
            if (first) atomicAdd(&cnt_lds[E + r], 1);
        }
        __syncthreads();
        // whole dwords (four byte counts each), so every line of the column
        // is written in full by this workgroup
        const size_t c = blockIdx.x;
        uint32_t* h32 = reinterpret_cast<uint32_t*>(hist + c * E);
        for (int i = threadIdx.x; i < (E >> 2); i += blockDim.x)
            h32[i] = (uint32_t)cnt_lds[4 * i] | ((uint32_t)cnt_lds[4 * i + 1] << 8) |
                     ((uint32_t)cnt_lds[4 * i + 2] << 16) | ((uint32_t)cnt_lds[4 * i + 3] << 24);
        for (int i = threadIdx.x; i < R; i += blockDim.x) rank_hist[c * R + i] = (uint8_t)cnt_lds[E + i];
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
        s[i] = active && e < E ? row[e] : 0.0f;
    }
    sigmoid_lane(s);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = i * kWave + lane;
        if (active && e < E) s_lds[wave][e] = s[i];
        else s[i] = 0.0f;
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

template <int EPL, int MC, int KF, int GF, int TPW>
hipError_t launch_pair_tpw(const Shape& s, int lpg_log2, const float* logits, int32_t* idx, float* w, uint8_t* hist,
                           uint8_t* rank_hist, hipStream_t st) {
    const int epr = s.E / s.R;
    const uint32_t magic = (uint32_t)((1ull << 32) / (uint64_t)epr + 1ull);
    if (hist) {
        constexpr int threads = kPairTokens / TPW * kWave;
        const int blocks = (s.T + kPairTokens - 1) / kPairTokens;
        hipLaunchKernelGGL((gate_pair_kernel<EPL, MC, true, KF, GF, TPW, kPairTokens>), dim3(blocks), dim3(threads),
                           0, st, logits, idx, w, s.T, s.E, s.G, s.TG, s.k, s.m, lpg_log2, hist, rank_hist, s.R,
                           magic);
    } else {
        // without counts a workgroup need not hold a whole column: smaller
        // workgroups spread small batches over more CUs, so fewer wavefronts
        // share a SIMD (128 tokens 4.5 -> 3.5 us, 1024 tokens 5.2 -> 4.0 us
        // back to back, the same at 4096)
        constexpr int tpb = TPW == 1 ? kRouteTokens : kPairTokens;
        constexpr int threads = tpb / TPW * kWave;
        const int blocks = (s.T + tpb - 1) / tpb;
        hipLaunchKernelGGL((gate_pair_kernel<EPL, MC, false, KF, GF, TPW, tpb>), dim3(blocks), dim3(threads), 0, st,
                           logits, idx, w, s.T, s.E, s.G, s.TG, s.k, s.m, lpg_log2, nullptr, nullptr, s.R, magic);
    }
    return hipGetLastError();
}

template <int EPL, int MC, int KF, int GF>
hipError_t launch_pair(const Shape& s, int tpw, int lpg_log2, const float* logits, int32_t* idx, float* w,
                       uint8_t* hist, uint8_t* rank_hist, hipStream_t st) {
    // one token per wave has E/64 <= 16 experts per lane (E <= 1024)
    if constexpr (EPL <= 16) {
        if (tpw == 1) return launch_pair_tpw<EPL, MC, KF, GF, 1>(s, lpg_log2, logits, idx, w, hist, rank_hist, st);
    }
    return launch_pair_tpw<EPL, MC, KF, GF, 2>(s, lpg_log2, logits, idx, w, hist, rank_hist, st);
}

template <int EPL>
hipError_t launch_pair_mc(const Shape& s, int tpw, int mc, int lpg_log2, const float* logits, int32_t* idx, float* w,
                          uint8_t* hist, uint8_t* rank_hist, hipStream_t st) {
    // k = 8 picks from 8 groups with up to 8 experts per lane (up to 256 or
    // 512 experts): the shape of the DeepSeek-style configurations.  (With
    // more experts per lane the unrolled rounds run out of scalar registers.)
    const bool k8g8 = EPL <= 8 && s.k == 8 && s.G == 8;
    if constexpr (EPL <= 8) {
        if (k8g8 && mc == 0) return launch_pair<EPL, 0, 8, 8>(s, tpw, lpg_log2, logits, idx, w, hist, rank_hist, st);
        if (k8g8 && mc == 2) return launch_pair<EPL, 2, 8, 8>(s, tpw, lpg_log2, logits, idx, w, hist, rank_hist, st);
    }
    if (mc == 0) return launch_pair<EPL, 0, 0, 0>(s, tpw, lpg_log2, logits, idx, w, hist, rank_hist, st);
    if (mc == 1) return launch_pair<EPL, 1, 0, 0>(s, tpw, lpg_log2, logits, idx, w, hist, rank_hist, st);
    return launch_pair<EPL, 2, 0, 0>(s, tpw, lpg_log2, logits, idx, w, hist, rank_hist, st);
}

// The pair kernel applies with `tpw` tokens per wavefront (LPT = 64 / tpw
// lanes per token): E/LPT experts per lane, a power of two from 4 to 32 (the
// kernel's instances, read 16 bytes at a time), E <= 1024, m <= 2, and
// either every group is kept or a group is a power-of-two run of whole lanes
// of the token's lanes.
bool pair_gate_shape(const Shape& s, int tpw, int* epl, int* lpg_log2, int* mc) {
    const int LPT = kWave / tpw;
    if (s.E % LPT != 0 || s.E < 4 * LPT || s.E > 32 * LPT || s.E > 1024 || s.m > 2) return false;
    const int GS = s.E / s.G;
    *epl = s.E / LPT;
    if ((*epl & (*epl - 1)) != 0) return false;  // 4, 8, 16 or 32 experts per lane
    *lpg_log2 = 0;
    while ((*epl << *lpg_log2) < GS) ++*lpg_log2;
    const bool lanes_ok = GS % *epl == 0 && (*epl << *lpg_log2) == GS && (1 << *lpg_log2) <= LPT;
    if (s.TG != s.G && !lanes_ok) return false;
    *mc = s.TG == s.G ? 0 : s.m;
    return true;
}

// Tokens per wavefront for this shape (0: the pair kernel does not apply).
// One up to GATE_ONE_TOKEN_MAX_T tokens, and at every size when the pick
// rounds read sorted keys (four experts per lane, k = 8, G = 8: 6000 tokens
// 9.0 -> 7.5 us, 16384 tokens 13.7 -> 13.0 us against two per wavefront).
int pair_tpw(const Shape& s, int* epl, int* lpg_log2, int* mc) {
    if (pair_gate_shape(s, 1, epl, lpg_log2, mc) &&
        (s.T <= GATE_ONE_TOKEN_MAX_T || (*epl == 4 && s.k == 8 && s.G == 8)))
        return 1;
    if (pair_gate_shape(s, 2, epl, lpg_log2, mc)) return 2;
    return 0;
}

hipError_t launch_pair_any(const Shape& s, int tpw, int epl, int lpg_log2, int mc, const float* logits,
                           int32_t* idx, float* w, uint8_t* hist, uint8_t* rank_hist, hipStream_t st) {
    if (epl == 4) return launch_pair_mc<4>(s, tpw, mc, lpg_log2, logits, idx, w, hist, rank_hist, st);
    if (epl == 8) return launch_pair_mc<8>(s, tpw, mc, lpg_log2, logits, idx, w, hist, rank_hist, st);
    if (epl == 16) return launch_pair_mc<16>(s, tpw, mc, lpg_log2, logits, idx, w, hist, rank_hist, st);
    if (epl == 32) return launch_pair_mc<32>(s, tpw, mc, lpg_log2, logits, idx, w, hist, rank_hist, st);
    return hipErrorInvalidValue;  // pair_gate_shape admits no other count
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
            const float4 v = reinterpret_cast<const float4*>(logits)[i];
            float f[4] = {v.x, v.y, v.z, v.w};
            sigmoid_lane(f);
            reinterpret_cast<float4*>(scores)[i] = float4{f[0], f[1], f[2], f[3]};
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
    {
        int pepl = 0, lpg_log2 = 0, pmc = 0;
        const int tpw = pair_tpw(s, &pepl, &lpg_log2, &pmc);
        if (tpw > 0)
            return launch_pair_any(s, tpw, pepl, lpg_log2, pmc, logits, topk_idx, topk_w, nullptr, nullptr, stream);
    }
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

bool route_hist_supported(const Shape& s) {
    int epl, lpg_log2, mc;
    return s.E <= kMaxExpertsHist && s.R <= s.E && pair_tpw(s, &epl, &lpg_log2, &mc) > 0;
}

int route_hist_columns(const Shape& s) { return (s.T + kPairTokens - 1) / kPairTokens; }

int route_hist_column_tokens() { return kPairTokens; }

hipError_t launch_route_hist(const Shape& s, const float* logits, int32_t* topk_idx, float* topk_w, uint8_t* hist,
                             uint8_t* rank_hist, hipStream_t stream) {
    if (s.T == 0) return hipSuccess;
    int epl = 0, lpg_log2 = 0, mc = 0;
    const int tpw = pair_tpw(s, &epl, &lpg_log2, &mc);
    if (tpw == 0) return hipErrorInvalidValue;
    return launch_pair_any(s, tpw, epl, lpg_log2, mc, logits, topk_idx, topk_w, hist, rank_hist, stream);
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
