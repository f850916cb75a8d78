// layout.hip -- routing layout: per-expert counts and offsets, per-rank
// token counts, and the canonical token -> receive-row map.
//
// The DeepEP blog "【Day2】DeepEP ..." (caption in "DeepEP是什么") has the host
// wait for the GPU's receive counts; here the receive buffer is statically
// T*k rows, so the counts stay on the device and nothing waits.
//
// Row order: one row per routed (token, expert) pair, grouped by expert,
// pairs in row-major (t, j) order within an expert.  The order is computed
// without order-dependent atomics, so the result is deterministic:
//   count  (C blocks)      per-block expert histograms and per-block counts
//                          of tokens per virtual rank (LDS atomic adds)
//   scan   (E + R blocks)  per-expert exclusive scan of the block
//                          histograms; per-rank totals
//   assign (C blocks)      expert offsets by a block-wide scan, then each
//                          wavefront sets one bit per pair in an LDS mask per
//                          expert (atomic OR commutes); a pair's rank inside
//                          its wavefront is the popcount of the mask bits of
//                          the lanes before it
// Workspace: hist [E][C] and rank counts [R][C], int32, C = ceil(T*k / P)
// with P = 64 * waves-per-block pairs per block.  Up to 64 count blocks the
// scan folds into the assign launch (layout_assign_scan_kernel); up to
// kSmallMaxPairs pairs one workgroup does all three steps in one launch
// (layout_small_kernel) and the workspace is not used.
#include "device.h"
#include "launch.h"

namespace ep {

namespace {

constexpr int kScanThreads = 256;

// waves per block of the count/assign kernels; the assign kernel needs
// (12 * W + 4) * E bytes of LDS
inline int layout_waves(int E) { return (100 * E <= 65536) ? 8 : 4; }

inline int layout_blocks(long P, int W) { return (int)((P + 64 * W - 1) / (64 * W)); }

// count blocks up to which the assign blocks scan the histograms themselves
// (two launches instead of three).  Measured per call on MI355X, 256
// experts, top-8: 1024 pairs 15.2 -> 11.4 us, 32768 pairs 14.9 -> 13.0 us;
// at 65536 pairs (128 blocks) 15.5 -> 16.0 us, so larger inputs keep the
// separate scan.
constexpr int kSelfScanMaxBlocks = 64;

// pairs up to which one workgroup does the whole layout in one launch
// (from 513 pairs a 1024-thread workgroup, when its LDS fits, so that all
// pairs are ranked in one chunk: 1024 pairs 6.8 -> 6.6 us).
// Measured per call on MI355X, 256 experts, top-8: 256 pairs 8.6 -> 5.7 us,
// 1024 pairs 8.0 -> 6.9 us; at 2048 pairs one workgroup is slower (9.0
// against 8.2 us).
constexpr long kSmallMaxPairs = 1024;
constexpr size_t kSmallMaxLds = 65536;

// exclusive block-wide prefix sum; `wsum` is LDS scratch of blockDim/64 ints.
// `again`: the caller scans again with the same scratch, so every wavefront
// must have read it before it returns; a single scan skips that barrier.
__device__ int block_exclusive_sum(int v, int* total, int* wsum, bool again) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int inc = wave_inclusive_sum(v);
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int pre = 0, tot = 0;
    for (int w = 0; w < nw; ++w) {
        const int x = wsum[w];
        pre += (w < wave) ? x : 0;
        tot += x;
    }
    if (again) __syncthreads();
    *total = tot;
    return pre + inc - v;
}

// Whether pick j of a token (expert ids at row[0..k)) is the token's first
// routed pick on the rank whose experts are [lo, lo + EPR): no earlier pick
// lies in that range (an unrouted id, negative or >= E, never does).  The
// earlier picks are read eight at a time with unconditional loads (indices
// clamped into the row, extra reads unused), so all eight are in flight
// together.
__device__ __forceinline__ bool first_on_rank(const int32_t* __restrict__ row, int j, int lo, int EPR) {
    bool first = true;
    for (int j0 = 0; j0 < j; j0 += 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = row[min(j0 + u, j - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (j0 + u < j && (unsigned)(v[u] - lo) < (unsigned)EPR) first = false;
    }
    return first;
}

__global__ __launch_bounds__(512) void layout_count_kernel(const int32_t* __restrict__ idx,
                                                           int32_t* __restrict__ hist,
                                                           int32_t* __restrict__ rk, long P, int k, int E,
                                                           int R, int EPR, int C) {
    extern __shared__ int32_t cnt_sm[];  // E expert counts, then R rank counts
    const int tid = threadIdx.x;
    // block c: XCD-contiguous order, so the column entries c of a histogram
    // row (adjacent ints) are written from one XCD's L2
    const int c = xcd_item(blockIdx.x, gridDim.x);
    for (int i = tid; i < E + R; i += blockDim.x) cnt_sm[i] = 0;
    __syncthreads();
    const long p = (long)c * blockDim.x + tid;
    if (p < P) {
        const int e = idx[p];
        if ((unsigned)e < (unsigned)E) {
            atomicAdd(&cnt_sm[e], 1);
            // a token counts once per rank: only its first pair on the rank adds
            const int r = e / EPR;
            const long t = p / k;
            if (first_on_rank(idx + t * k, (int)(p - t * k), r * EPR, EPR)) atomicAdd(&cnt_sm[E + r], 1);
        }
    }
    __syncthreads();
    for (int i = tid; i < E; i += blockDim.x) hist[(size_t)i * C + c] = cnt_sm[i];
    for (int i = tid; i < R; i += blockDim.x) rk[(size_t)i * C + c] = cnt_sm[E + i];
}

// block b < E: exclusive scan of hist[b][0..C) in place, cnt[b] = total;
// block E + r: ntok_rank[r] = sum of rk[r][0..C)
__global__ __launch_bounds__(kScanThreads) void layout_scan_kernel(int32_t* __restrict__ hist,
                                                                   const int32_t* __restrict__ rk,
                                                                   int32_t* __restrict__ cnt,
                                                                   int32_t* __restrict__ ntok_rank, int E,
                                                                   int C) {
    __shared__ int wsum[kScanThreads / 64];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    if (b < E) {
        int32_t* col = hist + (size_t)b * C;
        int carry = 0;
        for (int c0 = 0; c0 < C; c0 += kScanThreads) {
            const int c = c0 + tid;
            const int v = (c < C) ? col[c] : 0;
            int tile;
            const int ex = block_exclusive_sum(v, &tile, wsum, true);
            if (c < C) col[c] = carry + ex;
            carry += tile;
        }
        if (tid == 0) cnt[b] = carry;
    } else {
        const int32_t* row = rk + (size_t)(b - E) * C;
        int sum = 0;
        for (int c0 = 0; c0 < C; c0 += kScanThreads) {
            const int c = c0 + tid;
            const int v = (c < C) ? row[c] : 0;
            int tile;
            block_exclusive_sum(v, &tile, wsum, true);
            sum += tile;
        }
        if (tid == 0) ntok_rank[b - E] = sum;
    }
}

// Ranks inside one block of NT = W*64 consecutive pairs starting at pair
// p0 (thread tid takes pair p0 + tid, whose expert id `e` the caller has
// read: -1 if unrouted or past the end): each wavefront sets one bit per pair
// in an LDS mask per expert (64-bit atomic OR, which commutes), and a pair's
// rank within its wavefront is the popcount of the mask bits of the lanes
// before it.  `base[e]` holds the row of the block's first pair with expert
// e.  Writes slot and recv_token for the pairs below P.  `sync`: wait for
// the whole block before setting mask bits (needed when the masks were
// cleared since the block's last barrier).
template <int W>
__device__ void assign_pairs(int e, long p0, const int32_t* base, uint64_t* mask, int32_t* wpre,
                             int32_t* __restrict__ slot, int32_t* __restrict__ recv_token, long P, int k, int E,
                             int total, bool sync) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    constexpr int NT = W * 64;
    const long p = p0 + tid;
    if (sync) __syncthreads();
    if (e >= 0) atomicOr(reinterpret_cast<unsigned long long*>(&mask[wave * E + e]), 1ull << lane);
    __syncthreads();
    for (int i = tid; i < E; i += NT) {
        int run = 0;
        for (int w = 0; w < W; ++w) {
            wpre[w * E + i] = run;
            run += __popcll(mask[w * E + i]);
        }
    }
    __syncthreads();
    if (p < P) {
        int s = -1;
        if (e >= 0) {
            const uint64_t before = mask[wave * E + e] & ((1ull << lane) - 1ull);
            s = base[e] + wpre[wave * E + e] + __popcll(before);
            // rows lie below `total` by construction; the bound keeps a store
            // inside recv_token even if the counts were inconsistent
            if (recv_token && (unsigned)s < (unsigned)total) recv_token[s] = (int32_t)(p / k);
        }
        slot[p] = s;
        if (recv_token && p >= total) recv_token[p] = -1;
    }
}

// expert id of pair p for the assign step: -1 if unrouted or p >= P.
// `idx` may point to global memory or to LDS (the one-workgroup kernel
// stages the ids there), so this is a plain pointer load.
__device__ __forceinline__ int pair_expert(const int32_t* __restrict__ idx, long p, long P, int E) {
    if (p >= P) return -1;
    const int v = idx[p];
    return (unsigned)v < (unsigned)E ? v : -1;
}

// expert id of pair p0 + threadIdx.x, `idx` in GLOBAL memory only (chunks of
// at most 1024 pairs): -1 if unrouted or at or past P.  The load goes
// through a buffer resource over the chunk's pairs below P (none when
// P <= p0), so it is unconditional: no branch forces a wait on it before
// the value is used, and nothing outside [p0, P) is read (lanes past it
// read 0).  A buffer resource addresses global memory, so an LDS pointer
// must never reach it.
__device__ __forceinline__ int chunk_expert_global(const int32_t* __restrict__ idx, long p0, long P, int E) {
    const long n = P - p0;
    const uint32_t bytes = n <= 0 ? 0u : (uint32_t)(n < 1024 ? n : 1024) * 4u;
    const auto rs = buffer_rsrc(n > 0 ? idx + p0 : idx, bytes);
    const int v = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)threadIdx.x * 4, 0, kCached);
    return (long)threadIdx.x < n && (unsigned)v < (unsigned)E ? v : -1;
}

template <int W>
__device__ void assign_block(const int32_t* __restrict__ idx, const int32_t* base, uint64_t* mask, int32_t* wpre,
                             int32_t* __restrict__ slot, int32_t* __restrict__ recv_token, long P, int k, int E,
                             int total, int c, bool sync) {
    const long p0 = (long)c * (W * 64);
    assign_pairs<W>(pair_expert(idx, p0 + threadIdx.x, P, E), p0, base, mask, wpre, slot, recv_token, P, k, E, total,
                    sync);
}

template <int W>
__global__ __launch_bounds__(W * 64) void layout_assign_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ hist, const int32_t* __restrict__ cnt,
    int32_t* __restrict__ off, int32_t* __restrict__ slot, int32_t* __restrict__ recv_token, long P,
    int k, int E, int C) {
    extern __shared__ __align__(16) unsigned char asg_sm[];
    uint64_t* mask = reinterpret_cast<uint64_t*>(asg_sm);       // [W][E]
    int32_t* wpre = reinterpret_cast<int32_t*>(mask + W * E);    // [W][E]
    int32_t* base = wpre + W * E;                                // [E]
    __shared__ int wsum[W];

    const int tid = threadIdx.x;
    const int c = xcd_item(blockIdx.x, gridDim.x);  // XCD-contiguous, as in layout_assign_cols_kernel
    constexpr int NT = W * 64;

    for (int i = tid; i < W * E; i += NT) mask[i] = 0ull;

    // expert offsets: each thread scans EPT consecutive experts
    const int EPT = (E + NT - 1) / NT;
    const int e0 = tid * EPT;
    int local = 0;
    for (int i = 0; i < EPT; ++i)
        if (e0 + i < E) local += cnt[e0 + i];
    int total;
    int ex = block_exclusive_sum(local, &total, wsum, false);
    for (int i = 0; i < EPT; ++i) {
        const int e = e0 + i;
        if (e < E) {
            base[e] = ex + ((c < C) ? hist[(size_t)e * C + c] : 0);
            if (c == 0) off[e] = ex;
            ex += cnt[e];
        }
    }
    if (c == 0 && tid == 0) off[E] = total;
    assign_block<W>(idx, base, mask, wpre, slot, recv_token, P, k, E, total, c, false);
}

// Assign without a separate scan launch: each block sums the block
// histograms of every expert itself (the total, and the part before its own
// block), scans the totals into expert offsets, and block 0 writes the
// counts, offsets and per-rank token counts.  For up to kSelfScanMaxBlocks
// count blocks, where reading E * C ints per block stays cheap.
template <int W>
__global__ __launch_bounds__(W * 64) void layout_assign_scan_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ hist, const int32_t* __restrict__ rk,
    int32_t* __restrict__ cnt, int32_t* __restrict__ ntok_rank, int32_t* __restrict__ off,
    int32_t* __restrict__ slot, int32_t* __restrict__ recv_token, long P, int k, int E, int R, int C) {
    extern __shared__ __align__(16) unsigned char as_sm[];
    uint64_t* mask = reinterpret_cast<uint64_t*>(as_sm);        // [W][E]
    int32_t* wpre = reinterpret_cast<int32_t*>(mask + W * E);    // [W][E], used by the assign step only
    int32_t* base = wpre + W * E;                                // [E]
    int32_t* tot = wpre;                                         // [E], lives in wpre until the assign step
    __shared__ int wsum[W];

    const int tid = threadIdx.x;
    const int c = xcd_item(blockIdx.x, gridDim.x);  // XCD-contiguous, as in layout_assign_cols_kernel
    constexpr int NT = W * 64;

    for (int i = tid; i < W * E; i += NT) mask[i] = 0ull;
    for (int e = tid; e < E; e += NT) {
        const int32_t* row = hist + (size_t)e * C;
        int all = 0, pre = 0;
#pragma unroll 16
        for (int i = 0; i < C; ++i) {
            const int v = row[i];
            all += v;
            pre += i < c ? v : 0;
        }
        tot[e] = all;
        base[e] = pre;
    }
    if (c == 0) {
        for (int r = tid; r < R; r += NT) {
            const int32_t* row = rk + (size_t)r * C;
            int all = 0;
#pragma unroll 16
            for (int i = 0; i < C; ++i) all += row[i];
            ntok_rank[r] = all;
        }
    }
    __syncthreads();

    // expert offsets: each thread scans EPT consecutive experts
    const int EPT = (E + NT - 1) / NT;
    const int e0 = tid * EPT;
    int local = 0;
    for (int i = 0; i < EPT; ++i)
        if (e0 + i < E) local += tot[e0 + i];
    int total;
    int ex = block_exclusive_sum(local, &total, wsum, false);
    for (int i = 0; i < EPT; ++i) {
        const int e = e0 + i;
        if (e < E) {
            base[e] += ex;
            if (c == 0) {
                off[e] = ex;
                cnt[e] = tot[e];
            }
            ex += tot[e];
        }
    }
    if (c == 0 && tid == 0) off[E] = total;
    assign_block<W>(idx, base, mask, wpre, slot, recv_token, P, k, E, total, c, false);
}

// Small inputs in one launch and one workgroup: the P expert ids are
// staged in LDS once; LDS histograms of experts and of first-on-rank pairs,
// a block-wide scan into the expert offsets, then the pairs in chunks of
// W*64 in order, each chunk ranked as in assign_block while `base` carries
// every expert's next row from chunk to chunk.  For P up to kSmallMaxPairs,
// where one workgroup beats two launches.
template <int W>
__global__ __launch_bounds__(W * 64) void layout_small_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ cnt, int32_t* __restrict__ ntok_rank,
    int32_t* __restrict__ off, int32_t* __restrict__ slot, int32_t* __restrict__ recv_token, long P, int k,
    int E, int R, int EPR) {
    extern __shared__ __align__(16) unsigned char sm_sm[];
    uint64_t* mask = reinterpret_cast<uint64_t*>(sm_sm);        // [W][E]
    int32_t* wpre = reinterpret_cast<int32_t*>(mask + W * E);    // [W][E]
    int32_t* base = wpre + W * E;                                // [E]
    int32_t* ids = base + E;                                     // [P] expert ids, -1 if unrouted
    int32_t* tot = wpre;                                         // [E] counts, then [R] rank counts; in wpre
    int32_t* rtot = wpre + E;                                    //   until the first chunk is ranked
    __shared__ int wsum[W];

    const int tid = threadIdx.x;
    constexpr int NT = W * 64;
    // eight unconditional buffer loads in flight per thread (out of range
    // ones read 0 and are not kept), so staging waits about once per 8*NT
    // pairs instead of once per NT
    const auto ir = buffer_rsrc(idx, (uint32_t)P * 4u);
    for (int p0 = tid; p0 < P; p0 += 8 * NT) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = (int)__builtin_amdgcn_raw_buffer_load_b32(ir, (p0 + u * NT) * 4, 0, kCached);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int p = p0 + u * NT;
            if (p < P) ids[p] = (unsigned)v[u] < (unsigned)E ? v[u] : -1;
        }
    }
    for (int i = tid; i < W * E; i += NT) mask[i] = 0ull;
    for (int i = tid; i < E + R; i += NT) tot[i] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += NT) {
        const int e = ids[p];
        if (e >= 0) {
            atomicAdd(&tot[e], 1);
            // a token counts once per rank: only its first pair on the rank
            // adds (an earlier pick in [lo, lo + EPR); unrouted ids are -1)
            const int r = e / EPR;
            const int lo = r * EPR;
            const int t = p / k;
            bool first = true;
            for (int q = t * k; q < p; ++q)
                if ((unsigned)(ids[q] - lo) < (unsigned)EPR) first = false;
            if (first) atomicAdd(&rtot[r], 1);
        }
    }
    __syncthreads();
    for (int r = tid; r < R; r += NT) ntok_rank[r] = rtot[r];

    // expert offsets: each thread scans EPT consecutive experts
    const int EPT = (E + NT - 1) / NT;
    const int e0 = tid * EPT;
    int local = 0;
    for (int i = 0; i < EPT; ++i)
        if (e0 + i < E) local += tot[e0 + i];
    int total;
    int ex = block_exclusive_sum(local, &total, wsum, false);
    for (int i = 0; i < EPT; ++i) {
        const int e = e0 + i;
        if (e < E) {
            base[e] = ex;
            off[e] = ex;
            cnt[e] = tot[e];
            ex += tot[e];
        }
    }
    if (tid == 0) off[E] = total;
    const int C = (int)((P + NT - 1) / NT);
    for (int c = 0; c < C; ++c) {
        assign_block<W>(ids, base, mask, wpre, slot, recv_token, P, k, E, total, c, c > 0);
        __syncthreads();
        // the next chunk's rows start after this chunk's pairs
        for (int i = tid; i < E; i += NT) {
            base[i] += wpre[(W - 1) * E + i] + __popcll(mask[(W - 1) * E + i]);
            for (int w = 0; w < W; ++w) mask[w * E + i] = 0ull;
        }
    }
}

// 16-byte column loads in flight per thread, added as packed bytes (8 * 16
// < 256 keeps the byte sums of a batch exact)
constexpr int kColBatch = 8;
// rank-column loads of block 0 issued with the expert columns (the rows per
// thread, C / (NT / R), at 256 columns of 32 ranks)
constexpr int kRankBatch = 16;

// Layout from the routing step's per-column histograms (route_hist:
// columns of CT tokens, hist [C][E] and rank_hist [C][R] bytes), in one
// launch.  Block b takes the CB columns [b*CB, (b+1)*CB), i.e. the pairs of
// tokens [b*CB*CT, (b+1)*CB*CT), in chunks of NT = W*64 pairs:
//  1. per expert, the sum of all columns (its count) and of the columns
//     before the block (its rows before the block).  A 16-byte load holds
//     sixteen experts' counts of one column; thread (g, d) reads piece d of
//     the rows g, g + RG, ... (TPR = E/16 threads per row, RG = NT / TPR row
//     groups), kColBatch loads at a time through one buffer resource over
//     the columns (rows past the last read zeros), adds them as packed bytes and
//     unpacks each batch into 16-bit pairs (a column count is at most
//     CT = 16, so a batch's sum fits a byte; a sum of all C <= 256 columns
//     fits 16 bits).  The row groups inside a wavefront meet by lane
//     exchanges, the W wavefronts in LDS.
//  2. expert offsets by a block-wide scan; block 0 writes the counts,
//     offsets and per-rank token counts.
//  3. slots as in assign_pairs, chunk by chunk, carrying each expert's next
//     row; the first chunk's expert ids are read at the start, so that load
//     overlaps step 1.
template <int W>
__global__ __launch_bounds__(W * 64) void layout_assign_cols_kernel(
    const int32_t* __restrict__ idx, const uint8_t* __restrict__ hist, const uint8_t* __restrict__ rank_hist,
    int32_t* __restrict__ cnt, int32_t* __restrict__ ntok_rank, int32_t* __restrict__ off,
    int32_t* __restrict__ slot, int32_t* __restrict__ recv_token, long P, int k, int E, int R, int C, int CB,
    int CT) {
    extern __shared__ __align__(16) unsigned char ac_sm[];
    constexpr int NT = W * 64;
    uint64_t* mask = reinterpret_cast<uint64_t*>(ac_sm);        // [W][E]
    int32_t* wpre = reinterpret_cast<int32_t*>(mask + W * E);    // [W][E]; expert totals before step 3
    int32_t* base = wpre + W * E;                                // [E]
    int32_t* red = base + E;                                     // [2][W][E]: sums before the block, all
    int32_t* rtot = red + 2 * W * E;                             // [R]
    __shared__ int wsum[W];
    const int tid = threadIdx.x;
    // XCD-contiguous blocks: an expert's rows from adjacent blocks are
    // adjacent, so the lines of recv_token (a few rows from each block) are
    // written from one or two XCDs' L2 instead of all eight (6.36 -> 6.16 us
    // at 4096 tokens, 256 experts, top-8)
    const int c0 = xcd_item(blockIdx.x, gridDim.x) * CB;
    const long p_begin = (long)c0 * CT * k;
    const long p_end = min(P, (long)(c0 + CB) * CT * k);
    int e_first = chunk_expert_global(idx, p_begin, p_end, E);
    // block 0 also sums the rank columns (below); its first kRankBatch rows
    // per thread are loaded here, unconditionally (rows clamped into range,
    // C >= 1), so their latency overlaps the expert columns'
    const int NR = NT / R, rr = tid % R, rg = tid / R;
    uint32_t rv[kRankBatch];
    if (blockIdx.x == 0) {
#pragma unroll
        for (int u = 0; u < kRankBatch; ++u) {
            const int row = rg + u * NR;
            rv[u] = rank_hist[(size_t)(row < C ? row : C - 1) * R + rr];
        }
    }

    for (int i = tid; i < W * E; i += NT) mask[i] = 0ull;
    for (int i = tid; i < R; i += NT) rtot[i] = 0;
    {
        const int TPR = E >> 4;     // threads per row (a power of two <= 64)
        const int RG = NT / TPR;    // row groups
        const int d = tid & (TPR - 1), g = tid / TPR;
        // unconditional loads through one resource over the C columns (the
        // workspace, global memory): a row past the last reads zeros, so
        // only the rows before the block need a mask
        const auto hr = buffer_rsrc(hist, (uint32_t)C * (uint32_t)E);
        uint32_t pp[8], pa[8];  // 16-bit count pairs: word 2q + h holds experts 4q + 2h (low), 4q + 2h + 1
#pragma unroll
        for (int i = 0; i < 8; ++i) pp[i] = pa[i] = 0u;
        for (int r0 = g; r0 < C; r0 += kColBatch * RG) {
            u32x4 v[kColBatch];
            const uint32_t o0 = (uint32_t)r0 * (uint32_t)E + 16u * (uint32_t)d;
#pragma unroll
            for (int u = 0; u < kColBatch; ++u) {
                const i32x4 t = __builtin_amdgcn_raw_buffer_load_b128(hr, (int)(o0 + (uint32_t)(u * RG * E)), 0,
                                                                      kCached);
                v[u] = u32x4{(uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w};
            }
            u32x4 bp = u32x4{0, 0, 0, 0}, ba = u32x4{0, 0, 0, 0};  // packed byte sums of the batch
#pragma unroll
            for (int u = 0; u < kColBatch; ++u) {
                const int r = r0 + u * RG;
                const u32x4 z = u32x4{0, 0, 0, 0};
                ba += v[u];
                bp += r < c0 ? v[u] : z;  // c0 <= C
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                pp[2 * q] += (bp[q] & 0xFFu) | ((bp[q] & 0xFF00u) << 8);
                pp[2 * q + 1] += ((bp[q] >> 16) & 0xFFu) | ((bp[q] >> 8) & 0xFF0000u);
                pa[2 * q] += (ba[q] & 0xFFu) | ((ba[q] & 0xFF00u) << 8);
                pa[2 * q + 1] += ((ba[q] >> 16) & 0xFFu) | ((ba[q] >> 8) & 0xFF0000u);
            }
        }
        // the 64 / TPR row groups of a wavefront: lanes d, d + TPR, ...
        // (16-bit pair sums stay below 2^16, so packed adds are exact)
        lane_residue_sums(pp, TPR);
        lane_residue_sums(pa, TPR);
        if ((tid & (kWave - 1)) < TPR) {
            const int wv = tid >> 6;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = 16 * d + 2 * i;
                red[wv * E + e] = (int)(pp[i] & 0xFFFFu);
                red[wv * E + e + 1] = (int)(pp[i] >> 16);
                red[(W + wv) * E + e] = (int)(pa[i] & 0xFFFFu);
                red[(W + wv) * E + e + 1] = (int)(pa[i] >> 16);
            }
        }
    }
    if (blockIdx.x == 0) {
        // tokens per rank: thread (rg, rr) sums byte rr of the rows rg,
        // rg + NR, ... (R divides NT, so every thread has an rg < NR); the
        // first kRankBatch rows were loaded with the expert columns
        int acc = 0;
#pragma unroll
        for (int u = 0; u < kRankBatch; ++u) acc += rg + u * NR < C ? (int)rv[u] : 0;
        for (int row = rg + kRankBatch * NR; row < C; row += NR) acc += (int)rank_hist[(size_t)row * R + rr];
        __syncthreads();  // rtot cleared
        atomicAdd(&rtot[rr], acc);
    }
    __syncthreads();
    for (int e = tid; e < E; e += NT) {
        int before = 0, all = 0;
#pragma unroll
        for (int g = 0; g < W; ++g) {
            before += red[g * E + e];
            all += red[(W + g) * E + e];
        }
        base[e] = before;
        wpre[e] = all;
    }
    // with E <= NT the scan below reads only the expert each thread summed
    // (thread e), so only a wider E needs the block to wait here
    if (E > NT) __syncthreads();
    if (blockIdx.x == 0)
        for (int i = tid; i < R; i += NT) ntok_rank[i] = rtot[i];

    // expert offsets: each thread scans EPT consecutive experts
    const int EPT = (E + NT - 1) / NT;
    const int e0 = tid * EPT;
    int local = 0;
    for (int i = 0; i < EPT; ++i)
        if (e0 + i < E) local += wpre[e0 + i];
    int total;
    int ex = block_exclusive_sum(local, &total, wsum, false);
    for (int i = 0; i < EPT; ++i) {
        const int e = e0 + i;
        if (e < E) {
            const int t_e = wpre[e];
            base[e] += ex;
            if (blockIdx.x == 0) {
                off[e] = ex;
                cnt[e] = t_e;
            }
            ex += t_e;
        }
    }
    if (blockIdx.x == 0 && tid == 0) off[E] = total;

    for (long p0 = p_begin; p0 < p_end; p0 += NT) {
        const int e = p0 == p_begin ? e_first : chunk_expert_global(idx, p0, p_end, E);
        assign_pairs<W>(e, p0, base, mask, wpre, slot, recv_token, p_end, k, E, total, p0 != p_begin);
        if (p0 + NT >= p_end) break;  // (uniform) no next chunk
        __syncthreads();
        // the next chunk's rows start after this chunk's pairs
        for (int i = tid; i < E; i += NT) {
            base[i] += wpre[(W - 1) * E + i] + __popcll(mask[(W - 1) * E + i]);
            for (int w = 0; w < W; ++w) mask[w * E + i] = 0ull;
        }
    }
}

template <int W>
hipError_t launch_assign(const Shape& s, long P, int C, const int32_t* idx, const int32_t* hist,
                         const int32_t* cnt, int32_t* off, int32_t* slot, int32_t* recv_token,
                         hipStream_t st) {
    const size_t lds = (size_t)(12 * W + 4) * s.E;
    const int blocks = C > 0 ? C : 1;  // block 0 writes the offsets even with no pairs
    hipLaunchKernelGGL(layout_assign_kernel<W>, dim3(blocks), dim3(W * 64), lds, st, idx, hist, cnt, off,
                       slot, recv_token, P, s.k, s.E, C);
    return hipGetLastError();
}

// Rank layout input: pick p keeps its rank id when it is the first pick of
// its token on that rank, else -1 (a later pick on the same rank, or an
// unrouted pick).
__global__ __launch_bounds__(256) void rank_first_kernel(const int32_t* __restrict__ idx, int32_t* __restrict__ ridx,
                                                         long P, int k, int E, int EPR) {
    const long p = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= P) return;
    const int e = idx[p];
    int out = -1;
    if ((unsigned)e < (unsigned)E) {
        const int r = e / EPR;
        const long t = p / k;
        if (first_on_rank(idx + t * k, (int)(p - t * k), r * EPR, EPR)) out = r;
    }
    ridx[p] = out;
}

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// the layout over rank buckets: one bucket per virtual rank
inline Shape rank_shape(const Shape& s) {
    Shape r = s;
    r.E = s.R;
    return r;
}

}  // namespace

size_t layout_workspace_bytes(const Shape& s) {
    const long P = (long)s.T * s.k;
    const int C = layout_blocks(P, layout_waves(s.E));
    const size_t b = (size_t)(s.E + s.R) * (size_t)C * sizeof(int32_t);
    return align256(b);
}

hipError_t launch_layout(const Shape& s, const int32_t* topk_idx, int32_t* cnt, int32_t* ntok_rank,
                         int32_t* off, int32_t* slot, int32_t* recv_token, void* ws, hipStream_t stream) {
    const long P = (long)s.T * s.k;
    const int W = layout_waves(s.E);
    const int C = layout_blocks(P, W);
    int32_t* hist = static_cast<int32_t*>(ws);
    int32_t* rk = hist + (size_t)s.E * C;
    const size_t small_lds = (size_t)(12 * W + 4) * s.E + (size_t)P * sizeof(int32_t);
    const size_t wide_lds = (size_t)(12 * 16 + 4) * s.E + (size_t)P * sizeof(int32_t);
    if (P > 512 && P <= kSmallMaxPairs && wide_lds <= kSmallMaxLds) {
        // one 1024-thread workgroup ranks up to 1024 pairs in a single chunk
        hipLaunchKernelGGL(layout_small_kernel<16>, dim3(1), dim3(16 * 64), wide_lds, stream, topk_idx, cnt, ntok_rank,
                           off, slot, recv_token, P, s.k, s.E, s.R, s.E / s.R);
        return hipGetLastError();
    }
    if (P <= kSmallMaxPairs && small_lds <= kSmallMaxLds) {
        const size_t lds = small_lds;
        if (W == 8)
            hipLaunchKernelGGL(layout_small_kernel<8>, dim3(1), dim3(8 * 64), lds, stream, topk_idx, cnt, ntok_rank,
                               off, slot, recv_token, P, s.k, s.E, s.R, s.E / s.R);
        else
            hipLaunchKernelGGL(layout_small_kernel<4>, dim3(1), dim3(4 * 64), lds, stream, topk_idx, cnt, ntok_rank,
                               off, slot, recv_token, P, s.k, s.E, s.R, s.E / s.R);
        return hipGetLastError();
    }
    if (C > 0) {
        hipLaunchKernelGGL(layout_count_kernel, dim3(C), dim3(W * 64), (size_t)(s.E + s.R) * sizeof(int32_t),
                           stream, topk_idx, hist, rk, P, s.k, s.E, s.R, s.E / s.R, C);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (C >= 1 && C <= kSelfScanMaxBlocks) {
        const size_t lds = (size_t)(12 * W + 4) * s.E;
        if (W == 8)
            hipLaunchKernelGGL(layout_assign_scan_kernel<8>, dim3(C), dim3(8 * 64), lds, stream, topk_idx, hist, rk, cnt,
                               ntok_rank, off, slot, recv_token, P, s.k, s.E, s.R, C);
        else
            hipLaunchKernelGGL(layout_assign_scan_kernel<4>, dim3(C), dim3(4 * 64), lds, stream, topk_idx, hist, rk, cnt,
                               ntok_rank, off, slot, recv_token, P, s.k, s.E, s.R, C);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(layout_scan_kernel, dim3(s.E + s.R), dim3(kScanThreads), 0, stream, hist, rk, cnt,
                       ntok_rank, s.E, C);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (W == 8) return launch_assign<8>(s, P, C, topk_idx, hist, cnt, off, slot, recv_token, stream);
    return launch_assign<4>(s, P, C, topk_idx, hist, cnt, off, slot, recv_token, stream);
}

// Columns of the routing step's histograms per assign block (CB) and the
// launch shape of layout_assign_cols_kernel; false if the shape does not
// fit its limits (E/16 threads per histogram row, a power of two <= 64; the
// ranks must fit the block; the LDS must fit 64 KiB).
namespace {
constexpr int kColsPerAssignBlock = 4;
constexpr size_t kColsMaxLds = 65536;

size_t cols_lds_bytes(int W, int E, int R) {
    return (size_t)(12 * W + 4) * E + (size_t)2 * W * E * 4 + (size_t)R * 4;
}
}  // namespace

bool layout_from_hist_supported(const Shape& s) {
    const int W = layout_waves(s.E);
    const int NT = W * 64;
    const int tpr = s.E / 16;
    if (s.E % 16 != 0 || tpr > 64 || (tpr & (tpr - 1)) != 0) return false;
    if (s.R > NT || NT % s.R != 0) return false;
    return cols_lds_bytes(W, s.E, s.R) <= kColsMaxLds;
}

hipError_t launch_layout_from_hist(const Shape& s, const int32_t* topk_idx, const uint8_t* hist,
                                   const uint8_t* rank_hist, int C, int CT, int32_t* cnt, int32_t* ntok_rank,
                                   int32_t* off, int32_t* slot, int32_t* recv_token, hipStream_t stream) {
    const long P = (long)s.T * s.k;
    const int W = layout_waves(s.E);
    const int CB = kColsPerAssignBlock;
    const int blocks = C > 0 ? (C + CB - 1) / CB : 1;  // block 0 writes the counts even with no tokens
    const size_t lds = cols_lds_bytes(W, s.E, s.R);
    if (W == 8)
        hipLaunchKernelGGL(layout_assign_cols_kernel<8>, dim3(blocks), dim3(8 * 64), lds, stream, topk_idx, hist,
                           rank_hist, cnt, ntok_rank, off, slot, recv_token, P, s.k, s.E, s.R, C, CB, CT);
    else
        hipLaunchKernelGGL(layout_assign_cols_kernel<4>, dim3(blocks), dim3(4 * 64), lds, stream, topk_idx, hist,
                           rank_hist, cnt, ntok_rank, off, slot, recv_token, P, s.k, s.E, s.R, C, CB, CT);
    return hipGetLastError();
}

// Workspace: the rank-input array [T*k], R scratch counters, then the
// layout workspace of the rank buckets.
size_t rank_layout_workspace_bytes(const Shape& s) {
    const size_t P = (size_t)s.T * s.k;
    return align256(P * sizeof(int32_t)) + align256((size_t)s.R * sizeof(int32_t)) +
           layout_workspace_bytes(rank_shape(s));
}

hipError_t launch_rank_layout(const Shape& s, const int32_t* topk_idx, int32_t* rank_count, int32_t* rank_offset,
                              int32_t* rank_slot, int32_t* rank_token, void* ws, hipStream_t stream) {
    const long P = (long)s.T * s.k;
    char* base = static_cast<char*>(ws);
    int32_t* ridx = reinterpret_cast<int32_t*>(base);
    int32_t* ntok = reinterpret_cast<int32_t*>(base + align256((size_t)P * sizeof(int32_t)));
    void* rest = base + align256((size_t)P * sizeof(int32_t)) + align256((size_t)s.R * sizeof(int32_t));
    if (P > 0) {
        hipLaunchKernelGGL(rank_first_kernel, dim3((unsigned)((P + 255) / 256)), dim3(256), 0, stream, topk_idx,
                           ridx, P, s.k, s.E, s.E / s.R);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // with one bucket per rank, the per-rank token count the layout also
    // computes equals the bucket count: it goes to scratch
    return launch_layout(rank_shape(s), ridx, rank_count, ntok, rank_offset, rank_slot, rank_token, rest, stream);
}

}  // namespace ep
