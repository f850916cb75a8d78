// launch.h -- host-side launchers of the library's kernels (internal).
//
// Each launcher assumes its arguments were validated by the C ABI layer
// (api.hip): sizes within the documented limits, pointers non-null and
// aligned.  They enqueue on `stream` and return the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ep {

struct Shape {
    int T, H, E, G, TG, k, R, m;
};

hipError_t launch_route(const Shape& s, const float* logits, int32_t* topk_idx, float* topk_w,
                        hipStream_t stream);
hipError_t launch_scores(const Shape& s, const float* logits, float* scores, hipStream_t stream);

// Routing that also counts its picks per column of route_hist_column_tokens()
// tokens: hist [columns][E] and rank_hist [columns][R] bytes (gate.hip);
// the layout's assign step then reads these columns (layout.hip).
bool route_hist_supported(const Shape& s);
int route_hist_columns(const Shape& s);
int route_hist_column_tokens();
hipError_t launch_route_hist(const Shape& s, const float* logits, int32_t* topk_idx, float* topk_w, uint8_t* hist,
                             uint8_t* rank_hist, hipStream_t stream);

size_t layout_workspace_bytes(const Shape& s);
hipError_t launch_layout(const Shape& s, const int32_t* topk_idx, int32_t* cnt, int32_t* ntok_rank,
                         int32_t* off, int32_t* slot, int32_t* recv_token, void* ws,
                         hipStream_t stream);

// The layout from route_hist's columns in one launch (layout.hip).
bool layout_from_hist_supported(const Shape& s);
hipError_t launch_layout_from_hist(const Shape& s, const int32_t* topk_idx, const uint8_t* hist,
                                   const uint8_t* rank_hist, int C, int CT, int32_t* cnt, int32_t* ntok_rank,
                                   int32_t* off, int32_t* slot, int32_t* recv_token, hipStream_t stream);

// Per-rank deduplicated layout (the layout over "first pick of the token on
// this rank" entries, one bucket per rank).
size_t rank_layout_workspace_bytes(const Shape& s);
hipError_t launch_rank_layout(const Shape& s, const int32_t* topk_idx, int32_t* rank_count, int32_t* rank_offset,
                              int32_t* rank_slot, int32_t* rank_token, void* ws, hipStream_t stream);

// In-rank partial combine, and the unit-weight combine of partial rows.
hipError_t launch_combine_rank_partial(const Shape& s, const uint16_t* y, const int32_t* topk_idx,
                                       const int32_t* slot, const float* w, const int32_t* rank_slot,
                                       uint16_t* partial, hipStream_t stream);
hipError_t launch_combine_ranks(const Shape& s, const uint16_t* partial, const int32_t* rank_slot, uint16_t* out,
                                hipStream_t stream);

hipError_t launch_dispatch_fp8(const Shape& s, const uint16_t* x, const int32_t* slot, uint8_t* recv,
                               float* recv_scales, hipStream_t stream);
hipError_t launch_dispatch_bf16(const Shape& s, const uint16_t* x, const int32_t* slot, uint16_t* recv,
                                hipStream_t stream);

// combine over y of `nrows` rows (T * k for the normal layout, E * cap for
// the low-latency one); slots outside [0, nrows) are skipped
hipError_t launch_combine(const Shape& s, int nrows, const uint16_t* y, const int32_t* slot, const float* w,
                          uint16_t* out, hipStream_t stream);

// Low-latency path limits: T * k pairs, experts (LDS counters), picks
constexpr int kMaxPairsLL = 8192;
constexpr int kMaxExpertsLL = 1024;
constexpr int kMaxTopkLL = 32;

hipError_t launch_dispatch_ll(const Shape& s, int cap, bool fp8, const uint16_t* x, const int32_t* topk_idx,
                              void* recv, float* recv_scales, int32_t* recv_count, int32_t* recv_src,
                              int32_t* slot, hipStream_t stream);

// Grid of the row kernels (dispatch, combine): one-wave workgroups, each
// taking one 64-lane piece of a token's row (`segs` pieces per row) per
// iteration; the grid is capped and the workgroups stride over the T * segs
// pieces, so any T fits the launch limits.
struct RowGrid {
    int segs;   // 64-lane pieces per row
    int items;  // T * segs
    int blocks; // workgroups launched
};

// XCD-contiguous item order: consecutive workgroups go to the 8 XCDs of
// MI355X in turn, so workgroup v runs on XCD v % 8; this map gives XCD x the
// contiguous run of items [x*q + min(x, r), ...) of its share (q = n / 8,
// r = n % 8), a bijection of [0, n).  The grid cap is a multiple of 8, so
// the mapping holds across grid-stride iterations.  Dispatch uses it from
// kXcdOrderMinTokens tokens on: adjacent receive rows (and their shared
// scale cache lines) then come from one XCD's L2.  Measured on MI355X
// (7168 channels, top-8, one launch after the layout): 8192 tokens 127 ->
// 121 us, 16384 tokens 252 -> 238 us, but 4096 tokens 56.5 -> 59.8 us.
// Combine is slower with it at every size (99 vs 90 us at 4096 tokens).
__device__ __forceinline__ int xcd_item(int v, int n) {
    const int q = n >> 3, r = n & 7, x = v & 7, i = v >> 3;
    return x * q + (x < r ? x : r) + i;
}

constexpr int kXcdOrderMinTokens = 8192;

inline RowGrid row_grid(int T, int lanes_per_row) {
    constexpr int kMaxBlocks = 1 << 20;
    RowGrid g;
    g.segs = (lanes_per_row + 63) / 64;
    g.items = T * g.segs;
    g.blocks = g.items < kMaxBlocks ? g.items : kMaxBlocks;
    return g;
}

}  // namespace ep
