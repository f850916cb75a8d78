/*
 * ep.h -- C ABI of the MI355X (gfx950) MoE routing, dispatch and combine
 * library (libep.so).
 *
 * The library computes, on one GPU, the data-parallel core of expert-
 * parallel MoE communication as the DeepEP pages describe it:
 *   ep_route       group-limited top-k gating
 *   ep_get_layout  per-expert and per-rank receive counts, offsets, slots
 *   ep_dispatch    scatter of each token to its k experts' receive rows,
 *                  FP8 (E4M3 + fp32 scale per 128 channels) or BF16
 *   ep_combine     gather of each token's k expert outputs, weighted sum
 * Sources (titles of the pages, then the section):
 *   [NEWS]  news report on the DeepEP release (yunnanlong.com): feature list;
 *           "具体性能方面" (test settings: FP8 dispatch, BF16 combine)
 *   [DAY2]  blog "【Day2】DeepEP - 第一个用于 MoE 模型训练和推理的开源 EP 通信库":
 *           "DeepEP是什么" (dispatch and combine; the host waits for the
 *           receive count), "All-to-All通信" (combine accumulates),
 *           "DeepEP的关键技术" (native FP8 dispatch)
 *   [DE]    German summary page "DeepEP" (flashmla.org): group-limited gating
 * The pages print no formulas; every arithmetic rule below is the reading
 * this library implements and states.
 *
 * Expert parallelism is emulated on one GPU: virtual rank r owns experts
 * [r*E/R, (r+1)*E/R), and the receive buffers of all ranks are one buffer of
 * T*k rows ordered by expert, so rank r's rows start at expert_offset[r*E/R].
 *
 * Conventions for every call
 *  - Pointers named as device pointers must point to GPU memory (for
 *    example torch tensors) that stays alive until the work enqueued on
 *    `stream` has finished.  `cfg` is a host pointer read during the call.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    kernels and return; they never synchronise and never allocate.
 *  - Arrays are dense and row-major.  bf16 data is 16-bit brain float,
 *    fp8 data is OCP OFP8 E4M3 ("e4m3fn": max 448, no infinities).
 *  - Inputs are read-only.  Outputs are written in full unless stated
 *    otherwise, so callers need not clear them.  Inputs and outputs must not
 *    overlap.
 *  - Errors: negative return codes (below); validation happens before any
 *    HIP call, so an invalid call has no effect.  EP_ERR_HIP reports a
 *    failed kernel launch (ep_last_hip_error gives the hipError_t); the
 *    launch status is read with hipGetLastError, so an error that an
 *    earlier HIP call on the same thread left pending is reported (and
 *    cleared) by the next call here.
 *    Faults inside kernels surface as HIP errors at the caller's next
 *    synchronisation, as for any HIP kernel.
 *  - Calls are reentrant and keep no state between calls.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EP_API __attribute__((visibility("default")))

#define EP_ABI_VERSION 4

/* Return codes */
#define EP_OK               0
#define EP_ERR_INVALID_ARG (-1)  /* null pointer, inconsistent sizes       */
#define EP_ERR_ALIGNMENT   (-2)  /* pointer not aligned as required        */
#define EP_ERR_UNSUPPORTED (-3)  /* valid, but outside the kernels' limits */
#define EP_ERR_WORKSPACE   (-4)  /* workspace missing or too small         */
#define EP_ERR_HIP         (-5)  /* a kernel launch failed                 */
#define EP_ERR_SCRATCH_LIMIT (-6) /* needs more than the static scratch     */

/* Receive payload types for ep_dispatch */
#define EP_RECV_FP8_E4M3 0
#define EP_RECV_BF16     1

/* Problem description shared by all calls.
 *   num_tokens        T, 0 <= T <= 2^24, with T * topk < 2^31
 *   hidden            H, a multiple of 128, 128 <= H <= 16384
 *   num_experts       E, 1 <= E <= 1024
 *   num_groups        G, divides E, 1 <= G <= 64
 *   topk_groups       TG, 1 <= TG <= G
 *   topk              k, 1 <= k <= 32 and k <= TG * E / G
 *   num_ranks         R, divides E
 *   group_score_topm  m, the number of best scores summed into a group's
 *                     score; 0 selects max(1, k / TG); 1 <= m <= min(8, E/G)
 */
typedef struct ep_config {
    int32_t num_tokens;
    int32_t hidden;
    int32_t num_experts;
    int32_t num_groups;
    int32_t topk_groups;
    int32_t topk;
    int32_t num_ranks;
    int32_t group_score_topm;
} ep_config_t;

/* EP_ABI_VERSION of the built library. */
EP_API int ep_abi_version(void);

/* Static, NUL-terminated description of a return code. */
EP_API const char* ep_strerror(int code);

/* The hipError_t of the last failed launch seen by this library on the
 * calling thread (0 if none). */
EP_API int ep_last_hip_error(void);

/* EP_OK if `cfg` satisfies the limits above, else the error code any call
 * would return for it. */
EP_API int ep_validate_config(const ep_config_t* cfg);

/* Group-limited top-k gating ([NEWS] feature list; [DE]).
 *   logits    device, fp32 [T, E]
 *   topk_idx  device, int32 [T, k]  out: chosen experts, best first
 *   topk_w    device, fp32 [T, k]  out: gate weights, summing to one
 * Per token: s_e = 1 / (1 + exp(-logit_e)) in fp32, exp evaluated by Cody &
 * Waite range reduction and a degree-7 Taylor polynomial (exp(x) = +inf from
 * x = 88.72283935546875, the first fp32 value whose exponential exceeds
 * FLT_MAX, and 0 below -87.33654022216797, below which it is no longer a
 * normal number); a group's score is the sum of its m best scores,
 * largest first; the TG best groups are kept (score desc, index asc); the k
 * best experts of the kept groups are chosen (score desc, index asc); the
 * weight of pick j is s_j / ((s_0 + s_1) + ... + s_{k-1}).  Scores rank by
 * their IEEE bit pattern, which is numeric order for sigmoid's outputs.
 * Logits must not be NaN (the selection is then unspecified, still k
 * distinct in-range experts).
 * Alignment: 4 bytes.  Kernel: one 64-lane wavefront per token; above 4096
 * tokens, for the shapes whose lanes can hold runs of consecutive experts
 * (see ep_route_layout), one 32-lane half per token. */
EP_API int ep_route(const ep_config_t* cfg, const float* logits,
                    int32_t* topk_idx, float* topk_w, void* stream);

/* The gate's scores alone ([NEWS] feature list; [DE]): the router
 * probabilities that ep_route ranks, for callers that need them as well
 * (an auxiliary load-balancing loss, logging).
 *   logits    device, fp32 [T, E]
 *   scores    device, fp32 [T, E]  out: s = 1 / (1 + exp(-logit)), computed
 *             exactly as ep_route computes it (same exp, same roundings),
 *             so the bits equal those ep_route ranks
 * May alias logits (in place).  Alignment: 4 bytes.  Kernel: elementwise,
 * four values per lane when both pointers are 16-byte aligned. */
EP_API int ep_scores(const ep_config_t* cfg, const float* logits, float* scores, void* stream);

/* Bytes of device workspace ep_get_layout needs for `cfg` (0 if invalid). */
EP_API size_t ep_layout_workspace_bytes(const ep_config_t* cfg);

/* Routing layout ([DAY2] "DeepEP是什么": receive counts known before the
 * exchange).  One receive row per routed (token, expert) pair, rows grouped
 * by expert, tokens ascending within an expert.
 *   topk_idx       device, int32 [T, k]; entries outside [0, E) are
 *                  unrouted.  A token may name an expert more than once
 *                  (ep_route never does); each occurrence gets its own row.
 *   cnt_expert     device, int32 [E]     out: routed pairs per expert
 *   ntok_rank      device, int32 [R]     out: tokens with >= 1 routed expert
 *                                        on virtual rank r
 *   expert_offset  device, int32 [E + 1] out: exclusive prefix sum of
 *                                        cnt_expert; [E] = routed pairs
 *   slot           device, int32 [T, k]  out: receive row of pair (t, j) =
 *                  expert_offset[e] + number of earlier pairs (row-major
 *                  order) with the same expert; -1 if unrouted
 *   recv_token     device, int32 [T * k] out (may be NULL): token owning
 *                  each receive row; -1 for rows >= expert_offset[E]
 *   workspace      device, >= ep_layout_workspace_bytes(cfg) bytes, 16-byte
 *                  aligned; contents need not be initialised and are
 *                  scratch after the call
 * The receive buffer size is T*k rows whatever the routing, so the host
 * never has to wait for the counts.  Deterministic: counting uses
 * commutative operations only.  Alignment: 4 bytes (workspace 16). */
EP_API int ep_get_layout(const ep_config_t* cfg, const int32_t* topk_idx,
                         int32_t* cnt_expert, int32_t* ntok_rank,
                         int32_t* expert_offset, int32_t* slot,
                         int32_t* recv_token, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Bytes of device workspace ep_route_layout needs for `cfg` (0 if invalid). */
EP_API size_t ep_route_layout_workspace_bytes(const ep_config_t* cfg);

/* ep_route followed by ep_get_layout on its output, in fewer launches
 * (the [DE] gating, then [DAY2] "DeepEP是什么" receive counts).  Arguments
 * and results are those of the two calls (logits, topk_idx and topk_w as
 * for ep_route; counts, offsets, slot and recv_token as for ep_get_layout),
 * and the results are identical.  When the routing kernel that holds runs
 * of consecutive experts per lane applies (E = 128, 256, 512 or 1024,
 * m <= 2, a group covers whole lanes or TG = G), the assign step's scratch
 * fits its 64 KiB of LDS (E/16 a power of two; E up to 256 at 32 ranks) and
 * 1024 < T*k with T <= 4096, the routing kernel also counts its picks per
 * block of 16 tokens into the workspace, and one more launch sums those
 * counts, scans the offsets and assigns the rows, which saves the layout's
 * counting launch; other shapes run the two calls' kernels.
 *   workspace  device, >= ep_route_layout_workspace_bytes(cfg) bytes,
 *              16-byte aligned; scratch after the call
 * Errors as for ep_route and ep_get_layout. */
EP_API int ep_route_layout(const ep_config_t* cfg, const float* logits,
                           int32_t* topk_idx, float* topk_w,
                           int32_t* cnt_expert, int32_t* ntok_rank,
                           int32_t* expert_offset, int32_t* slot,
                           int32_t* recv_token, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Bytes of the device array ep_get_layout_static uses as its scratch. */
#define EP_STATIC_SCRATCH_BYTES (1u << 20)

/* ep_get_layout without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The
 * scratch ep_get_layout takes as `workspace` (ep_layout_workspace_bytes(cfg)
 * bytes) is instead a file-scope device array of EP_STATIC_SCRATCH_BYTES,
 * which the library holds on every GPU it runs on until the process ends;
 * its address on a device is looked up (hipGetSymbolAddress) on the first
 * call on that device and kept.  Arguments, results, determinism and
 * alignment as ep_get_layout.
 * Errors: as ep_get_layout, plus EP_ERR_SCRATCH_LIMIT, before any HIP call,
 * when ep_layout_workspace_bytes(cfg) > EP_STATIC_SCRATCH_BYTES (with 256
 * experts and 32 ranks: more than about 466,000 routed pairs; use
 * ep_get_layout then), and EP_ERR_HIP when the current device or the
 * array's address cannot be obtained.
 * Every call on one GPU uses that GPU's one array: calls whose work may
 * overlap on one GPU (streams not ordered with each other, or several host
 * threads) race, and the caller must serialise them.  The array keeps the
 * last call's contents; a call reads only scratch words it has written
 * first, so nothing needs clearing. */
EP_API int ep_get_layout_static(const ep_config_t* cfg, const int32_t* topk_idx,
                                int32_t* cnt_expert, int32_t* ntok_rank,
                                int32_t* expert_offset, int32_t* slot,
                                int32_t* recv_token, void* stream);

/* Dispatch ([DAY2] "DeepEP是什么"; FP8 payload: [NEWS] "具体性能方面",
 * [DAY2] "DeepEP的关键技术").
 *   x            device, bf16 [T, H], 16-byte aligned
 *   slot         device, int32 [T, k] from ep_get_layout; entries outside
 *                [0, T*k) are skipped
 *   recv_dtype   EP_RECV_FP8_E4M3 or EP_RECV_BF16
 *   recv         device, [T*k, H] of e4m3 codes (1 byte) or bf16, 16-byte
 *                aligned.  Row slot[t,j] receives token t; rows no slot
 *                names are not written.
 *   recv_scales  device, fp32 [T*k, H/128] for FP8 (NULL for BF16), 4-byte
 *                aligned; row slot[t,j] receives token t's scales
 * FP8, per token and 128-channel block: amax = max |x|, a = max(amax,
 * 1e-4), inv = 448 / a, scale = a / 448, code = e4m3(x * inv) rounded to
 * nearest even and saturated to +-448 (all fp32, correctly rounded).
 * BF16 copies the bits. */
EP_API int ep_dispatch(const ep_config_t* cfg, const void* x,
                       const int32_t* slot, int recv_dtype, void* recv,
                       float* recv_scales, void* stream);

/* Combine ([DAY2] "DeepEP是什么", and accumulation in "All-to-All通信";
 * BF16: [NEWS] "具体性能方面").
 *   y       device, bf16 [T*k, H] expert outputs in receive-row order,
 *           16-byte aligned
 *   slot    device, int32 [T, k]; pairs with slot outside [0, T*k) are
 *           skipped
 *   topk_w  device, fp32 [T, k]
 *   out     device, bf16 [T, H], 16-byte aligned
 * out[t,c] = bf16_rne(acc) where acc starts at +0 and, for j = 0..k-1 in
 * order, acc = fma(topk_w[t,j], y[slot[t,j], c], acc) in fp32. */
EP_API int ep_combine(const ep_config_t* cfg, const void* y,
                      const int32_t* slot, const float* topk_w, void* out,
                      void* stream);

/* Low-latency dispatch ([NEWS] feature list: low-latency kernels for
 * inference decoding; [DAY2] "DeepEP的关键技术" item 4 and "DeepEP 的性能表现":
 * 128 tokens per batch, FP8 dispatch, BF16 combine).  One kernel, no layout
 * pass: expert e owns `capacity` receive rows [e*capacity, (e+1)*capacity),
 * and routed pair (t, j) with expert e takes row e*capacity + pos, where pos
 * is the number of routed pairs before it in row-major (t, j) order with
 * the same expert (the in-expert order of ep_get_layout).  Pairs with
 * pos >= capacity are dropped (slot -1); capacity = T never drops a pair of
 * ep_route's output (it never repeats an expert within a token).
 *   x            device, bf16 [T, H], 16-byte aligned
 *   topk_idx     device, int32 [T, k]; entries outside [0, E) are unrouted
 *   capacity     rows per expert, >= 1, E * capacity < 2^31
 *   recv_dtype   EP_RECV_FP8_E4M3 or EP_RECV_BF16
 *   recv         device, [E * capacity, H] e4m3 codes or bf16, 16-byte
 *                aligned; rows no pair takes are not written
 *   recv_scales  device, fp32 [E * capacity, H/128] for FP8, NULL for BF16
 *   recv_count   device, int32 [E] out: routed pairs per expert (may exceed
 *                capacity; rows written = min(count, capacity))
 *   recv_src     device, int32 [E * capacity] out: token of each written
 *                row; other entries are not written
 *   slot         device, int32 [T, k] out: receive row of each pair, or -1
 * Payload arithmetic as ep_dispatch.  Limit: T * k <= 8192 (finding the
 * positions inside the dispatch costs O(T * k) per token), else
 * EP_ERR_UNSUPPORTED.  Alignment: 4 bytes for the int32 arrays. */
EP_API int ep_dispatch_ll(const ep_config_t* cfg, const void* x, const int32_t* topk_idx, int32_t capacity,
                          int recv_dtype, void* recv, float* recv_scales, int32_t* recv_count,
                          int32_t* recv_src, int32_t* slot, void* stream);

/* Low-latency combine: ep_combine over expert outputs y laid out as
 * ep_dispatch_ll's receive rows.
 *   capacity  as passed to ep_dispatch_ll
 *   y         device, bf16 [E * capacity, H], 16-byte aligned
 *   slot      device, int32 [T, k] from ep_dispatch_ll; entries outside
 *             [0, E * capacity) are skipped
 *   topk_w    device, fp32 [T, k]
 *   out       device, bf16 [T, H], 16-byte aligned
 * Arithmetic as ep_combine. */
EP_API int ep_combine_ll(const ep_config_t* cfg, int32_t capacity, const void* y, const int32_t* slot,
                         const float* topk_w, void* out, void* stream);

/* Per-rank deduplicated layout ([DAY2] "DeepEP是什么": the normal kernels
 * send a token once towards each destination and fan it out there;
 * "All-to-All通信": forward, then accumulate on the way back).  Pick j of
 * token t is the token's first pick on its virtual rank when no earlier
 * pick of t is routed to an expert of the same rank.  One receive row per
 * (token, rank) with a routed pick, rows grouped by rank, tokens ascending
 * within a rank (the order of ep_get_layout, one level up).
 *   topk_idx      device, int32 [T, k]; entries outside [0, E) are unrouted
 *   rank_count    device, int32 [R]     out: rows of rank r (tokens with a
 *                                       routed pick on r)
 *   rank_offset   device, int32 [R + 1] out: exclusive prefix sum of
 *                                       rank_count; [R] = rows in use
 *   rank_slot     device, int32 [T, k]  out: the (t, rank) row for a first
 *                                       pick on its rank, else -1
 *   rank_token    device, int32 [T * k] out (may be NULL): token of each
 *                                       row, -1 for rows >= rank_offset[R]
 *   workspace     device, >= ep_rank_layout_workspace_bytes(cfg) bytes,
 *                 256-byte aligned; scratch
 * Deduplicated dispatch is ep_dispatch with rank_slot as its slot map: each
 * token is written once per rank it needs (receive buffer of T*k rows, of
 * which rank_offset[R] are used).  Deterministic. */
EP_API size_t ep_rank_layout_workspace_bytes(const ep_config_t* cfg);
EP_API int ep_get_rank_layout(const ep_config_t* cfg, const int32_t* topk_idx, int32_t* rank_count,
                              int32_t* rank_offset, int32_t* rank_slot, int32_t* rank_token, void* workspace,
                              size_t workspace_bytes, void* stream);

/* In-rank partial combine: every rank sums its own experts' outputs for a
 * token before one row goes back ([DAY2] "All-to-All通信": forward and
 * accumulate).  For each first pick j on rank r of token t
 * (rank_slot[t,j] = row): acc = +0; for j' = 0..k-1 in order with pick j'
 * routed to rank r and slot[t,j'] in [0, T*k): acc = fma(topk_w[t,j'],
 * y[slot[t,j'], c], acc); partial[row, c] = bf16_rne(acc).
 *   y          device, bf16 [T*k, H] expert outputs in ep_get_layout's
 *              receive rows, 16-byte aligned
 *   topk_idx   device, int32 [T, k] (gives each pick's rank)
 *   slot       device, int32 [T, k] from ep_get_layout
 *   topk_w     device, fp32 [T, k]
 *   rank_slot  device, int32 [T, k] from ep_get_rank_layout
 *   partial    device, bf16 [T*k, H] out, 16-byte aligned; rows no
 *              rank_slot names are not written */
EP_API int ep_combine_rank_partial(const ep_config_t* cfg, const void* y, const int32_t* topk_idx,
                                   const int32_t* slot, const float* topk_w, const int32_t* rank_slot,
                                   void* partial, void* stream);

/* Combine of the partial rows: out[t,c] = bf16_rne(((+0 + p_0) + p_1) + ...)
 * over the token's partial rows p_i = partial[rank_slot[t,j]] for j
 * ascending with rank_slot[t,j] in [0, T*k), in fp32.
 *   partial    device, bf16 [T*k, H], 16-byte aligned
 *   rank_slot  device, int32 [T, k]
 *   out        device, bf16 [T, H], 16-byte aligned */
EP_API int ep_combine_ranks(const ep_config_t* cfg, const void* partial, const int32_t* rank_slot, void* out,
                            void* stream);

/* CU budget ([GH#6] "Technical Overview of DeepEP": SM-count control; [DAY2]
 * "All-to-All通信": communication kernels confined to a few SMs and
 * overlapped with the compute stream).  Creates a HIP stream whose kernels
 * run only on compute units [first_cu, first_cu + num_cus) of the current
 * device; pass it as `stream` to the calls above to cap the CUs they use,
 * and give the remaining CUs to a compute stream made the same way.  The
 * stream has the default priority.  On MI355X the HIP runtime accepts only
 * contiguous CU ranges, and a range paces the kernels by steps of 32 CUs:
 * prefill dispatch + combine take 505-508 us on every budget from 32 to 56
 * CUs and 297 us on 64 (measured), so budgets that are multiples of 32, or
 * below 32, use their CUs best.  A refused stream leaves no pending HIP error behind.
 *   first_cu, num_cus  0 <= first_cu, num_cus >= 1,
 *                      first_cu + num_cus <= the device's CU count
 *   stream             host, out: the new hipStream_t
 * Returns EP_ERR_INVALID_ARG for a bad range (no HIP call is made for a
 * negative or empty one) and EP_ERR_HIP if the runtime refuses the stream.
 * The caller owns the stream and releases it with ep_stream_destroy. */
EP_API int ep_stream_create_cu_range(int first_cu, int num_cus, void** stream);

/* Destroys a stream made by ep_stream_create_cu_range (after the work on it
 * has been waited for, as for hipStreamDestroy). */
EP_API int ep_stream_destroy(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */
