/*
 * oracle.h -- plain CPU statement of MoE routing, layout, dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code: it exists so that tests/, the smoke check and the
 * benchmark's CPU-baseline leg can check the HIP library against an
 * independent, slow, obviously-correct statement of what it computes.  It
 * shares no source with the HIP library.
 *
 * What the method is comes from four web pages about DeepEP (an expert-
 * parallel MoE communication library):
 *   [GH#6]   mirror of GitHub issue "DeepEP ... Co-Packaged Optics (CPO)",
 *            section "Technical Overview of DeepEP"
 *   [NEWS]   news report on the DeepEP release (yunnanlong.com), feature list
 *            and section "具体性能方面" (performance)
 *   [DAY2]   blog "【Day2】DeepEP - 第一个用于 MoE 模型训练和推理的开源 EP 通信库",
 *            sections "DeepEP的关键技术", "DeepEP是什么", "All-to-All通信",
 *            "DeepEP 的性能表现"
 *   [DE]     German summary page "DeepEP" (flashmla.org)
 * The pages name the steps (group-limited gating, dispatch, combine, FP8
 * dispatch with BF16 combine, receive counts known to the host) but print no
 * formula.  Each function below states which reading it implements.
 *
 * Conventions: all arrays row-major; bf16 values are passed as their uint16
 * bit patterns; fp8 e4m3fn values as uint8 codes; indices are int32.
 */
#ifndef ORACLE_H
#define ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- scalar helpers ---------------------------------------------------- */

/* exp(x) in fp32 by Cody & Waite additive range reduction and a degree-7
 * Taylor polynomial evaluated with fused multiply-add (W. J. Cody, W. Waite,
 * "Software Manual for the Elementary Functions", 1980).  Every step is one
 * correctly rounded IEEE-754 operation, so any implementation that follows
 * the same steps returns the same bits.  +inf from the first fp32 value
 * whose exponential exceeds FLT_MAX (88.72283935546875); 0 below the first
 * fp32 value whose exponential is a normal number (-87.33654022216797), so
 * there are no subnormal results. */
float orc_expf(float x);
/* The two cut-offs above, as derived by the oracle from log(). */
float orc_expf_hi(void);
float orc_expf_lo(void);
/* 1 / (1 + orc_expf(-x)), fp32, correctly rounded add and divide. */
float orc_sigmoid(float x);
/* fp32 -> OCP OFP8 E4M3 (bias 7, max 448, no infinities) with round to
 * nearest even and saturation to +-448; NaN -> 0x7F. */
uint8_t orc_e4m3_from_f32(float v);
/* E4M3 code -> its value (0x7F/0xFF -> NaN). */
float orc_e4m3_to_f32(uint8_t c);
/* fp32 -> bf16 bits, round to nearest even; NaN -> 0x7FC0 (sign kept). */
uint16_t orc_bf16_from_f32(float v);
float orc_bf16_to_f32(uint16_t b);

/* The same helpers applied elementwise to n values (for sweeps in tests). */
void orc_expf_n(long n, const float* x, float* y);
void orc_e4m3_from_f32_n(long n, const float* v, uint8_t* c);
void orc_bf16_from_f32_n(long n, const float* v, uint16_t* b);

/* ---- the four steps ------------------------------------------------------ */

/* Gating scores: s[t,e] = orc_sigmoid(logits[t,e]).  T x E. */
void orc_scores(int T, int E, const float* logits, float* s);

/* Group-limited top-k selection from scores s (T x E):
 *   group g owns experts [g*E/G, (g+1)*E/G);
 *   group score = sum of the group's m largest scores, added largest first;
 *   keep the TG best groups (score desc, then group index asc);
 *   pick the k best experts of the kept groups (score desc, index asc);
 *   w_j = s_j / S with S = ((s_0 + s_1) + ...) in pick order.
 * Scores compare by their IEEE bit pattern as unsigned integers, which for
 * the non-negative values sigmoid produces is numeric order.
 * Returns 0, or -1 on an invalid configuration. */
int orc_select(int T, int E, int G, int TG, int k, int m, const float* s,
               int32_t* topk_idx, float* topk_w);

/* orc_scores followed by orc_select. */
int orc_route(int T, int E, int G, int TG, int k, int m, const float* logits,
              int32_t* topk_idx, float* topk_w);

/* Routing layout from topk_idx (T x k).  Entries outside [0, E) are
 * unrouted.  Outputs:
 *   cnt[e]          number of routed (t, j) pairs with expert e      (E)
 *   off[e]          exclusive prefix sum of cnt, off[E] = total    (E + 1)
 *   ntok_rank[r]    tokens with at least one routed expert on virtual rank
 *                   r, where rank r owns experts [r*E/R, (r+1)*E/R)    (R)
 *   slot[t,j]       off[e] + number of routed pairs (t', j') that precede
 *                   (t, j) in row-major order with the same expert; -1 for
 *                   unrouted entries                                (T x k)
 *   recv_token[row] token whose pair owns receive row `row`, -1 for rows
 *                   >= off[E]; may be NULL                          (T * k)
 * Returns 0, or -1 on an invalid configuration. */
int orc_layout(int T, int k, int E, int R, const int32_t* topk_idx,
               int32_t* cnt, int32_t* off, int32_t* ntok_rank, int32_t* slot,
               int32_t* recv_token);

/* Low-latency receive layout ([NEWS] feature list and [DAY2]
 * "DeepEP的关键技术": low-latency kernels for decoding; the layout is this
 * library's reading).  Expert e owns `cap` receive rows [e*cap, (e+1)*cap).
 * Going through the routed pairs (t, j) in row-major order, the pair's
 * position pos is the number of routed pairs already seen with the same
 * expert; it takes row e*cap + pos when pos < cap and is dropped otherwise.
 *   count[e]   routed pairs with expert e (all of them, dropped or not)   (E)
 *   slot[t,j]  e*cap + pos, or -1 when unrouted or dropped            (T x k)
 *   src[row]   token of each taken row; other entries untouched     (E*cap)
 * Returns 0, or -1 on an invalid configuration. */
int orc_ll_layout(int T, int k, int E, int cap, const int32_t* topk_idx,
                  int32_t* count, int32_t* slot, int32_t* src);

/* FP8 dispatch.  For each token t and 128-channel block b of x (T x H bf16):
 *   amax = max |x|,  a = max(amax, 1e-4),  inv = 448 / a,  sc = a / 448,
 *   q = e4m3(x * inv);
 * then for every j with 0 <= slot[t,j] < nrows, row slot[t,j] of q
 * (nrows x H codes) and of sc (nrows x H/128 fp32) receives the token's
 * values.  Rows no slot names are left untouched. */
void orc_dispatch_fp8(int T, int H, int k, int nrows, const uint16_t* x,
                      const int32_t* slot, uint8_t* q, float* sc);

/* BF16 dispatch: copies each token's row of x to its k receive rows. */
void orc_dispatch_bf16(int T, int H, int k, int nrows, const uint16_t* x,
                       const int32_t* slot, uint16_t* recv);

/* Combine, as the fp32 reduction the method states:
 *   acc = 0; for j = 0..k-1 with 0 <= slot[t,j] < nrows:
 *       acc = fma(w[t,j], y[slot[t,j], c], acc)      (fp32, one rounding)
 *   out[t,c] = bf16_rne(acc). */
void orc_combine(int T, int H, int k, int nrows, const uint16_t* y,
                 const int32_t* slot, const float* w, uint16_t* out);

/* Per-rank deduplicated layout ([DAY2] "DeepEP是什么" and "All-to-All通信":
 * the normal kernels send a token once towards each destination and fan it
 * out there, and accumulate expert outputs on the way back; the layout
 * below is this library's reading for virtual ranks).  Rank r owns experts
 * [r*E/R, (r+1)*E/R).  Pick j of token t is the token's first pick on its
 * rank when no earlier pick j' < j of t is routed to an expert of the same
 * rank.  One receive row per (token, rank) with a routed pick; rows grouped
 * by rank, tokens ascending within a rank:
 *   rank_count[r]    tokens with a routed pick on rank r                  (R)
 *   rank_offset[r]   exclusive prefix sum of rank_count, [R] = total  (R + 1)
 *   rank_slot[t,j]   the (t, rank) row when pick j is the token's first pick
 *                    on its rank; -1 for later picks on the same rank and
 *                    for unrouted picks                               (T x k)
 *   rank_token[row]  token of each row, -1 for rows >= rank_offset[R]; may
 *                    be NULL                                          (T * k)
 * Returns 0, or -1 on an invalid configuration. */
int orc_rank_layout(int T, int k, int E, int R, const int32_t* topk_idx,
                    int32_t* rank_count, int32_t* rank_offset,
                    int32_t* rank_slot, int32_t* rank_token);

/* In-rank partial combine: for every pick j that is its token's first pick
 * on rank r (rank_slot[t,j] = row in [0, nrows_partial)):
 *   acc = 0; for j' = 0..k-1 with pick j' routed to rank r and
 *       0 <= slot[t,j'] < nrows:  acc = fma(w[t,j'], y[slot[t,j'], c], acc)
 *   partial[row, c] = bf16_rne(acc)
 * Rows no rank_slot names are left untouched. */
void orc_combine_rank_partial(int T, int H, int k, int E, int R, int nrows,
                              const uint16_t* y, const int32_t* topk_idx,
                              const int32_t* slot, const float* w,
                              const int32_t* rank_slot, int nrows_partial,
                              uint16_t* partial);

/* Combine of the partial rows: out[t,c] = bf16_rne(((0 + p_0) + p_1) + ...)
 * where p_0, p_1, ... are the token's partial rows partial[rank_slot[t,j]]
 * for j ascending with 0 <= rank_slot[t,j] < nrows_partial. */
void orc_combine_ranks(int T, int H, int k, int nrows_partial,
                       const uint16_t* partial, const int32_t* rank_slot,
                       uint16_t* out);

/* Combine in fp64: out[t,c] = sum_j w[t,j] * y[slot[t,j], c], where each
 * product is exact in fp64 (24 + 8 significant bits) and the sum of k of
 * them is within k * 2^-53 * sum_j |w y| of the exact value.  Used to bound
 * the fp32 result. */
void orc_combine_f64(int T, int H, int k, int nrows, const uint16_t* y,
                     const int32_t* slot, const float* w, double* out);

#ifdef __cplusplus
}
#endif
#endif
