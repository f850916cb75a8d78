/*
 * oracle.c -- plain CPU statement of MoE routing, layout, dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product path.  Single-threaded,
 * unblocked loops in the order the definitions are stated.  Built with
 * -ffp-contract=off so that every fp32 expression is evaluated exactly as
 * written (no implicit fused multiply-add).
 *
 * Page citations use the tags defined in oracle.h.
 */
#include "oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* ---------------------------------------------------------------------------
 * exp by Cody & Waite.  The constants are derived here from their
 * mathematical definitions rather than written out:
 *   L2E   = fp32(log2 e)
 *   C1    = fp32(ln 2) with the low 12 significand bits cleared, so that
 *           n * C1 is exact for |n| < 2^12
 *   C2    = fp32(ln 2 - C1)
 *   P[i]  = fp32(1 / i!)
 *   HI    = the smallest fp32 x with e^x > FLT_MAX (e^x then rounds to
 *           +inf), i.e. the first fp32 value above ln(FLT_MAX)
 *   LO    = the smallest fp32 x with e^x >= 2^-126 (the smallest normal),
 *           i.e. the first fp32 value at or above ln(2^-126)
 * Range: x >= HI -> +inf; x < LO -> 0 (no subnormal results).  In between,
 * n = rint(x * L2E) lies in [-126, 128]; p * 2^n is formed as
 * (p * 2^n1) * 2^n2 with n1 = floor(n / 2), n2 = n - n1, both factors
 * normal, so n = 128 (x just below HI) and n = -126 need no special case and
 * every step is one correctly rounded operation.  NaN propagates.
 * ------------------------------------------------------------------------- */
static int   g_consts_ready = 0;
static float g_l2e, g_c1, g_c2, g_p[8], g_hi, g_lo;

/* Runs when the library is loaded (before any caller's thread can reach
 * orc_expf), so the constants are never written while another thread reads
 * them; the calls below then only see g_consts_ready set. */
__attribute__((constructor)) static void exp_consts(void) {
    if (g_consts_ready) return;
    double ln2 = log(2.0);
    g_l2e = (float)(1.0 / ln2);
    g_c1 = u2f(f2u((float)ln2) & 0xFFFFF000u);
    g_c2 = (float)(ln2 - (double)g_c1);
    double fact = 1.0;
    for (int i = 0; i < 8; ++i) {
        if (i > 0) fact *= (double)i;
        g_p[i] = (float)(1.0 / fact);
    }
    double ln_max = log((double)FLT_MAX);
    g_hi = (float)ln_max;
    if ((double)g_hi <= ln_max) g_hi = nextafterf(g_hi, INFINITY);
    double ln_min = log(ldexp(1.0, -126));
    g_lo = (float)ln_min;
    if ((double)g_lo < ln_min) g_lo = nextafterf(g_lo, 0.0f);
    g_consts_ready = 1;
}

static float pow2i(int n) { return u2f((uint32_t)(n + 127) << 23); }  /* normal range only */

float orc_expf(float x) {
    exp_consts();
    if (x != x) return x;
    if (x >= g_hi) return INFINITY;
    if (x < g_lo) return 0.0f;
    float n = rintf(x * g_l2e);
    float r = fmaf(-n, g_c1, x);
    r = fmaf(-n, g_c2, r);
    float p = g_p[7];
    for (int i = 6; i >= 0; --i) p = fmaf(p, r, g_p[i]);
    int n1 = (int)floorf(n * 0.5f);
    int n2 = (int)n - n1;
    return (p * pow2i(n1)) * pow2i(n2);
}

float orc_expf_hi(void) { exp_consts(); return g_hi; }
float orc_expf_lo(void) { exp_consts(); return g_lo; }

float orc_sigmoid(float x) {
    return 1.0f / (1.0f + orc_expf(-x));
}

/* ---------------------------------------------------------------------------
 * OCP OFP8 E4M3 ("FN": no infinities, 0x7F/0xFF are NaN, largest finite
 * magnitude 448 = code 0x7E).  Value of code (s, e, m):
 *   e == 0 : (-1)^s * m * 2^-9                (subnormal)
 *   e >= 1 : (-1)^s * (8 + m) * 2^(e - 10)
 * Encoding rounds to the nearest code, ties to the even code, and saturates
 * magnitudes >= 448 to 448.  FP8 as the dispatch payload type: [NEWS]
 * feature list, [DAY2] "DeepEP的关键技术"; the E4M3 flavour is a reading.
 * ------------------------------------------------------------------------- */
uint8_t orc_e4m3_from_f32(float v) {
    uint8_t sign = (f2u(v) >> 31) ? 0x80 : 0x00;
    if (v != v) return (uint8_t)(sign | 0x7F);
    float a = fabsf(v);
    if (a >= 448.0f) return (uint8_t)(sign | 0x7E);
    if (a < 0x1p-6f) {
        /* subnormal range: code = nearest multiple of 2^-9; 8 * 2^-9 is the
         * smallest normal, whose code is 0x08 as well */
        float m = rintf(a * 0x1p9f);
        return (uint8_t)(sign | (uint8_t)m);
    }
    int ex;
    float f = frexpf(a, &ex);   /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;             /* a = mant * 2^e, mant in [1, 2) */
    float mant = 2.0f * f;
    float m = rintf((mant - 1.0f) * 8.0f);
    int mi = (int)m;
    if (mi == 8) { mi = 0; e += 1; }
    int code = ((e + 7) << 3) | mi;
    if (code > 0x7E) code = 0x7E;
    return (uint8_t)(sign | code);
}

float orc_e4m3_to_f32(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    float v = (e == 0) ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
    return s ? -v : v;
}

/* bf16 = the upper half of an fp32 pattern; rounding to nearest even adds
 * 0x7FFF plus the lowest kept bit before truncating. */
uint16_t orc_bf16_from_f32(float v) {
    uint32_t u = f2u(v);
    if (v != v) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

float orc_bf16_to_f32(uint16_t b) { return u2f((uint32_t)b << 16); }

void orc_expf_n(long n, const float* x, float* y) {
    for (long i = 0; i < n; ++i) y[i] = orc_expf(x[i]);
}

void orc_e4m3_from_f32_n(long n, const float* v, uint8_t* c) {
    for (long i = 0; i < n; ++i) c[i] = orc_e4m3_from_f32(v[i]);
}

void orc_bf16_from_f32_n(long n, const float* v, uint16_t* b) {
    for (long i = 0; i < n; ++i) b[i] = orc_bf16_from_f32(v[i]);
}

/* ---------------------------------------------------------------------------
 * Gating.  Group-limited gating is named by [NEWS] feature list and [DE];
 * the pages give no formula.  Readings: sigmoid scores; group score = sum
 * of the group's m best scores (m = k / TG by default); top-TG groups, then
 * top-k experts of those groups; weights normalised to sum to one.
 * ------------------------------------------------------------------------- */
void orc_scores(int T, int E, const float* logits, float* s) {
    for (long i = 0; i < (long)T * E; ++i) s[i] = orc_sigmoid(logits[i]);
}

/* a outranks b: larger score bits, then smaller index */
static int outranks(float sa, int ia, float sb, int ib) {
    uint32_t ua = f2u(sa), ub = f2u(sb);
    if (ua != ub) return ua > ub;
    return ia < ib;
}

int orc_select(int T, int E, int G, int TG, int k, int m, const float* s,
               int32_t* topk_idx, float* topk_w) {
    if (T < 0 || E <= 0 || G <= 0 || E % G != 0 || TG < 1 || TG > G) return -1;
    int GS = E / G;
    if (m < 1 || m > GS || k < 1 || k > TG * GS) return -1;

    float* gscore = (float*)malloc(sizeof(float) * G);
    char* gkept = (char*)malloc(G);
    char* taken = (char*)malloc(E);
    float* sel_s = (float*)malloc(sizeof(float) * k);
    for (int t = 0; t < T; ++t) {
        const float* st = s + (long)t * E;
        /* group scores: repeatedly take the best remaining expert of the
         * group and add it */
        for (int g = 0; g < G; ++g) {
            memset(taken, 0, E);
            float acc = 0.0f;
            for (int i = 0; i < m; ++i) {
                int best = -1;
                for (int e = g * GS; e < (g + 1) * GS; ++e)
                    if (!taken[e] && (best < 0 || outranks(st[e], e, st[best], best))) best = e;
                taken[best] = 1;
                acc = acc + st[best];
            }
            gscore[g] = acc;
        }
        /* keep the TG best groups */
        memset(gkept, 0, G);
        for (int i = 0; i < TG; ++i) {
            int best = -1;
            for (int g = 0; g < G; ++g)
                if (!gkept[g] && (best < 0 || outranks(gscore[g], g, gscore[best], best))) best = g;
            gkept[best] = 1;
        }
        /* the k best experts of the kept groups, in rank order */
        memset(taken, 0, E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (gkept[e / GS] && !taken[e] && (best < 0 || outranks(st[e], e, st[best], best))) best = e;
            taken[best] = 1;
            topk_idx[(long)t * k + j] = best;
            sel_s[j] = st[best];
        }
        float S = 0.0f;
        for (int j = 0; j < k; ++j) S = S + sel_s[j];
        for (int j = 0; j < k; ++j) topk_w[(long)t * k + j] = sel_s[j] / S;
    }
    free(gscore); free(gkept); free(taken); free(sel_s);
    return 0;
}

int orc_route(int T, int E, int G, int TG, int k, int m, const float* logits,
              int32_t* topk_idx, float* topk_w) {
    float* s = (float*)malloc(sizeof(float) * ((long)T * E + 1));
    orc_scores(T, E, logits, s);
    int rc = orc_select(T, E, G, TG, k, m, s, topk_idx, topk_w);
    free(s);
    return rc;
}

/* ---------------------------------------------------------------------------
 * Layout.  The host must learn how many rows each receiver gets ([DAY2]
 * caption under "DeepEP是什么": the CPU waits for the GPU's receive count).
 * Readings: one receive row per routed (token, expert) pair, grouped by
 * expert, tokens ascending within an expert; virtual rank r owns a
 * contiguous block of E/R experts.
 * ------------------------------------------------------------------------- */
int orc_layout(int T, int k, int E, int R, const int32_t* topk_idx,
               int32_t* cnt, int32_t* off, int32_t* ntok_rank, int32_t* slot,
               int32_t* recv_token) {
    if (T < 0 || k < 1 || E < 1 || R < 1 || E % R != 0) return -1;
    long P = (long)T * k;
    int EPR = E / R;

    for (int e = 0; e < E; ++e) cnt[e] = 0;
    for (long p = 0; p < P; ++p) {
        int e = topk_idx[p];
        if (e >= 0 && e < E) cnt[e] += 1;
    }
    off[0] = 0;
    for (int e = 0; e < E; ++e) off[e + 1] = off[e] + cnt[e];

    int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    for (long p = 0; p < P; ++p) {   /* row-major (t, j) order */
        int e = topk_idx[p];
        if (e >= 0 && e < E) {
            slot[p] = off[e] + fill[e];
            fill[e] += 1;
        } else {
            slot[p] = -1;
        }
    }
    free(fill);

    if (recv_token) {
        for (long r = 0; r < P; ++r) recv_token[r] = -1;
        for (long p = 0; p < P; ++p)
            if (slot[p] >= 0) recv_token[slot[p]] = (int32_t)(p / k);
    }

    char* seen = (char*)malloc((size_t)R);
    for (int r = 0; r < R; ++r) ntok_rank[r] = 0;
    for (int t = 0; t < T; ++t) {
        memset(seen, 0, (size_t)R);
        for (int j = 0; j < k; ++j) {
            int e = topk_idx[(long)t * k + j];
            if (e >= 0 && e < E) seen[e / EPR] = 1;
        }
        for (int r = 0; r < R; ++r) ntok_rank[r] += seen[r];
    }
    free(seen);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Low-latency receive layout: fixed rows per expert, positions in the order
 * the pairs are met (row-major), overflow dropped.
 * ------------------------------------------------------------------------- */
int orc_ll_layout(int T, int k, int E, int cap, const int32_t* topk_idx,
                  int32_t* count, int32_t* slot, int32_t* src) {
    if (T < 0 || k < 1 || E < 1 || cap < 1) return -1;
    long P = (long)T * k;
    for (int e = 0; e < E; ++e) count[e] = 0;
    for (long p = 0; p < P; ++p) {
        int e = topk_idx[p];
        if (e < 0 || e >= E) {
            slot[p] = -1;
            continue;
        }
        int pos = count[e];
        count[e] += 1;
        if (pos < cap) {
            slot[p] = e * cap + pos;
            src[(long)e * cap + pos] = (int32_t)(p / k);
        } else {
            slot[p] = -1;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Dispatch.  Sends each token to the experts its gate picked ([DAY2]
 * "DeepEP是什么"; [NEWS] feature list), with an FP8 payload for dispatch
 * ([NEWS] "具体性能方面").  Readings: E4M3 codes with one fp32 scale per
 * 128 channels of a token, scale = amax / 448 with amax floored at 1e-4.
 * ------------------------------------------------------------------------- */
void orc_dispatch_fp8(int T, int H, int k, int nrows, const uint16_t* x,
                      const int32_t* slot, uint8_t* q, float* sc) {
    int B = H / 128;
    uint8_t* qrow = (uint8_t*)malloc((size_t)H + 1);
    float* srow = (float*)malloc(sizeof(float) * ((size_t)B + 1));
    for (int t = 0; t < T; ++t) {
        const uint16_t* xt = x + (long)t * H;
        for (int b = 0; b < B; ++b) {
            float amax = 0.0f;
            for (int c = 0; c < 128; ++c) {
                float a = fabsf(orc_bf16_to_f32(xt[b * 128 + c]));
                if (a > amax) amax = a;
            }
            float a = amax > 1e-4f ? amax : 1e-4f;
            float inv = 448.0f / a;
            srow[b] = a / 448.0f;
            for (int c = 0; c < 128; ++c) {
                float v = orc_bf16_to_f32(xt[b * 128 + c]);
                qrow[b * 128 + c] = orc_e4m3_from_f32(v * inv);
            }
        }
        for (int j = 0; j < k; ++j) {
            int r = slot[(long)t * k + j];
            if (r < 0 || r >= nrows) continue;
            memcpy(q + (long)r * H, qrow, (size_t)H);
            memcpy(sc + (long)r * B, srow, sizeof(float) * (size_t)B);
        }
    }
    free(qrow);
    free(srow);
}

void orc_dispatch_bf16(int T, int H, int k, int nrows, const uint16_t* x,
                       const int32_t* slot, uint16_t* recv) {
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int r = slot[(long)t * k + j];
            if (r < 0 || r >= nrows) continue;
            memcpy(recv + (long)r * H, x + (long)t * H, sizeof(uint16_t) * (size_t)H);
        }
}

/* ---------------------------------------------------------------------------
 * Combine.  Brings the experts' outputs back to each token and accumulates
 * them ([DAY2] "DeepEP是什么", and the receive-and-accumulate stages in
 * "All-to-All通信"), in BF16 ([NEWS] "具体性能方面").  Reading: weighted by
 * the gate weights, fp32 accumulation in pick order, one bf16 rounding.
 * ------------------------------------------------------------------------- */
void orc_combine(int T, int H, int k, int nrows, const uint16_t* y,
                 const int32_t* slot, const float* w, uint16_t* out) {
    for (int t = 0; t < T; ++t)
        for (int c = 0; c < H; ++c) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) {
                int r = slot[(long)t * k + j];
                if (r < 0 || r >= nrows) continue;
                acc = fmaf(w[(long)t * k + j], orc_bf16_to_f32(y[(long)r * H + c]), acc);
            }
            out[(long)t * H + c] = orc_bf16_from_f32(acc);
        }
}

void orc_combine_f64(int T, int H, int k, int nrows, const uint16_t* y,
                     const int32_t* slot, const float* w, double* out) {
    for (int t = 0; t < T; ++t)
        for (int c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                int r = slot[(long)t * k + j];
                if (r < 0 || r >= nrows) continue;
                acc += (double)w[(long)t * k + j] * (double)orc_bf16_to_f32(y[(long)r * H + c]);
            }
            out[(long)t * H + c] = acc;
        }
}

/* ---------------------------------------------------------------------------
 * Per-rank deduplication: a token travels once to each rank it needs, and a
 * rank sums its own experts' outputs for the token before sending one row
 * back ([DAY2] "DeepEP是什么", "All-to-All通信").
 * ------------------------------------------------------------------------- */
static int first_on_rank(const int32_t* picks, int j, int E, int EPR) {
    int e = picks[j];
    if (e < 0 || e >= E) return 0;
    for (int jj = 0; jj < j; ++jj) {
        int e2 = picks[jj];
        if (e2 >= 0 && e2 < E && e2 / EPR == e / EPR) return 0;
    }
    return 1;
}

int orc_rank_layout(int T, int k, int E, int R, const int32_t* topk_idx,
                    int32_t* rank_count, int32_t* rank_offset,
                    int32_t* rank_slot, int32_t* rank_token) {
    if (T < 0 || k < 1 || E < 1 || R < 1 || E % R != 0) return -1;
    int EPR = E / R;
    long P = (long)T * k;
    for (int r = 0; r < R; ++r) rank_count[r] = 0;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j)
            if (first_on_rank(topk_idx + (long)t * k, j, E, EPR))
                rank_count[topk_idx[(long)t * k + j] / EPR] += 1;
    rank_offset[0] = 0;
    for (int r = 0; r < R; ++r) rank_offset[r + 1] = rank_offset[r] + rank_count[r];
    int32_t* fill = (int32_t*)calloc((size_t)R, sizeof(int32_t));
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            long p = (long)t * k + j;
            if (first_on_rank(topk_idx + (long)t * k, j, E, EPR)) {
                int r = topk_idx[p] / EPR;
                rank_slot[p] = rank_offset[r] + fill[r];
                fill[r] += 1;
            } else {
                rank_slot[p] = -1;
            }
        }
    free(fill);
    if (rank_token) {
        for (long row = 0; row < P; ++row) rank_token[row] = -1;
        for (long p = 0; p < P; ++p)
            if (rank_slot[p] >= 0) rank_token[rank_slot[p]] = (int32_t)(p / k);
    }
    return 0;
}

void orc_combine_rank_partial(int T, int H, int k, int E, int R, int nrows,
                              const uint16_t* y, const int32_t* topk_idx,
                              const int32_t* slot, const float* w,
                              const int32_t* rank_slot, int nrows_partial,
                              uint16_t* partial) {
    int EPR = E / R;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int row = rank_slot[(long)t * k + j];
            if (row < 0 || row >= nrows_partial) continue;
            int rank = topk_idx[(long)t * k + j] / EPR;
            for (int c = 0; c < H; ++c) {
                float acc = 0.0f;
                for (int jj = 0; jj < k; ++jj) {
                    int e = topk_idx[(long)t * k + jj];
                    if (e < 0 || e >= E || e / EPR != rank) continue;
                    int r = slot[(long)t * k + jj];
                    if (r < 0 || r >= nrows) continue;
                    acc = fmaf(w[(long)t * k + jj], orc_bf16_to_f32(y[(long)r * H + c]), acc);
                }
                partial[(long)row * H + c] = orc_bf16_from_f32(acc);
            }
        }
}

void orc_combine_ranks(int T, int H, int k, int nrows_partial,
                       const uint16_t* partial, const int32_t* rank_slot,
                       uint16_t* out) {
    for (int t = 0; t < T; ++t)
        for (int c = 0; c < H; ++c) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) {
                int row = rank_slot[(long)t * k + j];
                if (row < 0 || row >= nrows_partial) continue;
                acc = acc + orc_bf16_to_f32(partial[(long)row * H + c]);
            }
            out[(long)t * H + c] = orc_bf16_from_f32(acc);
        }
}
