/*
 * moe_oracle.c -- plain, slow CPU oracle of one GPU's forward pass through a
 * routed (expert-parallel) MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code with the HIP library.
 *
 * What it computes (the five stages of an MoE layer under expert parallelism,
 * Weave: "Fine-Grained Dynamic SM Scheduling in an MoE Megakernel", §2.1 and
 * Figure 3): a learned gate picks top-k experts per token; dispatch groups the
 * routed tokens by expert; each expert runs GEMM0 (up and gate projections),
 * the SiLU-times-multiply activation and GEMM1 (down projection); combine sums
 * the expert outputs weighted by the gates, back in token order.  The same
 * pages' schedulers change only the order of tiles, never the math (X-Stage,
 * §5.3 and §7 on MegaMoE), so a direct evaluation of the definition is the
 * oracle.
 *
 * Precision (readings where the pages are silent):
 *  - Router logits are computed in float32 in one defined order, because they
 *    decide integers (the expert ids): each logit is the sum over 16 equal,
 *    contiguous chunks of the hidden dimension; each chunk is summed
 *    sequentially from +0.0f in ascending index; the 16 chunk sums are
 *    combined by a balanced pairwise tree ((s0+s1)+(s2+s3))+...; then the
 *    optional float32 bias is added.  Every bf16*bf16 product is exact in
 *    float32, so a fused multiply-add and a multiply-then-add agree.
 *  - Selection: the k largest logits, ties broken toward the lower expert id,
 *    listed by (logit descending, id ascending).
 *  - Gates: softmax over the k selected logits (the renormalised softmax),
 *    evaluated in double and stored as float.
 *  - Expert FFN and combine in double, with no intermediate rounding:
 *    h = silu(x.Wg) * (x.Wu), silu(z) = z / (1 + exp(-z)); y = h.Wd;
 *    out[t] = sum over local slots j (ascending) of gate[t,j] * y[t,j].
 *  - Dispatch order: stable by source token inside each expert segment;
 *    segments in expert order, unpadded.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC.  OpenMP only splits
 * independent tokens/rows across threads; it does not reorder any sum.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

static inline float bf(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

int oracle_version(void) { return 1; }

#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int oracle_num_threads(void) { return 1; }
void oracle_set_num_threads(int n) { (void)n; }
#endif

/* ---------------------------------------------------------------- routing */

/* One router logit in the defined float32 order (see header). d % 16 == 0. */
static float logit_defined(const uint16_t *x, const uint16_t *w, int64_t d) {
    const int64_t dc = d / 16;
    float s[16];
    for (int c = 0; c < 16; ++c) {
        float acc = 0.0f;
        for (int64_t i = c * dc; i < (c + 1) * dc; ++i) {
            float p = bf(x[i]) * bf(w[i]); /* exact */
            acc = acc + p;
        }
        s[c] = acc;
    }
    for (int width = 16; width > 1; width /= 2)
        for (int c = 0; c < width / 2; ++c)
            s[c] = s[2 * c] + s[2 * c + 1];
    return s[0];
}

/* Router logits l[t,e] (float32, defined order) for all tokens and experts.
 * x [T,d] bf16, w_router [E,d] bf16, bias [E] float or NULL, logits [T,E]. */
int oracle_router_logits(int64_t T, int64_t d, int64_t E, const uint16_t *x,
                         const uint16_t *w_router, const float *bias, float *logits) {
    if (T < 0 || d <= 0 || d % 16 != 0 || E <= 0 || !x || !w_router || !logits)
        return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t e = 0; e < E; ++e) {
            float l = logit_defined(x + t * d, w_router + e * d, d);
            if (bias) l = l + bias[e];
            logits[t * E + e] = l;
        }
    return ORACLE_OK;
}

/* Same logits in double (exact bf16 products, double sums), for error-bound
 * checks of the float32 order. */
int oracle_router_logits_f64(int64_t T, int64_t d, int64_t E, const uint16_t *x,
                             const uint16_t *w_router, const float *bias, double *logits,
                             double *abs_dot) {
    if (T < 0 || d <= 0 || E <= 0 || !x || !w_router || !logits) return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t e = 0; e < E; ++e) {
            double s = 0.0, a = 0.0;
            for (int64_t i = 0; i < d; ++i) {
                double p = (double)bf(x[t * d + i]) * (double)bf(w_router[e * d + i]);
                s += p;
                a += fabs(p);
            }
            if (bias) s += (double)bias[e];
            logits[t * E + e] = s;
            if (abs_dot) abs_dot[t * E + e] = a;
        }
    return ORACLE_OK;
}

/* "a ranks before b": larger logit first, ties to the lower expert id. */
static int ranks_before(float la, int64_t a, float lb, int64_t b) {
    if (la > lb) return 1;
    if (la < lb) return 0;
    return a < b;
}

/* Top-k selection and renormalised-softmax gates from given logits.
 * ids [T,k] int32, gates [T,k] float. */
int oracle_topk_gates(int64_t T, int64_t E, int64_t k, const float *logits, int32_t *ids,
                      float *gates) {
    if (T < 0 || E <= 0 || k <= 0 || k > E || !logits || !ids || !gates) return ORACLE_EINVAL;
    int rc = ORACLE_OK;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * E;
        unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
        if (!taken) { rc = ORACLE_EINVAL; continue; }
        for (int64_t j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || ranks_before(l[e], e, l[best], best)) best = e;
            }
            taken[best] = 1;
            ids[t * k + j] = (int32_t)best;
        }
        free(taken);
        /* softmax over the selected logits, in double */
        double m = (double)l[ids[t * k]];
        double z = 0.0;
        for (int64_t j = 0; j < k; ++j) z += exp((double)l[ids[t * k + j]] - m);
        for (int64_t j = 0; j < k; ++j)
            gates[t * k + j] = (float)(exp((double)l[ids[t * k + j]] - m) / z);
    }
    return rc;
}

/* Full routing: logits (optional output), ids, gates. */
int oracle_route(int64_t T, int64_t d, int64_t E, int64_t k, const uint16_t *x,
                 const uint16_t *w_router, const float *bias, int32_t *ids, float *gates,
                 float *logits_out) {
    if (T < 0 || d <= 0 || d % 16 != 0 || E <= 0 || k <= 0 || k > E) return ORACLE_EINVAL;
    float *l = logits_out ? logits_out : (float *)malloc(sizeof(float) * (size_t)(T * E + 1));
    if (!l) return ORACLE_EINVAL;
    int rc = oracle_router_logits(T, d, E, x, w_router, bias, l);
    if (rc == ORACLE_OK) rc = oracle_topk_gates(T, E, k, l, ids, gates);
    if (!logits_out) free(l);
    return rc;
}

/* --------------------------------------------------------------- dispatch */

/* Expert histogram, exclusive offsets and the stable permutation.
 * Local experts are [e_lo, e_hi).  counts [E_loc], offsets [E_loc+1],
 * perm_src [T*k] (only the first offsets[E_loc] entries are written),
 * inv_perm [T,k] (-1 for a non-local slot). */
int oracle_permute(int64_t T, int64_t k, int64_t E, int64_t e_lo, int64_t e_hi,
                   const int32_t *ids, int32_t *counts, int32_t *offsets, int32_t *perm_src,
                   int32_t *inv_perm) {
    if (T < 0 || k <= 0 || e_lo < 0 || e_hi > E || e_lo >= e_hi || !ids || !counts || !offsets ||
        !perm_src || !inv_perm)
        return ORACLE_EINVAL;
    const int64_t EL = e_hi - e_lo;
    for (int64_t e = 0; e < EL; ++e) counts[e] = 0;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < k; ++j) {
            int64_t e = ids[t * k + j];
            if (e < 0 || e >= E) return ORACLE_EINVAL;
            if (e >= e_lo && e < e_hi) counts[e - e_lo] += 1;
        }
    offsets[0] = 0;
    for (int64_t e = 0; e < EL; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *run = (int32_t *)calloc((size_t)EL, sizeof(int32_t));
    if (!run) return ORACLE_EINVAL;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < k; ++j) {
            int64_t e = ids[t * k + j];
            if (e >= e_lo && e < e_hi) {
                int32_t pos = offsets[e - e_lo] + run[e - e_lo]++;
                perm_src[pos] = (int32_t)t;
                inv_perm[t * k + j] = pos;
            } else {
                inv_perm[t * k + j] = -1;
            }
        }
    free(run);
    return ORACLE_OK;
}

/* ------------------------------------------------------------- expert FFN */

/* SwiGLU FFN of one row through one expert, in double.
 * x [d] bf16; wg, wu [f,d] bf16; wd [d,f] bf16; h scratch [f]; y [d]. */
static void ffn_row(int64_t d, int64_t f, const uint16_t *x, const uint16_t *wg,
                    const uint16_t *wu, const uint16_t *wd, double *h, double *y) {
    for (int64_t n = 0; n < f; ++n) {
        double g = 0.0, u = 0.0;
        const uint16_t *rg = wg + n * d, *ru = wu + n * d;
        for (int64_t i = 0; i < d; ++i) {
            double xi = (double)bf(x[i]);
            g += xi * (double)bf(rg[i]);
            u += xi * (double)bf(ru[i]);
        }
        double silu = g / (1.0 + exp(-g));
        h[n] = silu * u;
    }
    for (int64_t o = 0; o < d; ++o) {
        double s = 0.0;
        const uint16_t *rd = wd + o * f;
        for (int64_t n = 0; n < f; ++n) s += h[n] * (double)bf(rd[n]);
        y[o] = s;
    }
}

/* FFN of n rows; row r goes through local expert expert_of_row[r] (0-based
 * among the local experts).  x_rows [n,d] bf16, weights of the E_loc local
 * experts, y [n,d] double.  Also returns h [n,f] double if h_out != NULL. */
int oracle_expert_rows(int64_t n, int64_t d, int64_t f, int64_t E_loc, const uint16_t *x_rows,
                       const int32_t *expert_of_row, const uint16_t *w_gate,
                       const uint16_t *w_up, const uint16_t *w_down, double *y, double *h_out) {
    if (n < 0 || d <= 0 || f <= 0 || E_loc <= 0 || !x_rows || !expert_of_row || !w_gate ||
        !w_up || !w_down || !y)
        return ORACLE_EINVAL;
    for (int64_t r = 0; r < n; ++r)
        if (expert_of_row[r] < 0 || expert_of_row[r] >= E_loc) return ORACLE_EINVAL;
    int rc = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
        int64_t e = expert_of_row[r];
        double *h = h_out ? h_out + r * f : (double *)malloc(sizeof(double) * (size_t)f);
        if (!h) { rc = ORACLE_EINVAL; continue; }
        ffn_row(d, f, x_rows + r * d, w_gate + e * f * d, w_up + e * f * d, w_down + e * d * f, h,
                y + r * d);
        if (!h_out) free(h);
    }
    return rc;
}

/* ---------------------------------------------------------------- combine */

/* out[t] = sum over slots j (ascending) with inv_perm[t,j] >= 0 of
 * gates[t,j] * y_perm[inv_perm[t,j]], in double.  y_perm [N,d] double. */
int oracle_combine(int64_t T, int64_t k, int64_t d, const double *y_perm, const int32_t *inv_perm,
                   const float *gates, double *out) {
    if (T < 0 || k <= 0 || d <= 0 || !inv_perm || !gates || !out) return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double *o = out + t * d;
        for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            int32_t p = inv_perm[t * k + j];
            if (p < 0) continue;
            double w = (double)gates[t * k + j];
            const double *yr = y_perm + (int64_t)p * d;
            for (int64_t c = 0; c < d; ++c) o[c] += w * yr[c];
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------ whole layer */

/* The layer's output for a list of tokens, computed token by token from the
 * definition: route the token, run its local selected experts, combine.
 * tokens [n] indices into x; ids/gates of those tokens are also returned
 * (ids_out [n,k], gates_out [n,k], both optional); out [n,d] double. */
int oracle_layer_tokens(int64_t n, const int64_t *tokens, int64_t T, int64_t d, int64_t f,
                        int64_t E, int64_t k, int64_t e_lo, int64_t e_hi, const uint16_t *x,
                        const uint16_t *w_router, const float *bias, const uint16_t *w_gate,
                        const uint16_t *w_up, const uint16_t *w_down, int32_t *ids_out,
                        float *gates_out, double *out) {
    if (n < 0 || !tokens || T < 0 || d <= 0 || d % 16 != 0 || f <= 0 || E <= 0 || k <= 0 ||
        k > E || e_lo < 0 || e_hi > E || e_lo >= e_hi || !x || !w_router || !w_gate || !w_up ||
        !w_down || !out)
        return ORACLE_EINVAL;
    for (int64_t r = 0; r < n; ++r)
        if (tokens[r] < 0 || tokens[r] >= T) return ORACLE_EINVAL;
    int rc = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
        const uint16_t *xt = x + tokens[r] * d;
        float *l = (float *)malloc(sizeof(float) * (size_t)E);
        int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
        float *g = (float *)malloc(sizeof(float) * (size_t)k);
        double *h = (double *)malloc(sizeof(double) * (size_t)f);
        double *y = (double *)malloc(sizeof(double) * (size_t)d);
        if (!l || !ids || !g || !h || !y) {
            rc = ORACLE_EINVAL;
        } else {
            oracle_router_logits(1, d, E, xt, w_router, bias, l);
            oracle_topk_gates(1, E, k, l, ids, g);
            double *o = out + r * d;
            for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
            for (int64_t j = 0; j < k; ++j) {
                int64_t e = ids[j];
                if (e < e_lo || e >= e_hi) continue;
                int64_t el = e - e_lo;
                ffn_row(d, f, xt, w_gate + el * f * d, w_up + el * f * d, w_down + el * d * f, h, y);
                for (int64_t c = 0; c < d; ++c) o[c] += (double)g[j] * y[c];
            }
            if (ids_out) memcpy(ids_out + r * k, ids, sizeof(int32_t) * (size_t)k);
            if (gates_out) memcpy(gates_out + r * k, g, sizeof(float) * (size_t)k);
        }
        free(l); free(ids); free(g); free(h); free(y);
    }
    return rc;
}

/* ------------------------------------------------ W8A8 (fp8) expert FFN */
/*
 * The W8A8 variant of the expert FFN that X-Stage ("Modeling Post-Issue
 * Backpressure in GPU Communication-Computation Fusion", §5.3) evaluates for
 * MegaMoE.  The pages name the precision only, so the recipe is a reading:
 *  - element format: OCP 8-bit floating point E4M3 ("fn": no infinities, one
 *    NaN pattern per sign, largest finite magnitude 448); a code is
 *    sign(1) | exponent(4, bias 7) | mantissa(3), exponent field 0 holding
 *    the subnormals M/8 * 2^-6;
 *  - one scale per row of each operand: per token for activations, per
 *    output channel for weights.  The scale of a row is the smallest power of
 *    two 2^e with max|row| <= 448 * 2^e (e clamped to >= -126; 1 for an
 *    all-zero row).  Dividing by a power of two is exact, so the code of an
 *    element is the only rounding: the E4M3 value nearest to x / 2^e, ties to
 *    the even code, magnitudes above 448 saturating to 448;
 *  - GEMM0: g = sx * sg[c] * sum_i dec(xq_i) dec(wgq[c,i]) (likewise u), all
 *    in double; h = silu(g) * u, rounded to bf16 (h is materialised in bf16
 *    between the two GEMMs, as in the bf16 path), then quantised per row like
 *    the activations;
 *  - GEMM1: y[o] = sh * sd[o] * sum_n dec(hq_n) dec(wdq[o,n]), in double.
 */

/* Value of an E4M3 code, from the format's definition (NaN for 0x7F/0xFF). */
double oracle_e4m3_value(int32_t code) {
    const int s = (code >> 7) & 1, E = (code >> 3) & 15, M = code & 7;
    if (E == 15 && M == 7) return NAN;
    const double mag = E == 0 ? ldexp((double)M / 8.0, -6) : ldexp(1.0 + (double)M / 8.0, E - 7);
    return s ? -mag : mag;
}

/* Code of the E4M3 value nearest to v (v finite), ties to the even code,
 * saturating at 448.  Finite non-negative codes 0..0x7E are in increasing
 * order of value, so a binary search finds the neighbours of |v|.  The sign
 * bit is the sign bit of v. */
static uint8_t e4m3_encode(float v) {
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    const double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);  /* saturation */
    int lo = 0, hi = 0x7E;  /* value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (oracle_e4m3_value(mid) <= a) lo = mid;
        else hi = mid;
    }
    const double dl = a - oracle_e4m3_value(lo), dh = oracle_e4m3_value(hi) - a;
    const int best = dl < dh ? lo : dh < dl ? hi : ((lo & 1) == 0 ? lo : hi);
    return (uint8_t)(sign | best);
}

/* Exported for the tests. */
int32_t oracle_e4m3_encode(float v) { return e4m3_encode(v); }

/* Exponent e of the row scale 2^e for a row whose largest magnitude is amax. */
static int row_scale_exp(double amax) {
    if (amax == 0.0) return 0;
    int e = -126;
    while (amax > ldexp(448.0, e)) ++e;
    return e;
}

/* Quantise one row of n float values (already exact floats). */
static void quant_row(int64_t n, const float *x, uint8_t *q, float *scale) {
    double amax = 0.0;
    for (int64_t i = 0; i < n; ++i) amax = fmax(amax, fabs((double)x[i]));
    const int e = row_scale_exp(amax);
    *scale = (float)ldexp(1.0, e);
    for (int64_t i = 0; i < n; ++i) q[i] = e4m3_encode((float)ldexp((double)x[i], -e));
}

/* rows x cols bf16 -> codes [rows, cols] and one float scale per row. */
int oracle_quantize_rows_e4m3(int64_t rows, int64_t cols, const uint16_t *x, uint8_t *q,
                              float *scale) {
    if (rows < 0 || cols <= 0 || !x || !q || !scale) return ORACLE_EINVAL;
    int rc = ORACLE_OK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float *row = (float *)malloc(sizeof(float) * (size_t)cols);
        if (!row) { rc = ORACLE_EINVAL; continue; }
        for (int64_t i = 0; i < cols; ++i) row[i] = bf(x[r * cols + i]);
        quant_row(cols, row, q + r * cols, scale + r);
        free(row);
    }
    return rc;
}

/* Nearest bf16 value to a double (ties to even), as a float. */
static float bf16_round(double v) {
    if (v == 0.0 || !isfinite(v)) return (float)v;
    int p;
    (void)frexp(v, &p);                 /* |v| in [2^(p-1), 2^p) */
    int q = p - 8;                      /* quantum of an 8-significant-bit value */
    if (q < -133) q = -133;             /* bf16 subnormal quantum */
    return (float)ldexp(nearbyint(ldexp(v, -q)), q);
}

/* W8A8 FFN of n rows; row r goes through local expert expert_of_row[r].
 * x_rows [n,d] bf16; wq_gate, wq_up [E_loc,f,d] and wq_down [E_loc,d,f] E4M3
 * codes with scales s_gate, s_up [E_loc,f] and s_down [E_loc,d]; y [n,d]
 * double; h_out [n,f] (optional) receives the bf16-rounded h. */
int oracle_expert_rows_fp8(int64_t n, int64_t d, int64_t f, int64_t E_loc,
                           const uint16_t *x_rows, const int32_t *expert_of_row,
                           const uint8_t *wq_gate, const float *s_gate, const uint8_t *wq_up,
                           const float *s_up, const uint8_t *wq_down, const float *s_down,
                           double *y, double *h_out) {
    if (n < 0 || d <= 0 || f <= 0 || E_loc <= 0 || !x_rows || !expert_of_row || !wq_gate ||
        !s_gate || !wq_up || !s_up || !wq_down || !s_down || !y)
        return ORACLE_EINVAL;
    for (int64_t r = 0; r < n; ++r)
        if (expert_of_row[r] < 0 || expert_of_row[r] >= E_loc) return ORACLE_EINVAL;
    double lut[256];
    for (int c = 0; c < 256; ++c) lut[c] = oracle_e4m3_value(c);
    int rc = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
        const int64_t e = expert_of_row[r];
        float *xr = (float *)malloc(sizeof(float) * (size_t)d);
        float *hb = (float *)malloc(sizeof(float) * (size_t)f);
        uint8_t *xq = (uint8_t *)malloc((size_t)d);
        uint8_t *hq = (uint8_t *)malloc((size_t)f);
        if (!xr || !hb || !xq || !hq) {
            rc = ORACLE_EINVAL;
        } else {
            float sx, sh;
            for (int64_t i = 0; i < d; ++i) xr[i] = bf(x_rows[r * d + i]);
            quant_row(d, xr, xq, &sx);
            for (int64_t c = 0; c < f; ++c) {
                const uint8_t *rg = wq_gate + (e * f + c) * d, *ru = wq_up + (e * f + c) * d;
                double g = 0.0, u = 0.0;
                for (int64_t i = 0; i < d; ++i) {
                    g += lut[xq[i]] * lut[rg[i]];
                    u += lut[xq[i]] * lut[ru[i]];
                }
                g *= (double)sx * (double)s_gate[e * f + c];
                u *= (double)sx * (double)s_up[e * f + c];
                hb[c] = bf16_round(g / (1.0 + exp(-g)) * u);
                if (h_out) h_out[r * f + c] = hb[c];
            }
            quant_row(f, hb, hq, &sh);
            for (int64_t o = 0; o < d; ++o) {
                const uint8_t *rd = wq_down + (e * d + o) * f;
                double s = 0.0;
                for (int64_t c = 0; c < f; ++c) s += lut[hq[c]] * lut[rd[c]];
                y[r * d + o] = s * (double)sh * (double)s_down[e * d + o];
            }
        }
        free(xr); free(hb); free(xq); free(hq);
    }
    return rc;
}

/* The two GEMMs of the W8A8 FFN on their own (same recipe as above), so that
 * each can be checked separately against a GPU that rounds differently.
 *
 * oracle_gate_up_rows_fp8: h[r,c] = silu(g) * u, in double and NOT rounded,
 * with g = sx * sg[c] * sum_i dec(xq_i) dec(wgq[c,i]) (u likewise), xq and sx
 * the row's own E4M3 codes and scale.  h [n,f] double. */
int oracle_gate_up_rows_fp8(int64_t n, int64_t d, int64_t f, int64_t E_loc,
                            const uint16_t *x_rows, const int32_t *expert_of_row,
                            const uint8_t *wq_gate, const float *s_gate, const uint8_t *wq_up,
                            const float *s_up, double *h) {
    if (n < 0 || d <= 0 || f <= 0 || E_loc <= 0 || !x_rows || !expert_of_row || !wq_gate ||
        !s_gate || !wq_up || !s_up || !h)
        return ORACLE_EINVAL;
    for (int64_t r = 0; r < n; ++r)
        if (expert_of_row[r] < 0 || expert_of_row[r] >= E_loc) return ORACLE_EINVAL;
    double lut[256];
    for (int c = 0; c < 256; ++c) lut[c] = oracle_e4m3_value(c);
    int rc = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
        const int64_t e = expert_of_row[r];
        float *xr = (float *)malloc(sizeof(float) * (size_t)d);
        uint8_t *xq = (uint8_t *)malloc((size_t)d);
        if (!xr || !xq) {
            rc = ORACLE_EINVAL;
        } else {
            float sx;
            for (int64_t i = 0; i < d; ++i) xr[i] = bf(x_rows[r * d + i]);
            quant_row(d, xr, xq, &sx);
            for (int64_t c = 0; c < f; ++c) {
                const uint8_t *rg = wq_gate + (e * f + c) * d, *ru = wq_up + (e * f + c) * d;
                double g = 0.0, u = 0.0;
                for (int64_t i = 0; i < d; ++i) {
                    g += lut[xq[i]] * lut[rg[i]];
                    u += lut[xq[i]] * lut[ru[i]];
                }
                g *= (double)sx * (double)s_gate[e * f + c];
                u *= (double)sx * (double)s_up[e * f + c];
                h[r * f + c] = g / (1.0 + exp(-g)) * u;
            }
        }
        free(xr); free(xq);
    }
    return rc;
}

/* oracle_down_rows_fp8: y[r,o] = sh[r] * sd[o] * sum_c dec(hq[r,c]) dec(wdq[o,c])
 * in double, from given codes hq [n,f] and row scales sh [n] of h. */
int oracle_down_rows_fp8(int64_t n, int64_t d, int64_t f, int64_t E_loc, const uint8_t *hq,
                         const float *sh, const int32_t *expert_of_row, const uint8_t *wq_down,
                         const float *s_down, double *y) {
    if (n < 0 || d <= 0 || f <= 0 || E_loc <= 0 || !hq || !sh || !expert_of_row || !wq_down ||
        !s_down || !y)
        return ORACLE_EINVAL;
    for (int64_t r = 0; r < n; ++r)
        if (expert_of_row[r] < 0 || expert_of_row[r] >= E_loc) return ORACLE_EINVAL;
    double lut[256];
    for (int c = 0; c < 256; ++c) lut[c] = oracle_e4m3_value(c);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
        const int64_t e = expert_of_row[r];
        for (int64_t o = 0; o < d; ++o) {
            const uint8_t *rd = wq_down + (e * d + o) * f;
            double s = 0.0;
            for (int64_t c = 0; c < f; ++c) s += lut[hq[r * f + c]] * lut[rd[c]];
            y[r * d + o] = s * (double)sh[r] * (double)s_down[e * d + o];
        }
    }
    return ORACLE_OK;
}
