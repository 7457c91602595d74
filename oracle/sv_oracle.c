/*
 * sv_oracle.c -- plain, slow, single-threaded CPU oracle for speculative-sampling
 * verification.  TEST INFRASTRUCTURE ONLY: it is built, loaded and called by the
 * tests, by the smoke check and by the benchmark's CPU-baseline leg, never by the
 * product path.  It shares no code, header or table with the HIP library.
 *
 * What it computes, in the order the pages give the procedure
 * (ReSpec blog, "speculative decoding" steps 1-4; slime/Notion post, intro):
 *   the target scores the k drafted tokens in one pass; the target and draft
 *   distributions are compared token by token; the first token the draft got
 *   wrong is resampled from the target side; if every draft token passes, the
 *   target samples one more token.
 * The acceptance test is the one-shot test of Leviathan et al. 2023 that the
 * ReSpec notes name as Eq.1 ("2 . background", acceptance test): draft token x
 * at position i is kept iff u_i < min(1, p_i(x)/q_i(x)).  On rejection the
 * token is redrawn from the residual r(x) = max(0, p - q) / sum max(0, p - q)
 * (same section).  p and q are temperature softmaxes of the target and draft
 * logits over the whole vocabulary.  The top-32 target logits of every verified
 * position are the soft targets the ReSpec notes store for drafter KD
 * ("4 . G2", worked example: V = 151936, top-K = 32).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - temperature T scales both logits rows: p = softmax(t/T), q = softmax(d/T);
 *     T == 0 is greedy verification (argmax-prefix match);
 *   - uniforms[b] has k+2 slots: u[0..k-1] acceptance, u[k] residual draw,
 *     u[k+1] bonus draw;
 *   - draws are by inverse CDF over ascending token index: the first x whose
 *     cumulative mass C(x) exceeds tau = u * R, with R the unnormalised total;
 *   - q(x) == 0: ratio is +inf when p(x) > 0, else 0;
 *   - a residual with R == 0 (only through rounding) falls back to p_j;
 *   - top-32 order is (value desc, index asc) under float comparison; values
 *     are the raw target logits; fewer than 32 tokens pad with (-inf, -1).
 *
 * Everything is fp64: inputs (fp32 or bf16) convert exactly to double; every sum
 * runs sequentially in ascending token order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_TOPK 32

/* data-error bits per sequence (same meaning as the library's status bits) */
#define ORC_BAD_TOKEN 1
#define ORC_NAN 2
#define ORC_POSINF 4
#define ORC_EMPTY_ROW 8
#define ORC_BAD_UNIFORM 16

static double elem(const void *row, int dtype, int64_t x) {
    if (dtype == ORC_F32) return (double)((const float *)row)[x];
    uint32_t bits = (uint32_t)((const uint16_t *)row)[x] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ---- row statistics: m = max_x t_x, s = sum_x exp((t_x - m)/T) ---------- */
typedef struct { double m, s; int has_nan, has_posinf; } row_stats;

static row_stats stats_of(const void *row, int dtype, int V, double T) {
    row_stats r = { -INFINITY, 0.0, 0, 0 };
    for (int x = 0; x < V; ++x) {
        double v = elem(row, dtype, x);
        if (isnan(v)) r.has_nan = 1;
        else if (v == INFINITY) r.has_posinf = 1;
        else if (v > r.m) r.m = v;
    }
    if (r.has_nan || r.has_posinf || r.m == -INFINITY) return r;
    for (int x = 0; x < V; ++x) r.s += exp((elem(row, dtype, x) - r.m) / T);
    return r;
}

/* probability of token x under the temperature softmax of a row */
static double prob(const void *row, int dtype, int64_t x, row_stats st, double T) {
    return exp((elem(row, dtype, x) - st.m) / T) / st.s;
}

/* ---- inverse-CDF draw over ascending x --------------------------------- */
/* mass(x) >= 0 for every x; R is its sequential sum.  Returns the first x with
 * C(x) > tau = u * R and the distance of tau to the chosen interval's nearer
 * edge, in units of R.  If no such x exists (only possible for u >= 1), the last
 * x with positive mass is returned with margin 0. */
typedef double (*mass_fn)(int64_t x, const void *ctx);

static int32_t inverse_cdf(mass_fn mass, const void *ctx, int V, double R, double u, double *margin) {
    double tau = u * R, C = 0.0;
    int32_t last_pos = -1;
    for (int x = 0; x < V; ++x) {
        double w = mass(x, ctx);
        if (w > 0.0) last_pos = x;
        double Cprev = C;
        C += w;
        if (C > tau) {
            double lo = tau - Cprev, hi = C - tau;
            *margin = (lo < hi ? lo : hi) / R;
            return x;
        }
    }
    *margin = 0.0;
    return last_pos;
}

typedef struct {
    const void *t, *d; int dtype; double T; row_stats st, sd; int use_p_only;
} residual_ctx;

/* r(x) = max(0, p(x) - q(x)); with use_p_only the fallback mass p(x) */
static double residual_mass(int64_t x, const void *vctx) {
    const residual_ctx *c = (const residual_ctx *)vctx;
    double p = prob(c->t, c->dtype, x, c->st, c->T);
    if (c->use_p_only) return p;
    double q = prob(c->d, c->dtype, x, c->sd, c->T);
    return p > q ? p - q : 0.0;
}

typedef struct { const void *t; int dtype; double T; double m; } bonus_ctx;

/* unnormalised target mass exp((t_x - m)/T); its total is the row's s */
static double bonus_mass(int64_t x, const void *vctx) {
    const bonus_ctx *c = (const bonus_ctx *)vctx;
    return exp((elem(c->t, c->dtype, x) - c->m) / c->T);
}

/* ---- top-32 by sorting every (value, index) pair ----------------------- */
typedef struct { double v; int32_t x; } vi_pair;

static int by_value_desc_index_asc(const void *a, const void *b) {
    const vi_pair *p = (const vi_pair *)a, *q = (const vi_pair *)b;
    if (p->v > q->v) return -1;
    if (p->v < q->v) return 1;
    return (p->x > q->x) - (p->x < q->x);
}

static void top32(const void *row, int dtype, int V, float *val, int32_t *idx, vi_pair *scratch) {
    int has_nan = 0;
    for (int x = 0; x < V; ++x) {
        scratch[x].v = elem(row, dtype, x);
        scratch[x].x = x;
        if (isnan(scratch[x].v)) has_nan = 1;
    }
    if (has_nan) {     /* no order exists: the whole slot is (NaN, -1) */
        for (int r = 0; r < ORC_TOPK; ++r) { val[r] = NAN; idx[r] = -1; }
        return;
    }
    qsort(scratch, (size_t)V, sizeof(vi_pair), by_value_desc_index_asc);
    for (int r = 0; r < ORC_TOPK; ++r) {
        if (r < V) { val[r] = (float)scratch[r].v; idx[r] = scratch[r].x; }
        else { val[r] = -INFINITY; idx[r] = -1; }
    }
}

/* lowest index among the maximal values (numpy argmax) */
static int32_t argmax_row(const void *row, int dtype, int V) {
    int32_t best = 0;
    double bv = elem(row, dtype, 0);
    for (int x = 1; x < V; ++x) {
        double v = elem(row, dtype, x);
        if (v > bv) { bv = v; best = x; }
    }
    return best;
}

static int row_has_nan(const void *row, int dtype, int V) {
    for (int x = 0; x < V; ++x) if (isnan(elem(row, dtype, x))) return 1;
    return 0;
}

/*
 * orc_verify: all arrays are host arrays, contiguous, row-major.
 *   target  [B, k+1, V]   fp32 or bf16 bit patterns
 *   draft   [B, k, V]     same dtype; unused (may be NULL) when temperature == 0
 *   tokens  [B, k]        drafted tokens
 *   uniforms[B, k+2]      unused (may be NULL) when temperature == 0
 * outputs:
 *   accepted_len[B], out_tokens[B, k+1], topk_val/topk_idx[B, k+1, 32], status[B]
 *   optional (NULL = skip): lse_target[B, k+1], lse_draft[B, k], p_tok[B, k] and
 *   q_tok[B, k] (every drafted position, whether or not the chain reached it),
 *   margin_accept[B, k] (NaN where no test ran), margin_cdf[B] (NaN where no
 *   draw ran).
 * Returns 0, or -1 for bad arguments.
 */
int orc_verify(int B, int k, int V, int dtype, float temperature,
               const void *target, const void *draft, const int32_t *tokens, const float *uniforms,
               int32_t *accepted_len, int32_t *out_tokens, float *topk_val, int32_t *topk_idx,
               int32_t *status, double *lse_target, double *lse_draft, double *p_tok, double *q_tok,
               double *margin_accept, double *margin_cdf) {
    if (B < 0 || k < 0 || V < 1 || (dtype != ORC_F32 && dtype != ORC_BF16)) return -1;
    if (!(temperature >= 0.0f) || isinf(temperature)) return -1;
    const double T = (double)temperature;
    const int greedy = (temperature == 0.0f);
    const size_t e = dtype == ORC_F32 ? 4 : 2;
    const int K1 = k + 1;
    vi_pair *scratch = (vi_pair *)malloc(sizeof(vi_pair) * (size_t)V);
    row_stats *st = (row_stats *)malloc(sizeof(row_stats) * (size_t)(2 * K1));
    if (!scratch || !st) { free(scratch); free(st); return -1; }

    for (int b = 0; b < B; ++b) {
        const char *tb = (const char *)target + (size_t)b * K1 * V * e;
        const char *db = greedy ? NULL : (const char *)draft + (size_t)b * k * V * e;
        const int32_t *xb = tokens + (size_t)b * k;
        const float *ub = greedy ? NULL : uniforms + (size_t)b * (K1 + 1);
        int32_t flags = 0;

        /* soft targets: top-32 of every target row, both modes */
        for (int i = 0; i < K1; ++i)
            top32(tb + (size_t)i * V * e, dtype, V,
                  topk_val + ((size_t)b * K1 + i) * ORC_TOPK, topk_idx + ((size_t)b * K1 + i) * ORC_TOPK,
                  scratch);
        if (margin_accept) for (int i = 0; i < k; ++i) margin_accept[(size_t)b * k + i] = NAN;
        if (margin_cdf) margin_cdf[b] = NAN;
        for (int i = 0; i < k; ++i) if (xb[i] < 0 || xb[i] >= V) flags |= ORC_BAD_TOKEN;

        int32_t j = k, chosen = -1;
        if (greedy) {
            for (int i = 0; i < K1; ++i) if (row_has_nan(tb + (size_t)i * V * e, dtype, V)) flags |= ORC_NAN;
            if (!flags) {
                /* T -> 0: accept while the drafted token is the target argmax */
                for (int i = 0; i < k; ++i)
                    if (xb[i] != argmax_row(tb + (size_t)i * V * e, dtype, V)) { j = i; break; }
                chosen = argmax_row(tb + (size_t)j * V * e, dtype, V);
            }
        } else {
            for (int i = 0; i < K1 + 1; ++i)
                if (!(ub[i] >= 0.0f && ub[i] < 1.0f)) flags |= ORC_BAD_UNIFORM;
            for (int i = 0; i < K1; ++i) st[i] = stats_of(tb + (size_t)i * V * e, dtype, V, T);
            for (int i = 0; i < k; ++i) st[K1 + i] = stats_of(db + (size_t)i * V * e, dtype, V, T);
            for (int r = 0; r < K1 + k; ++r) {
                if (st[r].has_nan) flags |= ORC_NAN;
                else if (st[r].has_posinf) flags |= ORC_POSINF;
                else if (st[r].m == -INFINITY) flags |= ORC_EMPTY_ROW;
            }
            for (int i = 0; i < K1; ++i)
                if (lse_target) lse_target[(size_t)b * K1 + i] = st[i].m / T + log(st[i].s);
            for (int i = 0; i < k; ++i)
                if (lse_draft) lse_draft[(size_t)b * k + i] = st[K1 + i].m / T + log(st[K1 + i].s);
            if (!flags) {
                /* p_i(x_i) and q_i(x_i) of every drafted position */
                for (int i = 0; i < k; ++i) {
                    if (p_tok) p_tok[(size_t)b * k + i] = prob(tb + (size_t)i * V * e, dtype, xb[i], st[i], T);
                    if (q_tok) q_tok[(size_t)b * k + i] = prob(db + (size_t)i * V * e, dtype, xb[i], st[K1 + i], T);
                }
                /* acceptance chain: token i survives iff u_i < min(1, p/q) */
                for (int i = 0; i < k; ++i) {
                    const void *ti = tb + (size_t)i * V * e, *di = db + (size_t)i * V * e;
                    double p = prob(ti, dtype, xb[i], st[i], T);
                    double q = prob(di, dtype, xb[i], st[K1 + i], T);
                    double ratio = q > 0.0 ? p / q : (p > 0.0 ? INFINITY : 0.0);
                    double a = ratio < 1.0 ? ratio : 1.0;
                    double u = (double)ub[i];
                    if (margin_accept) margin_accept[(size_t)b * k + i] = u - a;
                    if (!(u < a)) { j = i; break; }
                }
                double margin = NAN;
                if (j < k) {
                    /* first rejection: redraw from max(0, p_j - q_j), normalised */
                    residual_ctx c = { tb + (size_t)j * V * e, db + (size_t)j * V * e, dtype, T,
                                       st[j], st[K1 + j], 0 };
                    double R = 0.0;
                    for (int x = 0; x < V; ++x) R += residual_mass(x, &c);
                    if (R == 0.0) {
                        c.use_p_only = 1;
                        for (int x = 0; x < V; ++x) R += residual_mass(x, &c);
                    }
                    chosen = inverse_cdf(residual_mass, &c, V, R, (double)ub[k], &margin);
                } else {
                    /* every draft token accepted: bonus token from p_k */
                    bonus_ctx c = { tb + (size_t)k * V * e, dtype, T, st[k].m };
                    chosen = inverse_cdf(bonus_mass, &c, V, st[k].s, (double)ub[k + 1], &margin);
                }
                if (margin_cdf) margin_cdf[b] = margin;
            }
        }
        status[b] = flags;
        if (flags) {
            accepted_len[b] = -1;
            for (int i = 0; i < K1; ++i) out_tokens[(size_t)b * K1 + i] = -1;
            continue;
        }
        accepted_len[b] = j;
        for (int i = 0; i < K1; ++i)
            out_tokens[(size_t)b * K1 + i] = i < j ? xb[i] : (i == j ? chosen : -1);
    }
    free(scratch);
    free(st);
    return 0;
}
