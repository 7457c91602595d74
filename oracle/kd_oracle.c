/*
 * kd_oracle.c -- plain, slow, single-threaded CPU oracle for the reward-weighted
 * distillation of the drafter over the stored top-32 soft targets.  TEST
 * INFRASTRUCTURE ONLY: built, loaded and called by the tests, the smoke check
 * and the benchmark's CPU-baseline leg, never by the product path.  It shares
 * no code, header or table with the HIP library.
 *
 * What it computes (ReSpec notes, "4 . G2": the verification keeps the target
 * logits, top-32 per position, as the soft target of an on-policy KD of the
 * drafter, loss KL(softmax(log p) || q_theta), gradient through q_theta only;
 * "5 . G3": the per-sample KD loss is multiplied by w(r), the reward by
 * default, normalised and clipped in practice; its GRPO example normalises the
 * rewards of one group by their sum), row by row:
 *   pt(j)   = exp(v_j - max v) / sum_j' exp(v_j' - max v)   over the used stored entries
 *   lse     = max z + ln sum_x exp(z_x - max z)              over the whole drafter row
 *   KL      = sum_j pt(j) * (ln pt(j) - (z_{x_j} - lse))      (terms with pt(j) = 0 are 0)
 *   w       = clip(r_s / sum of the rewards of s's group, 0, w_max), 0 if that sum <= 0
 *   loss    = sum over rows without a data error and with w > 0 of w * KL
 *   grad(x) = w * (exp(z_x - lse) - pt(x)), pt(x) = pt(j) where x = x_j, else 0
 *
 * Readings where the pages are silent (listed in the design notes): both
 * distributions at temperature 1; positions are summed, not averaged; a stored
 * entry with value -inf or id -1 is padding; the clip bound is the caller's;
 * the stored ids of a row are distinct (a top-32 lists each token once), so a
 * row where two non-padding entries name the same id is a data error
 * (KD_DUP_INDEX): such a row is no distribution over tokens.
 *
 * Everything is fp64; every sum runs sequentially in ascending order.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define KD_F32 0
#define KD_BF16 1
#define KD_TOP 32

#define KD_BAD_INDEX 1
#define KD_NAN 2
#define KD_POSINF 4
#define KD_EMPTY 8
#define KD_DUP_INDEX 16

static double kd_elem(const void *row, int dtype, int64_t x) {
    if (dtype == KD_F32) return (double)((const float *)row)[x];
    uint32_t bits = (uint32_t)((const uint16_t *)row)[x] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* the weight of sample s: its reward over its group's sum, clipped */
static double kd_weight(const float *rewards, int S, int group, double w_max, int s) {
    if (s < 0 || s >= S) return 0.0;
    const int g0 = (s / group) * group;
    double sum = 0.0;
    for (int t = g0; t < g0 + group; ++t) sum += (double)rewards[t];
    double w = sum > 0.0 ? (double)rewards[s] / sum : 0.0;
    if (!(w > 0.0)) w = 0.0;
    if (w > w_max) w = w_max;
    return w;
}

/*
 * N rows of V drafter logits (dtype, row stride `stride` elements), stored
 * values [N,32] and ids [N,32], row_sample [N], rewards [S].  Outputs kl [N]
 * (NaN for a row with a data error), weight [N], status [N], loss [1], and,
 * when grad is not NULL, grad [N,V] in fp64.
 */
int kd_oracle(int N, int V, int dtype, int64_t stride, int S, int group, double w_max,
              const void *logits, const float *tval, const int32_t *tidx, const int32_t *row_sample,
              const float *rewards, double *kl, double *weight, int32_t *status, double *loss, double *grad) {
    const int esz = dtype == KD_BF16 ? 2 : 4;
    double total = 0.0;
    for (int n = 0; n < N; ++n) {
        const char *row = (const char *)logits + (int64_t)n * stride * esz;
        const float *v = tval + (int64_t)n * KD_TOP;
        const int32_t *x = tidx + (int64_t)n * KD_TOP;
        int st = 0;

        /* the drafter row's log-normaliser */
        double mz = -INFINITY;
        int nan = 0, pinf = 0;
        for (int64_t i = 0; i < V; ++i) {
            const double z = kd_elem(row, dtype, i);
            if (z != z) nan = 1;
            else if (z == INFINITY) pinf = 1;
            else if (z > mz) mz = z;
        }
        double sz = 0.0;
        for (int64_t i = 0; i < V; ++i) sz += exp(kd_elem(row, dtype, i) - mz);
        const double lse = mz + log(sz);
        if (nan) st |= KD_NAN;
        else if (pinf) st |= KD_POSINF;
        else if (mz == -INFINITY) st |= KD_EMPTY;

        /* the stored entries and the sample id: their own error bits, which
           entries are used, and the softmax over them */
        int est = 0;
        int used[KD_TOP];
        double mv = -INFINITY;
        for (int j = 0; j < KD_TOP; ++j) {
            const int pad = v[j] == -INFINITY || x[j] == -1;
            if (v[j] != v[j]) est |= KD_NAN;
            else if (v[j] == INFINITY) est |= KD_POSINF;
            if (!pad && (x[j] < 0 || x[j] >= V)) est |= KD_BAD_INDEX;
        }
        for (int j = 0; j < KD_TOP; ++j) {
            if (v[j] == -INFINITY || x[j] == -1 || x[j] < 0 || x[j] >= V) continue;
            for (int i = 0; i < j; ++i)
                if (!(v[i] == -INFINITY || x[i] == -1) && x[i] == x[j]) est |= KD_DUP_INDEX;
        }
        const int s = row_sample[n];
        if (s < 0 || s >= S) est |= KD_BAD_INDEX;
        for (int j = 0; j < KD_TOP; ++j) {
            used[j] = !est && !(v[j] == -INFINITY || x[j] == -1);
            if (used[j] && (double)v[j] > mv) mv = (double)v[j];
        }
        if (!est && mv == -INFINITY) est |= KD_EMPTY;
        st |= est;
        double sv = 0.0;
        for (int j = 0; j < KD_TOP; ++j)
            if (used[j]) sv += exp((double)v[j] - mv);

        const double w = kd_weight(rewards, S, group, w_max, s);
        double d = 0.0;
        for (int j = 0; j < KD_TOP && !st; ++j) {
            if (!used[j]) continue;
            const double pt = exp((double)v[j] - mv) / sv;
            if (pt == 0.0) continue;
            const double lpt = ((double)v[j] - mv) - log(sv);
            const double lq = kd_elem(row, dtype, x[j]) - lse;
            d += pt * (lpt - lq);
        }
        kl[n] = st ? NAN : d;
        weight[n] = w;
        status[n] = st;
        if (!st && w > 0.0) total += w * d;

        if (grad) {
            double *g = grad + (int64_t)n * V;
            for (int64_t i = 0; i < V; ++i) g[i] = st ? 0.0 : w * exp(kd_elem(row, dtype, i) - lse);
            if (!st)
                for (int j = 0; j < KD_TOP; ++j)
                    if (used[j]) g[x[j]] = w * (exp(kd_elem(row, dtype, x[j]) - lse) - exp((double)v[j] - mv) / sv);
        }
    }
    *loss = total;
    return 0;
}
