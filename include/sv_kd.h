/*
 * sv_kd.h -- C ABI of the reward-weighted drafter distillation step over the
 * stored top-32 soft targets, for AMD MI355X (gfx950).  Same library as
 * spec_verify.h (libspec_verify.so).
 *
 * The operation (ReSpec notes, "4 . G2": the verification's target logits are
 * kept as the soft target of an on-policy KD of the drafter, only the top-32
 * per position being stored, and the loss is KL(softmax(log p) || q_theta);
 * "5 . G3": each sample's KD loss is weighted by w(r), by default the reward,
 * normalised and clipped in practice; worked examples there: one sample,
 * loss = 0.85 * (0.32 + 0.18 + 0); a GRPO group with rewards
 * [1.0, 0.8, 0.3, 0.3, 0.0] weighted about 0.42 and 0.33 for the first two):
 * for each row n (one stored position) with drafter logits z_n[0..V-1], stored
 * target logits v_n[0..31] at token ids x_n[0..31], and sample s = row_sample[n],
 *   pt_n(j)  = exp(v_n[j]) / sum_j' exp(v_n[j'])        (softmax over the stored 32)
 *   q_n(x)   = exp(z_n[x] - lse_n),  lse_n = ln sum_x exp(z_n[x])
 *   KL_n     = sum_j pt_n(j) * (ln pt_n(j) - ln q_n(x_n[j]))
 *   w_s      = clip(r_s / sum_{s' in group(s)} r_s', 0, w_max)   (0 when the sum is 0)
 *   loss     = sum_n w_{s(n)} * KL_n  (rows with w = 0 contribute 0)
 *   grad_n(x) = d loss / d z_n[x] = w_{s(n)} * (q_n(x) - pt_n(x)),  pt_n(x) = pt_n(j)
 *               where x = x_n[j], else 0
 * Groups are runs of `group` consecutive samples.  Readings where the pages are
 * silent: both distributions at temperature 1 (raw logits); the sum over
 * positions is not averaged; the clip bound w_max is the caller's (+inf: none).
 *
 * Results are deterministic: vocabulary tiles have a fixed size and every
 * reduction runs in a fixed order.
 */
#ifndef SV_KD_H
#define SV_KD_H

#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

/* per-row data-error bits written to `status` (device side) */
#define SV_KD_BAD_INDEX 1   /* a stored entry with a finite value has an id outside [0, V) */
#define SV_KD_NAN 2         /* the drafter row or a stored value holds a NaN */
#define SV_KD_POSINF 4      /* the drafter row or a stored value holds +inf */
#define SV_KD_EMPTY 8       /* the drafter row is all -inf, or no stored entry is finite */
#define SV_KD_DUP_INDEX 16  /* two non-padding stored entries of the row name the same id */
#define SV_KD_SYNC_TIMEOUT 32 /* internal: a bounded wait gave up or the workspace was not
                                 zero-filled (never expected) */

typedef struct {
    int32_t N;            /* rows (stored positions), >= 0 (0: nothing to do) */
    int32_t V;            /* vocabulary size, 1 .. 524288 (bf16) or 262144 (fp32) */
    int32_t dtype;        /* sv_dtype_t of the drafter logits */
    int32_t grad_dtype;   /* sv_dtype_t of the gradient output */
    int64_t row_stride;   /* elements between drafter rows; 0 means V */
    int32_t S;            /* samples, >= 1 when N > 0 */
    int32_t group;        /* samples per reward group, >= 1, dividing S */
    float w_max;          /* clip of the normalised weight, > 0 (+inf: no clip) */
} sv_kd_shape_t;

/* Bytes of device workspace one call with this shape needs. */
size_t sv_kd_workspace_bytes(const sv_kd_shape_t *shape);

/*
 * Enqueue one distillation loss (and, if grad is not NULL, its gradient with
 * respect to the drafter logits) on `stream` (a hipStream_t; NULL = default
 * stream) and return without synchronising.
 *
 * Inputs (device pointers, caller-owned):
 *   draft_logits [N, V] (dtype) with row stride row_stride; 16-byte aligned rows
 *                run fastest
 *   topk_val     [N, 32] fp32 stored target logits; an entry with value -inf
 *                or id -1 is padding (weight 0)
 *   topk_idx     [N, 32] int32 token ids, distinct within a row (a top-32 lists each
 *                token once); a row naming one id in two non-padding entries is
 *                a data error (SV_KD_DUP_INDEX)
 *   row_sample   [N] int32 sample of each row, in [0, S)
 *   rewards      [S] fp32
 * Outputs (device pointers, caller-owned):
 *   kl      [N] fp32 KL_n; NaN for a row with a data error
 *   weight  [N] fp32 w of the row's sample, or NULL
 *   status  [N] int32 SV_KD_* bits, or NULL
 *   loss    [1] fp64 sum of w * KL over the rows without a data error
 *   grad    [N, V] (grad_dtype, row stride V) or NULL; zero rows for rows with
 *           a data error
 * Workspace: at least sv_kd_workspace_bytes(shape) bytes, 256-byte aligned,
 *   zero-filled before its first use; every call without SV_KD_SYNC_TIMEOUT
 *   leaves it zero-filled again.  After SV_KD_SYNC_TIMEOUT it may hold
 *   leftovers and a fault word the library never clears (every later call
 *   reports SV_KD_SYNC_TIMEOUT) until the caller zero-fills it again.  Calls
 *   that share a workspace must not overlap in time.
 * Errors: argument errors return a negative SV_ERR_* code before anything is
 *   enqueued.  Data errors set the row's status bits (a row_sample outside
 *   [0, S) counts as SV_KD_BAD_INDEX).
 * N = 0: returns SV_OK, enqueues nothing and leaves every output, loss
 *   included, untouched (the caller sets loss = 0 for an empty batch).
 * Execution: one kernel launch, one workgroup per (row, 16 KB tile).  The
 *   workgroups of a row exchange their tile statistics and wait for one
 *   another.  Assumption: the GPU starts a launch's workgroups in index order
 *   within each XCD, so a row's workgroups, which are consecutive, run
 *   together (nT <= 64 of them); HIP does not promise this for an ordinary
 *   launch.  Each wait gives up after 0.2 s and sets SV_KD_SYNC_TIMEOUT.
 */
int sv_kd(const sv_kd_shape_t *shape, const void *draft_logits, const float *topk_val,
          const int32_t *topk_idx, const int32_t *row_sample, const float *rewards,
          float *kl, float *weight, int32_t *status, double *loss, void *grad,
          void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SV_KD_H */
