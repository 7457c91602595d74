/*
 * spec_verify.h -- C ABI of the speculative-sampling verification library for
 * AMD MI355X (gfx950).
 *
 * The operation (ReSpec notes, "2 . background": one-shot acceptance test Eq.1
 * of Leviathan et al. 2023 and the residual r(x) = max(0, p - q) / sum max(0, p - q);
 * ReSpec blog, speculative-decoding steps 1-4; slime/Notion post, introduction):
 * for each of B sequences with k drafted tokens x_0..x_{k-1},
 *   p_i = softmax(target_logits[b,i,:] / T)  for i = 0..k,
 *   q_i = softmax(draft_logits[b,i,:] / T)   for i = 0..k-1,
 *   draft token i is accepted while u[b,i] < min(1, p_i(x_i) / q_i(x_i));
 *   at the first rejection j the token is redrawn from the residual
 *   max(0, p_j - q_j), normalised, by inverse CDF with u[b,k];
 *   if all k drafts pass, a bonus token is drawn from p_k with u[b,k+1].
 * With T == 0 the step is greedy: draft i is accepted while it equals the
 * argmax of target row i (lowest index on ties), and the argmax of the first
 * mismatching row (or of row k) is emitted.
 * In both modes the 32 largest target logits of every verified position are
 * returned, the soft targets stored for drafter distillation (ReSpec notes,
 * "4 . G2", worked example: V = 151936, top-K = 32).
 *
 * Conventions where the pages are silent:
 *   - inverse CDF walks tokens in ascending index and takes the first x whose
 *     cumulative mass exceeds u * R (R the unnormalised total); tokens of zero
 *     mass are never drawn;
 *   - q_i(x_i) == 0 counts as ratio +inf when p_i(x_i) > 0, else 0;
 *   - a residual with no mass left (only through rounding) falls back to p_j;
 *   - top-32 order is (value descending, index ascending) under float
 *     comparison (-0.0 == +0.0); values are the raw target logits as fp32; rows
 *     with V < 32 pad with (-inf, -1); rows holding a NaN give (NaN, -1).
 *
 * Results are deterministic: vocabulary tiles have a fixed size and every
 * reduction runs in a fixed order, so a row's result does not depend on B, on
 * the other rows or on the launch size.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_TOPK 32

/* element type of the logits */
typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype_t;

/* return codes (host-detected; nothing is launched when one is returned) */
#define SV_OK 0
#define SV_ERR_NULL (-1)        /* a required pointer is NULL */
#define SV_ERR_SHAPE (-2)       /* B < 0, k < 0, V < 1, V above the maximum (524288 for bf16,
                                   262144 for fp32), a row stride < V, sizes too large, or an
                                   unknown aux->item_layout or aux->variant */
#define SV_ERR_TEMPERATURE (-3) /* temperature < 0, NaN or infinite */
#define SV_ERR_DTYPE (-4)       /* dtype not SV_F32 / SV_BF16 */
#define SV_ERR_WORKSPACE (-5)   /* workspace NULL or smaller than spec_verify_workspace_bytes */
#define SV_ERR_HIP (-6)         /* a HIP runtime call or the kernel launch failed */
#define SV_ERR_DEVICE (-7)      /* current device is not usable */
#define SV_ERR_SCRATCH (-8)     /* spec_verify_noalloc: the shape needs more workspace than
                                   SV_NOALLOC_MAX_BYTES */

/* per-sequence data-error bits written to aux->status (device side) */
#define SV_STATUS_BAD_TOKEN 1    /* a draft token is outside [0, V) */
#define SV_STATUS_NAN 2          /* a used row holds a NaN */
#define SV_STATUS_POSINF 4       /* sampling: a used row holds +inf (softmax undefined) */
#define SV_STATUS_EMPTY_ROW 8    /* sampling: a used row is all -inf (no distribution) */
#define SV_STATUS_BAD_UNIFORM 16 /* sampling: a uniform is outside [0, 1) */
#define SV_STATUS_SYNC_TIMEOUT 32 /* internal: a bounded cross-workgroup wait gave up, or the
                                     workspace was not zero-filled (never expected) */

typedef struct {
    int32_t B;                  /* sequences, >= 0 (0: nothing to do) */
    int32_t k;                  /* drafted tokens per sequence, >= 0 */
    int32_t V;                  /* vocabulary size, 1 .. 524288 (bf16) or 262144 (fp32) */
    int32_t dtype;              /* sv_dtype_t of both logits tensors */
    int64_t target_row_stride;  /* elements between target rows (b,i) and (b,i+1), and
                                   between (b,k) and (b+1,0); 0 means V */
    int64_t draft_row_stride;   /* same for draft rows; 0 means V */
    float temperature;          /* > 0: sampling; == 0: greedy */
} sv_shape_t;

/* optional outputs (device pointers; any may be NULL) */
typedef struct {
    int32_t *status;     /* [B]    SV_STATUS_* bits; 0 = valid sequence */
    float *lse_target;   /* [B,k+1] ln sum_x exp(t_x / T)   (sampling only) */
    float *lse_draft;    /* [B,k]   ln sum_x exp(d_x / T)   (sampling only) */
    float *p_tok;        /* [B,k]   p_i(x_i)                (sampling only) */
    float *q_tok;        /* [B,k]   q_i(x_i)                (sampling only) */
    int32_t item_layout; /* order in which the streaming workgroups take the (group, tile)
                            items: SV_LAYOUT_AUTO (0, the library's measured table),
                            SV_LAYOUT_LAUNCH (launch order) or SV_LAYOUT_XCD_RUNS (one
                            contiguous run of items per XCD); results are identical */
    int32_t variant;     /* build of the kernel: SV_VARIANT_AUTO (0, the library's measured
                            table), SV_VARIANT_BASE (bf16 at 6 waves per SIMD) or
                            SV_VARIANT_HIGH_OCC (bf16 at 8 waves per SIMD; fp32 has one
                            build, taken for both); results are identical */
} sv_aux_t;

#define SV_LAYOUT_AUTO 0
#define SV_LAYOUT_LAUNCH 1
#define SV_LAYOUT_XCD_RUNS 2

#define SV_VARIANT_AUTO 0
#define SV_VARIANT_BASE 1
#define SV_VARIANT_HIGH_OCC 2

/* Bytes of device workspace one call with this shape needs. */
size_t spec_verify_workspace_bytes(const sv_shape_t *shape);

/* The item layout (SV_LAYOUT_LAUNCH or SV_LAYOUT_XCD_RUNS) that SV_LAYOUT_AUTO
 * takes for this shape: SV_LAYOUT_XCD_RUNS when a row's number of 16 KB tiles
 * is divisible by 4 (launch order would crowd the merges onto one or two
 * XCDs); else the
 * faster one in a table measured on MI355X at V = 151936 over batch sizes
 * 1..256, draft lengths 0..15, both dtypes and both modes (the entry nearest
 * in log B and k).  Returns 0 for an invalid shape. */
int spec_verify_layout_choice(const sv_shape_t *shape);

/* The kernel build (SV_VARIANT_BASE or SV_VARIANT_HIGH_OCC) that
 * SV_VARIANT_AUTO takes for this shape: for bf16 logits the faster one in the
 * same measured table (the entry nearest in log B and k); a build with more
 * waves per SIMD keeps more workgroups resident, which pays at large batches
 * and costs at small ones.  SV_VARIANT_BASE for fp32.  Returns 0 for an invalid
 * shape. */
int spec_verify_variant_choice(const sv_shape_t *shape);

/*
 * Enqueue one verification step on `stream` (a hipStream_t; NULL = default
 * stream) and return without synchronising.  Outputs are valid once the
 * stream has reached this point.
 *
 * Inputs (device pointers, caller-owned, row-major, 16-byte aligned rows run
 * fastest; other alignments are accepted):
 *   target_logits [B, k+1, V] with row stride target_row_stride
 *   draft_logits  [B, k, V]   with row stride draft_row_stride; ignored and
 *                             may be NULL when temperature == 0
 *   draft_tokens  [B, k] int32
 *   uniforms      [B, k+2] fp32 in [0,1): u[0..k-1] acceptance, u[k] residual
 *                 draw, u[k+1] bonus draw; ignored and may be NULL when
 *                 temperature == 0
 * Outputs (device pointers, caller-owned):
 *   accepted_len  [B] int32, in [0, k]; -1 for a sequence with a data error
 *   out_tokens    [B, k+1] int32: drafts 0..j-1, the drawn token at j, -1 after;
 *                 all -1 for a sequence with a data error
 *   topk_val      [B, k+1, 32] fp32 and topk_idx [B, k+1, 32] int32
 *   aux           optional outputs; NULL for none
 * Workspace: device memory of at least spec_verify_workspace_bytes(shape)
 *   bytes, 256-byte aligned, zero-filled before its first use.  Every call
 *   whose sequences carry no SV_STATUS_SYNC_TIMEOUT leaves it zero-filled
 *   again for the next one.  A call that reports SV_STATUS_SYNC_TIMEOUT may
 *   leave counters and records behind, and it sets a fault word in the
 *   workspace that is never cleared by the library: every later call on that
 *   workspace reports SV_STATUS_SYNC_TIMEOUT too, until the caller zero-fills
 *   the whole workspace again.  Calls that share a workspace must not overlap
 *   in time.
 * Errors: host-detectable argument errors return a negative SV_ERR_* code
 *   before anything is enqueued.  Data errors (bad token, NaN, +inf, all -inf
 *   row, bad uniform) cannot be seen without a device sync; they set the
 *   SV_STATUS_* bits of that sequence and make its accepted_len and
 *   out_tokens -1.
 * B = 0: returns SV_OK after the argument checks and enqueues nothing.
 * Execution: one kernel launch.  Its streaming workgroups read every logit
 *   once (per-tile statistics and candidates, per-group merges, per-sequence
 *   assembly); in sampling mode draw workgroups follow (residual or bonus
 *   draw).  A workgroup waits only for workgroups of lower index or for the
 *   other draw workgroups of its sequence, always with a time bound.
 *   Assumption behind every such wait: the GPU starts the workgroups of a
 *   launch in index order within each of its XCDs (workgroups are dealt to
 *   the XCDs round robin), so a waited-for workgroup has started or can start
 *   once earlier ones finish; nothing in HIP promises this for an ordinary
 *   launch.  Should a wait still not end, it gives up after 0.2 s, sets
 *   SV_STATUS_SYNC_TIMEOUT in the sequences assembled after it, and the
 *   kernel completes (its results are then not to be used).
 * The library allocates no memory and keeps no per-call state; it is safe to
 * call from several host threads with separate workspaces.
 */
int spec_verify(const sv_shape_t *shape,
                const void *target_logits, const void *draft_logits,
                const int32_t *draft_tokens, const float *uniforms,
                int32_t *accepted_len, int32_t *out_tokens,
                float *topk_val, int32_t *topk_idx,
                const sv_aux_t *aux,
                void *workspace, size_t workspace_bytes, void *stream);

/* Size of the static scratch array behind spec_verify_noalloc, per GPU. */
#define SV_NOALLOC_MAX_BYTES (8u << 20)

/*
 * spec_verify without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same inputs, outputs, results, errors and stream
 * semantics as spec_verify; it calls no hipMalloc, hipFree or other allocating
 * routine.  Its workspace is a static device array of SV_NOALLOC_MAX_BYTES
 * (8 MiB) inside the library: each GPU the library runs on holds its own copy
 * until the process ends, and the first call on a device looks up that copy's
 * address.  Every call enqueues a small fill kernel that zeroes the part of the
 * array its shape uses, then the verification kernel, both on `stream`.
 * Limit: shapes whose spec_verify_workspace_bytes exceeds SV_NOALLOC_MAX_BYTES
 * return SV_ERR_SCRATCH before anything is enqueued (every workload of up to
 * B = 32, k = 15, V = 151936 fits; so does B = 256, k = 3, V = 128256).
 * All calls on one GPU share the one array: calls that overlap in time on the
 * same GPU (other streams, other host threads) race and must not be made.
 */
int spec_verify_noalloc(const sv_shape_t *shape,
                        const void *target_logits, const void *draft_logits,
                        const int32_t *draft_tokens, const float *uniforms,
                        int32_t *accepted_len, int32_t *out_tokens,
                        float *topk_val, int32_t *topk_idx,
                        const sv_aux_t *aux, void *stream);

/* Static description of a return code. */
const char *spec_verify_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
