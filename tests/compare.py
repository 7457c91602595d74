"""Element-by-element comparison of the HIP path with the oracle.

accepted_len, out_tokens and top-32 indices must match exactly.  The only
allowed differences are sequences whose first difference sits at a decision the
oracle flags as within 1e-5 of its boundary: |u - min(1, p/q)| < 1e-5 for an
acceptance decision, or the drawn token's cumulative-mass interval within 1e-5
(normalised) of tau.  Their differing positions count as exceptions, which must
stay under 0.1% of all positions B(k+1).
"""
import numpy as np

FLAG = 1e-5


def gpu_to_numpy(res):
    return {k: (None if v is None else v.detach().cpu().numpy()) for k, v in res._asdict().items()}


def compare_decisions(orc, gpu, k, flag=FLAG):
    B = len(orc["accepted_len"])
    fails, exc_seq, exc_pos = [], 0, 0
    for b in range(B):
        if int(orc["status"][b]) != int(gpu["status"][b]):
            fails.append((b, "status", int(orc["status"][b]), int(gpu["status"][b])))
            continue
        ol, gl = int(orc["accepted_len"][b]), int(gpu["accepted_len"][b])
        ot, gt = orc["out_tokens"][b], gpu["out_tokens"][b]
        if ol == gl and np.array_equal(ot, gt):
            continue
        if ol != gl:
            i = min(ol, gl)
            m = orc["margin_accept"][b, i] if i < k else np.nan
            flagged = bool(np.isfinite(m) and abs(m) < flag)
            where = ("accept", i, float(m))
        else:
            flagged = bool(abs(orc["margin_cdf"][b]) < flag)
            where = ("draw", ol, float(orc["margin_cdf"][b]))
        if flagged:
            exc_seq += 1
            exc_pos += int(np.sum(ot != gt))
        else:
            fails.append((b, *where, ot.tolist(), gt.tolist()))
    return dict(fails=fails, exc_seq=exc_seq, exc_pos=exc_pos, positions=B * (k + 1))


def compare_topk(orc, gpu):
    """Exact top-32: indices equal; values equal bit for bit (NaN rows: NaN)."""
    oi, gi = orc["topk_idx"], gpu["topk_idx"]
    bad_idx = np.argwhere(oi != gi)
    ov, gv = orc["topk_val"], gpu["topk_val"]
    nan_ok = np.array_equal(np.isnan(ov), np.isnan(gv))
    fin = ~np.isnan(ov)
    val_ok = np.array_equal(ov[fin].view(np.uint32), gv[fin].view(np.uint32))
    return bad_idx, nan_ok and val_ok


def rel_err(a, b):
    """Largest relative difference of b from a.  An entry that is not finite on
    one side must be the same non-finite value on the other (NaN with NaN, an
    infinity with the same infinity); any other pairing is an infinite error."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    fa, fb = np.isfinite(a), np.isfinite(b)
    if not np.array_equal(fa, fb):
        return float("inf")
    nf = ~fa
    if not (np.array_equal(np.isnan(a[nf]), np.isnan(b[nf])) and
            np.array_equal(a[nf][~np.isnan(a[nf])], b[nf][~np.isnan(b[nf])])):
        return float("inf")
    if not fa.any():
        return 0.0
    return float(np.max(np.abs(a[fa] - b[fa]) / np.maximum(np.abs(a[fa]), 1e-300)))
