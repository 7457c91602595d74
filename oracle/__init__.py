"""ctypes wrapper of the plain-C fp64 oracles: sv_oracle.c (verification) and
kd_oracle.c (reward-weighted drafter distillation over the stored top-32).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP
library and never calls it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sv_oracle.c")
_SRCS = [_SRC, os.path.join(_HERE, "kd_oracle.c")]
_LIB = os.path.join(_HERE, "libsv_oracle.so")

STATUS_BAD_TOKEN, STATUS_NAN, STATUS_POSINF, STATUS_EMPTY_ROW, STATUS_BAD_UNIFORM = 1, 2, 4, 8, 16
TOPK = 32


CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(srcs=None, out=None, extra=()) -> str:
    """Compile the oracle with gcc (plain C99, no fast-math, no FMA contraction).
    srcs/out: other sources and library path (the tests build altered copies to
    check that the pins catch them); extra: more gcc flags (sanitizers)."""
    srcs = list(srcs or _SRCS)
    out = out or _LIB
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", *CFLAGS, *extra, "-o", tmp, *srcs, "-lm"])
    os.replace(tmp, out)
    return out


_lib = None


def bind(path) -> ctypes.CDLL:
    """Load an oracle library and declare its two entry points."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.orc_verify.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                               P, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.orc_verify.restype = ctypes.c_int
    lib.kd_oracle.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                              ctypes.c_double, P, P, P, P, P, P, P, P, P, P]
    lib.kd_oracle.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(os.path.getmtime(f) for f in _SRCS):
            build()
        _lib = bind(_LIB)
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class OracleResult(dict):
    __getattr__ = dict.__getitem__


def verify(target, draft, draft_tokens, uniforms, temperature, dtype, aux=True) -> OracleResult:
    """Run the oracle.  target [B,k+1,V] and draft [B,k,V] are float32 arrays, or
    uint16 bf16 bit patterns with dtype=1; draft_tokens [B,k] int32; uniforms
    [B,k+2] float32.  Returns a dict of numpy arrays."""
    lib = _load()
    target = np.ascontiguousarray(target)
    B, K1, V = target.shape
    k = K1 - 1
    greedy = float(temperature) == 0.0
    want = np.float32 if dtype == 0 else np.uint16
    assert target.dtype == want
    draft = None if (greedy and draft is None) else np.ascontiguousarray(draft, dtype=want)
    if draft is not None:
        assert draft.shape == (B, k, V)
    tokens = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, k)
    u = None if (greedy and uniforms is None) else np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, K1 + 1)
    r = OracleResult(
        accepted_len=np.empty(B, np.int32), out_tokens=np.empty((B, K1), np.int32),
        topk_val=np.empty((B, K1, TOPK), np.float32), topk_idx=np.empty((B, K1, TOPK), np.int32),
        status=np.empty(B, np.int32))
    if aux:
        r.update(lse_target=np.full((B, K1), np.nan), lse_draft=np.full((B, k), np.nan),
                 p_tok=np.full((B, k), np.nan), q_tok=np.full((B, k), np.nan),
                 margin_accept=np.full((B, k), np.nan), margin_cdf=np.full(B, np.nan))
    g = r.get
    rc = lib.orc_verify(B, k, V, int(dtype), float(temperature), _ptr(target), _ptr(draft), _ptr(tokens), _ptr(u),
                        _ptr(r["accepted_len"]), _ptr(r["out_tokens"]), _ptr(r["topk_val"]), _ptr(r["topk_idx"]),
                        _ptr(r["status"]), _ptr(g("lse_target")), _ptr(g("lse_draft")), _ptr(g("p_tok")),
                        _ptr(g("q_tok")), _ptr(g("margin_accept")), _ptr(g("margin_cdf")))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return r


def verify_workload(w, aux=True) -> OracleResult:
    """Oracle on an sv_inputs.Workload."""
    return verify(w.target, None if w.temperature == 0 else w.draft, w.draft_tokens,
                  None if w.temperature == 0 else w.uniforms, w.temperature, w.dtype, aux=aux)


KD_BAD_INDEX, KD_NAN, KD_POSINF, KD_EMPTY, KD_DUP_INDEX = 1, 2, 4, 8, 16


def kd(logits, topk_val, topk_idx, row_sample, rewards, group, w_max=float("inf"), dtype=0, grad=True) -> OracleResult:
    """Reward-weighted distillation oracle.  logits [N,V] float32, or uint16 bf16
    bit patterns with dtype=1; topk_val [N,32] float32; topk_idx [N,32] int32;
    row_sample [N] int32; rewards [S] float32.  Returns kl, weight, status
    [N], loss (float) and, with grad, grad [N,V] (fp64)."""
    lib = _load()
    want = np.float32 if dtype == 0 else np.uint16
    z = np.ascontiguousarray(logits)
    assert z.dtype == want and z.ndim == 2
    N, V = z.shape
    tv = np.ascontiguousarray(topk_val, dtype=np.float32).reshape(N, TOPK)
    ti = np.ascontiguousarray(topk_idx, dtype=np.int32).reshape(N, TOPK)
    rs = np.ascontiguousarray(row_sample, dtype=np.int32).reshape(N)
    rw = np.ascontiguousarray(rewards, dtype=np.float32).reshape(-1)
    r = OracleResult(kl=np.empty(N), weight=np.empty(N), status=np.empty(N, np.int32),
                     grad=np.empty((N, V)) if grad else None)
    loss = np.zeros(1)
    rc = lib.kd_oracle(N, V, int(dtype), V, rw.size, int(group), float(w_max), _ptr(z), _ptr(tv), _ptr(ti), _ptr(rs),
                       _ptr(rw), _ptr(r["kl"]), _ptr(r["weight"]), _ptr(r["status"]), _ptr(loss), _ptr(r["grad"]))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    r["loss"] = float(loss[0])
    return r


def kd_workload(w, grad=True, rows=None) -> OracleResult:
    """KD oracle on an sv_inputs.KDWorkload (optionally on a subset of its rows;
    each row's weight still comes from its own sample's group)."""
    z = w.logits if rows is None else w.logits[rows]
    tv = w.topk_val if rows is None else w.topk_val[rows]
    ti = w.topk_idx if rows is None else w.topk_idx[rows]
    rs = w.row_sample if rows is None else w.row_sample[rows]
    return kd(z, tv, ti, rs, w.rewards, w.group, w.w_max, w.dtype, grad=grad)
