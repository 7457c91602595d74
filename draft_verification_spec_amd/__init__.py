"""Python binding of the library's C ABI: spec_verify (include/spec_verify.h)
and sv_kd (include/sv_kd.h).

Argument marshalling only: every step of the verification runs in the HIP
library libspec_verify.so built next to this file.  PyTorch supplies device
memory and the stream.  Importing works without a GPU; calling spec_verify or
verify needs the built library and an MI355X, and raises if either is missing.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import re
from collections import namedtuple
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspec_verify.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "spec_verify.h")
HEADER_PATHS = [HEADER_PATH, os.path.join(os.path.dirname(_HERE), "include", "sv_kd.h")]

SV_F32, SV_BF16 = 0, 1
TOPK = 32
SV_OK = 0
SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_TEMPERATURE, SV_ERR_DTYPE = -1, -2, -3, -4
SV_ERR_WORKSPACE, SV_ERR_HIP, SV_ERR_DEVICE, SV_ERR_SCRATCH = -5, -6, -7, -8
SV_NOALLOC_MAX_BYTES = 8 << 20
STATUS_BAD_TOKEN, STATUS_NAN, STATUS_POSINF, STATUS_EMPTY_ROW = 1, 2, 4, 8
STATUS_BAD_UNIFORM, STATUS_SYNC_TIMEOUT = 16, 32


class sv_shape_t(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("k", ctypes.c_int32), ("V", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("target_row_stride", ctypes.c_int64), ("draft_row_stride", ctypes.c_int64),
                ("temperature", ctypes.c_float)]


class sv_aux_t(ctypes.Structure):
    _fields_ = [("status", ctypes.c_void_p), ("lse_target", ctypes.c_void_p), ("lse_draft", ctypes.c_void_p),
                ("p_tok", ctypes.c_void_p), ("q_tok", ctypes.c_void_p), ("item_layout", ctypes.c_int32),
                ("variant", ctypes.c_int32)]


SV_LAYOUT_AUTO, SV_LAYOUT_LAUNCH, SV_LAYOUT_XCD_RUNS = 0, 1, 2
SV_VARIANT_AUTO, SV_VARIANT_BASE, SV_VARIANT_HIGH_OCC = 0, 1, 2


class sv_kd_shape_t(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("V", ctypes.c_int32), ("dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32),
                ("row_stride", ctypes.c_int64), ("S", ctypes.c_int32), ("group", ctypes.c_int32),
                ("w_max", ctypes.c_float)]


KD_BAD_INDEX, KD_NAN, KD_POSINF, KD_EMPTY, KD_DUP_INDEX, KD_SYNC_TIMEOUT = 1, 2, 4, 8, 16, 32


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"spec_verify failed with {code}: {spec_verify_error_string(code)}")
        self.code = code


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libspec_verify.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python __graft_entry__.py build)")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        lib.spec_verify_workspace_bytes.argtypes = [ctypes.POINTER(sv_shape_t)]
        lib.spec_verify_workspace_bytes.restype = ctypes.c_size_t
        lib.spec_verify_layout_choice.argtypes = [ctypes.POINTER(sv_shape_t)]
        lib.spec_verify_layout_choice.restype = ctypes.c_int
        lib.spec_verify_variant_choice.argtypes = [ctypes.POINTER(sv_shape_t)]
        lib.spec_verify_variant_choice.restype = ctypes.c_int
        lib.spec_verify_error_string.argtypes = [ctypes.c_int]
        lib.spec_verify_error_string.restype = ctypes.c_char_p
        lib.spec_verify.argtypes = [ctypes.POINTER(sv_shape_t), P, P, P, P, P, P, P, P,
                                    ctypes.POINTER(sv_aux_t), P, ctypes.c_size_t, P]
        lib.spec_verify.restype = ctypes.c_int
        lib.spec_verify_noalloc.argtypes = [ctypes.POINTER(sv_shape_t), P, P, P, P, P, P, P, P,
                                            ctypes.POINTER(sv_aux_t), P]
        lib.spec_verify_noalloc.restype = ctypes.c_int
        lib.sv_kd_workspace_bytes.argtypes = [ctypes.POINTER(sv_kd_shape_t)]
        lib.sv_kd_workspace_bytes.restype = ctypes.c_size_t
        lib.sv_kd.argtypes = [ctypes.POINTER(sv_kd_shape_t), P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.sv_kd.restype = ctypes.c_int
        _lib = lib
    return _lib


def declared_functions() -> list:
    """Names of the functions include/spec_verify.h and include/sv_kd.h declare."""
    names = []
    for path in HEADER_PATHS:
        text = open(path).read()
        names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*((?:spec_verify|sv_kd)\w*)\s*\(", text, flags=re.M)
    return names


def make_shape(B, k, V, dtype, temperature, target_row_stride=0, draft_row_stride=0) -> sv_shape_t:
    return sv_shape_t(int(B), int(k), int(V), int(dtype), int(target_row_stride), int(draft_row_stride),
                      float(temperature))


def spec_verify_workspace_bytes(shape: sv_shape_t) -> int:
    return int(load_library().spec_verify_workspace_bytes(ctypes.byref(shape)))


def spec_verify_layout_choice(shape: sv_shape_t) -> int:
    return int(load_library().spec_verify_layout_choice(ctypes.byref(shape)))


def spec_verify_variant_choice(shape: sv_shape_t) -> int:
    return int(load_library().spec_verify_variant_choice(ctypes.byref(shape)))


def spec_verify_error_string(code: int) -> str:
    return load_library().spec_verify_error_string(int(code)).decode()


def spec_verify(shape: Optional[sv_shape_t], target_logits, draft_logits, draft_tokens, uniforms,
                accepted_len, out_tokens, topk_val, topk_idx, aux: Optional[sv_aux_t],
                workspace, workspace_bytes, stream) -> int:
    """Direct call of the C entry point with raw device addresses (ints or None)."""
    return int(load_library().spec_verify(None if shape is None else ctypes.byref(shape),
                                          target_logits, draft_logits, draft_tokens, uniforms,
                                          accepted_len, out_tokens, topk_val, topk_idx,
                                          None if aux is None else ctypes.byref(aux),
                                          workspace, int(workspace_bytes), stream))


def spec_verify_noalloc(shape: Optional[sv_shape_t], target_logits, draft_logits, draft_tokens, uniforms,
                        accepted_len, out_tokens, topk_val, topk_idx, aux: Optional[sv_aux_t], stream) -> int:
    """Direct call of the no-allocation C entry point (the library's static
    scratch in place of a workspace) with raw device addresses (ints or None)."""
    return int(load_library().spec_verify_noalloc(None if shape is None else ctypes.byref(shape),
                                                  target_logits, draft_logits, draft_tokens, uniforms,
                                                  accepted_len, out_tokens, topk_val, topk_idx,
                                                  None if aux is None else ctypes.byref(aux), stream))


# ------------------------------------------------------------ torch front end
Result = namedtuple("Result", "accepted_len out_tokens topk_val topk_idx status lse_target lse_draft p_tok q_tok")

_workspaces = {}


def _release_workspaces():
    """At interpreter exit, before native tear-down (a profiler's or the HIP
    runtime's own exit handlers run after Python's): drop the cached
    workspaces, so that no device buffer of this module outlives them."""
    _workspaces.clear()


atexit.register(_release_workspaces)


def workspace_for(device, nbytes: int):
    """A zero-filled per-device workspace of at least nbytes (reused: every
    successful call leaves it zero-filled).  A new workspace is zero-filled and
    the filling stream synchronised before it is returned, so a launch on any
    stream finds it zero.  Calls on different streams sharing it must not
    overlap.  After a call reports STATUS_SYNC_TIMEOUT (or KD_SYNC_TIMEOUT)
    the workspace may hold leftovers: call reset_workspaces() before reusing it."""
    import torch
    key = torch.device(device).index
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        torch.cuda.current_stream(ws.device).synchronize()
        _workspaces[key] = ws
    return ws


def reset_workspaces():
    """Zero every cached workspace again (after a SYNC_TIMEOUT status), waiting
    for all work on their devices first."""
    import torch
    for ws in _workspaces.values():
        torch.cuda.synchronize(ws.device)
        ws.zero_()
        torch.cuda.synchronize(ws.device)


def _row_stride(t, rows_per_seq):
    """Uniform row stride of a [B, R, V] tensor with unit element stride, or None."""
    if t.stride(2) != 1:
        return None
    rs = t.stride(1)
    if t.shape[1] > 1 and t.shape[0] > 1 and t.stride(0) != rs * rows_per_seq:
        return None
    if t.shape[1] == 1:
        rs = t.stride(0) if t.shape[0] > 1 else t.shape[2]
    return rs if rs >= t.shape[2] else None


def verify(target, draft, draft_tokens, uniforms, temperature: float, *, aux: bool = False,
           workspace=None, stream=None, events=None, layout: int = SV_LAYOUT_AUTO,
           variant: int = SV_VARIANT_AUTO) -> Result:
    """Verify on torch tensors of one device.

    target [B,k+1,V] and draft [B,k,V] (float32 or bfloat16, same dtype; draft
    may be None when temperature == 0), draft_tokens [B,k] int32, uniforms
    [B,k+2] float32 (None allowed when temperature == 0).  events: optional
    pair of torch.cuda.Event recorded on the current stream right before and
    after the call (the launch must then be on the current stream).  layout:
    SV_LAYOUT_* order of the streaming items, variant: SV_VARIANT_* kernel build
    (results depend on neither).  Returns device tensors.
    """
    import torch
    if target.dim() != 3:
        raise ValueError("target must be [B, k+1, V]")
    B, K1, V = target.shape
    k = K1 - 1
    greedy = float(temperature) == 0.0
    if target.dtype == torch.bfloat16:
        dt = SV_BF16
    elif target.dtype == torch.float32:
        dt = SV_F32
    else:
        raise TypeError("logits must be float32 or bfloat16")
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    ts = _row_stride(target, K1)
    if ts is None:
        target = target.contiguous()
        ts = V
    ds = 0
    if not greedy:
        if draft is None or uniforms is None:
            raise ValueError("sampling needs draft logits and uniforms")
        if draft.dtype != target.dtype or tuple(draft.shape) != (B, k, V) or draft.device != dev:
            raise ValueError("draft must be [B, k, V] with the target's dtype and device")
        ds = _row_stride(draft, k) if k > 0 else V
        if ds is None:
            draft = draft.contiguous()
            ds = V
        uniforms = uniforms.to(device=dev, dtype=torch.float32).contiguous()
        if tuple(uniforms.shape) != (B, k + 2):
            raise ValueError("uniforms must be [B, k+2]")
    draft_tokens = draft_tokens.to(device=dev, dtype=torch.int32).contiguous()
    if tuple(draft_tokens.shape) != (B, k):
        raise ValueError("draft_tokens must be [B, k]")
    shape = make_shape(B, k, V, dt, temperature, ts, ds)
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    acc = torch.empty(B, **i32)
    out = torch.empty(B, K1, **i32)
    tv = torch.empty(B, K1, TOPK, **f32)
    ti = torch.empty(B, K1, TOPK, **i32)
    st = torch.empty(B, **i32)
    a = sv_aux_t(st.data_ptr(), None, None, None, None, int(layout), int(variant))
    lt = ld = pt = qt = None
    if aux and not greedy:
        lt = torch.empty(B, K1, **f32)
        ld = torch.empty(B, k, **f32)
        pt = torch.empty(B, k, **f32)
        qt = torch.empty(B, k, **f32)
        a = sv_aux_t(st.data_ptr(), lt.data_ptr(), ld.data_ptr(), pt.data_ptr(), qt.data_ptr(), int(layout),
                     int(variant))
    nbytes = spec_verify_workspace_bytes(shape)
    ws = workspace if workspace is not None else workspace_for(dev, nbytes)
    cur = torch.cuda.current_stream(dev)
    if stream is None:
        stream = cur.cuda_stream
    if events is not None:
        if stream != cur.cuda_stream:
            raise ValueError("events are recorded on the current stream: launch there")
        events[0].record(cur)
    rc = spec_verify(shape, target.data_ptr(), None if greedy else draft.data_ptr(),
                     draft_tokens.data_ptr() if k > 0 else None, None if greedy else uniforms.data_ptr(),
                     acc.data_ptr(), out.data_ptr(), tv.data_ptr(), ti.data_ptr(), a,
                     ws.data_ptr(), ws.numel(), stream)
    if events is not None:
        events[1].record(cur)
    if rc != SV_OK:
        raise SpecVerifyError(rc)
    return Result(acc, out, tv, ti, st, lt, ld, pt, qt)


def to_device(w, device="cuda"):
    """Upload an sv_inputs.Workload: (target, draft, draft_tokens, uniforms) tensors."""
    import numpy as np
    import torch
    if w.dtype == SV_BF16:
        t = torch.from_numpy(w.target.view(np.int16)).view(torch.bfloat16)
        d = torch.from_numpy(w.draft.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(w.target)
        d = torch.from_numpy(w.draft)
    return (t.to(device), d.to(device), torch.from_numpy(w.draft_tokens).to(device),
            torch.from_numpy(w.uniforms).to(device))


# ---------------------------------------------------------------- distillation
KDResult = namedtuple("KDResult", "kl weight status loss grad")


def make_kd_shape(N, V, dtype, grad_dtype, S, group, w_max=float("inf"), row_stride=0) -> sv_kd_shape_t:
    return sv_kd_shape_t(int(N), int(V), int(dtype), int(grad_dtype), int(row_stride), int(S), int(group),
                         float(w_max))


def sv_kd_workspace_bytes(shape: sv_kd_shape_t) -> int:
    return int(load_library().sv_kd_workspace_bytes(ctypes.byref(shape)))


def sv_kd(shape: Optional[sv_kd_shape_t], draft_logits, topk_val, topk_idx, row_sample, rewards, kl, weight, status,
          loss, grad, workspace, workspace_bytes, stream) -> int:
    """Direct call of the C entry point with raw device addresses (ints or None)."""
    return int(load_library().sv_kd(None if shape is None else ctypes.byref(shape), draft_logits, topk_val, topk_idx,
                                    row_sample, rewards, kl, weight, status, loss, grad, workspace,
                                    int(workspace_bytes), stream))


def kd(draft_logits, topk_val, topk_idx, row_sample, rewards, group: int, *, w_max: float = float("inf"),
       grad: bool = True, grad_dtype=None, workspace=None, stream=None, events=None) -> KDResult:
    """Reward-weighted distillation loss (and gradient) on torch tensors of one
    device.  draft_logits [N,V] float32 or bfloat16 (unit element stride);
    topk_val [N,32] float32; topk_idx [N,32] int32; row_sample [N] int32;
    rewards [S] float32.  grad_dtype defaults to the logits' dtype.  events:
    optional pair of torch.cuda.Event recorded around the kernel."""
    import torch
    if draft_logits.dim() != 2 or draft_logits.stride(1) != 1:
        raise ValueError("draft_logits must be [N, V] with unit element stride")
    N, V = draft_logits.shape
    dev = draft_logits.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    dts = {torch.float32: SV_F32, torch.bfloat16: SV_BF16}
    if draft_logits.dtype not in dts:
        raise TypeError("draft logits must be float32 or bfloat16")
    dt = dts[draft_logits.dtype]
    gtorch = grad_dtype if grad_dtype is not None else draft_logits.dtype
    gdt = dts[gtorch]
    tv = topk_val.to(device=dev, dtype=torch.float32).contiguous()
    ti = topk_idx.to(device=dev, dtype=torch.int32).contiguous()
    rs = row_sample.to(device=dev, dtype=torch.int32).contiguous()
    rw = rewards.to(device=dev, dtype=torch.float32).contiguous()
    if tuple(tv.shape) != (N, TOPK) or tuple(ti.shape) != (N, TOPK) or tuple(rs.shape) != (N,):
        raise ValueError("topk_val/topk_idx must be [N, 32] and row_sample [N]")
    shape = make_kd_shape(N, V, dt, gdt, rw.numel(), group, w_max, draft_logits.stride(0) if N > 1 else V)
    f32 = dict(dtype=torch.float32, device=dev)
    kl = torch.empty(N, **f32)
    wt = torch.empty(N, **f32)
    st = torch.empty(N, dtype=torch.int32, device=dev)
    loss = torch.zeros(1, dtype=torch.float64, device=dev)
    g = torch.empty(N, V, dtype=gtorch, device=dev) if grad else None
    nbytes = sv_kd_workspace_bytes(shape)
    ws = workspace if workspace is not None else workspace_for(dev, nbytes)
    cur = torch.cuda.current_stream(dev)
    if stream is None:
        stream = cur.cuda_stream
    if events is not None:
        if stream != cur.cuda_stream:
            raise ValueError("events are recorded on the current stream: launch there")
        events[0].record(cur)
    rc = sv_kd(shape, draft_logits.data_ptr(), tv.data_ptr(), ti.data_ptr(), rs.data_ptr(), rw.data_ptr(),
               kl.data_ptr(), wt.data_ptr(), st.data_ptr(), loss.data_ptr(), None if g is None else g.data_ptr(),
               ws.data_ptr(), ws.numel(), stream)
    if events is not None:
        events[1].record(cur)
    if rc != SV_OK:
        raise SpecVerifyError(rc)
    return KDResult(kl, wt, st, loss, g)


def kd_to_device(w, device="cuda"):
    """Upload an sv_inputs.KDWorkload: (logits, topk_val, topk_idx, row_sample, rewards) tensors."""
    import numpy as np
    import torch
    z = torch.from_numpy(w.logits.view(np.int16)).view(torch.bfloat16) if w.dtype == SV_BF16 \
        else torch.from_numpy(w.logits)
    return (z.to(device), torch.from_numpy(w.topk_val).to(device), torch.from_numpy(w.topk_idx).to(device),
            torch.from_numpy(w.row_sample).to(device), torch.from_numpy(w.rewards).to(device))
