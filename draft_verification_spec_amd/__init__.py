"""Python binding of the spec_verify C ABI (include/spec_verify.h).

Argument marshalling only: every step of the verification runs in the HIP
library libspec_verify.so built next to this file.  PyTorch supplies device
memory and the stream.  Importing works without a GPU; calling spec_verify or
verify needs the built library and an MI355X, and raises if either is missing.
"""
from __future__ import annotations

import ctypes
import os
import re
from collections import namedtuple
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspec_verify.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "spec_verify.h")

SV_F32, SV_BF16 = 0, 1
TOPK = 32
SV_OK = 0
SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_TEMPERATURE, SV_ERR_DTYPE = -1, -2, -3, -4
SV_ERR_WORKSPACE, SV_ERR_HIP, SV_ERR_DEVICE = -5, -6, -7
STATUS_BAD_TOKEN, STATUS_NAN, STATUS_POSINF, STATUS_EMPTY_ROW = 1, 2, 4, 8
STATUS_BAD_UNIFORM, STATUS_SYNC_TIMEOUT = 16, 32


class sv_shape_t(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("k", ctypes.c_int32), ("V", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("target_row_stride", ctypes.c_int64), ("draft_row_stride", ctypes.c_int64),
                ("temperature", ctypes.c_float)]


class sv_aux_t(ctypes.Structure):
    _fields_ = [("status", ctypes.c_void_p), ("lse_target", ctypes.c_void_p), ("lse_draft", ctypes.c_void_p),
                ("p_tok", ctypes.c_void_p), ("q_tok", ctypes.c_void_p),
                ("event_begin", ctypes.c_void_p), ("event_end", ctypes.c_void_p)]


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
        lib.spec_verify_error_string.argtypes = [ctypes.c_int]
        lib.spec_verify_error_string.restype = ctypes.c_char_p
        lib.spec_verify.argtypes = [ctypes.POINTER(sv_shape_t), P, P, P, P, P, P, P, P,
                                    ctypes.POINTER(sv_aux_t), P, ctypes.c_size_t, P]
        lib.spec_verify.restype = ctypes.c_int
        _lib = lib
    return _lib


def declared_functions() -> list:
    """Names of the functions include/spec_verify.h declares."""
    text = open(HEADER_PATH).read()
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(spec_verify\w*)\s*\(", text, flags=re.M)


def make_shape(B, k, V, dtype, temperature, target_row_stride=0, draft_row_stride=0) -> sv_shape_t:
    return sv_shape_t(int(B), int(k), int(V), int(dtype), int(target_row_stride), int(draft_row_stride),
                      float(temperature))


def spec_verify_workspace_bytes(shape: sv_shape_t) -> int:
    return int(load_library().spec_verify_workspace_bytes(ctypes.byref(shape)))


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


# ------------------------------------------------------------ torch front end
Result = namedtuple("Result", "accepted_len out_tokens topk_val topk_idx status lse_target lse_draft p_tok q_tok")

_workspaces = {}


def workspace_for(device, nbytes: int):
    """A zero-filled per-device workspace of at least nbytes (reused: every call
    leaves it zero-filled).  Calls on different streams sharing it must not overlap."""
    import torch
    key = torch.device(device).index
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


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
           workspace=None, stream=None, events=None) -> Result:
    """Verify on torch tensors of one device.

    target [B,k+1,V] and draft [B,k,V] (float32 or bfloat16, same dtype; draft
    may be None when temperature == 0), draft_tokens [B,k] int32, uniforms
    [B,k+2] float32 (None allowed when temperature == 0).  events: optional
    pair of torch.cuda.Event recorded right before and after the streaming
    kernel on the launch stream.  Returns device tensors.
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
    a = sv_aux_t(st.data_ptr(), None, None, None, None, None, None)
    lt = ld = pt = qt = None
    if aux and not greedy:
        lt = torch.empty(B, K1, **f32)
        ld = torch.empty(B, k, **f32)
        pt = torch.empty(B, k, **f32)
        qt = torch.empty(B, k, **f32)
        a = sv_aux_t(st.data_ptr(), lt.data_ptr(), ld.data_ptr(), pt.data_ptr(), qt.data_ptr(), None, None)
    if events is not None:
        a.event_begin, a.event_end = events[0].cuda_event, events[1].cuda_event
    nbytes = spec_verify_workspace_bytes(shape)
    ws = workspace if workspace is not None else workspace_for(dev, nbytes)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = spec_verify(shape, target.data_ptr(), None if greedy else draft.data_ptr(),
                     draft_tokens.data_ptr() if k > 0 else None, None if greedy else uniforms.data_ptr(),
                     acc.data_ptr(), out.data_ptr(), tv.data_ptr(), ti.data_ptr(), a,
                     ws.data_ptr(), ws.numel(), stream)
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
