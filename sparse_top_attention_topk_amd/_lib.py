"""ctypes binding of libsmla (the C ABI declared in include/smla.h).

Argument marshalling only: shapes, dtypes, devices and contiguity are checked,
outputs are allocated with torch when the caller does not pass them, and the
pointers plus torch's current HIP stream go to the library.  Every step of the
computation runs in the library's HIP kernels; there is no other code path.
If the library is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsmla.so")

SMLA_OK = 0


class SmlaDims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("S_kv", ctypes.c_int32), ("H", ctypes.c_int32),
                ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32), ("W", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class SmlaError(RuntimeError):
    pass


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run sparse_top_attention_topk_amd.build_lib.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32P, F32P = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    D = ctypes.POINTER(SmlaDims)
    lib.smla_fwd.argtypes = [D, P, P, I32P, I32P, F32P, P, F32P, P]
    lib.smla_fwd.restype = ctypes.c_int
    lib.smla_fwd_splitkv_workspace_size.argtypes = [D]
    lib.smla_fwd_splitkv_workspace_size.restype = ctypes.c_size_t
    lib.smla_fwd_splitkv.argtypes = [D, P, P, I32P, I32P, F32P, P, F32P, P, ctypes.c_size_t, P]
    lib.smla_fwd_splitkv.restype = ctypes.c_int
    lib.smla_bwd_preprocess.argtypes = [D, P, P, F32P, P]
    lib.smla_bwd_preprocess.restype = ctypes.c_int
    lib.smla_bwd_delta_exact.argtypes = [D, P, P, P, F32P, I32P, I32P, F32P, F32P, P]
    lib.smla_bwd_delta_exact.restype = ctypes.c_int
    lib.smla_bwd_workspace_size.argtypes = [D]
    lib.smla_bwd_workspace_size.restype = ctypes.c_size_t
    lib.smla_bwd_chunk_tokens.argtypes = [D, ctypes.c_size_t]
    lib.smla_bwd_chunk_tokens.restype = ctypes.c_int
    lib.smla_bwd.argtypes = [D, P, P, P, F32P, F32P, I32P, I32P, F32P, P, F32P, F32P, P,
                             ctypes.c_size_t, P]
    lib.smla_bwd.restype = ctypes.c_int
    lib.smla_bwd_from_o.argtypes = [D, P, P, P, P, F32P, F32P, I32P, I32P, F32P, P, F32P, F32P, P,
                                    ctypes.c_size_t, P]
    lib.smla_bwd_from_o.restype = ctypes.c_int
    lib.smla_bwd_profiled.argtypes = [D, P, P, P, F32P, F32P, I32P, I32P, F32P, P, F32P, F32P, P,
                                      ctypes.c_size_t, P, ctypes.POINTER(ctypes.c_void_p),
                                      ctypes.c_int]
    lib.smla_bwd_profiled.restype = ctypes.c_int
    lib.smla_bwd_noalloc.argtypes = [D, P, P, P, F32P, F32P, I32P, I32P, F32P, P, F32P, F32P, P]
    lib.smla_bwd_noalloc.restype = ctypes.c_int
    lib.smla_status_string.argtypes = [ctypes.c_int]
    lib.smla_status_string.restype = ctypes.c_char_p
    return lib


LIB = _load()

EXPORTED = ("smla_fwd", "smla_fwd_splitkv_workspace_size", "smla_fwd_splitkv", "smla_bwd_preprocess", "smla_bwd_delta_exact", "smla_bwd_workspace_size",
            "smla_bwd_chunk_tokens", "smla_bwd", "smla_bwd_from_o", "smla_bwd_profiled", "smla_bwd_noalloc", "smla_status_string")

SMLA_NOALLOC_SCRATCH_BYTES = 256 << 20

BWD_STAGES = ("index_inversion", "sdp_dq", "dq_merge", "dkv", "dkv_reduce", "dsink")


def _check(status: int, what: str):
    if status != SMLA_OK:
        msg = LIB.smla_status_string(status).decode()
        raise SmlaError(f"{what}: {msg} (status {status})")


def _ptr(x):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(x, name, dtype, device, ndim=None):
    if x is None:
        return
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {x.dtype}")
    if x.device != device:
        raise ValueError(f"{name} must be on {device}, got {x.device}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and x.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(x.shape)}")


def make_dims(T, S_kv, H, d_qk, d_v, W, scale) -> SmlaDims:
    return SmlaDims(int(T), int(S_kv), int(H), int(d_qk), int(d_v), int(W), float(scale))


def _dims_from(q, kv, topk_idxs, scale, d_v):
    T, H, d_qk = q.shape
    return make_dims(T, kv.shape[0], H, d_qk, d_v, topk_idxs.shape[1], scale)


def smla_fwd(q, kv, topk_idxs, topk_length, attn_sink, scale, o=None, lse=None, stream=None,
             d_v=512):
    """Forward; returns (o bf16 [T,H,d_v], lse fp32 [T,H] sink-free)."""
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 3)
    _need(kv, "kv", torch.bfloat16, dev, 2)
    _need(topk_idxs, "topk_idxs", torch.int32, dev, 2)
    _need(topk_length, "topk_length", torch.int32, dev, 1)
    _need(attn_sink, "attn_sink", torch.float32, dev, 1)
    T, H, _ = q.shape
    if topk_idxs.shape[0] != T or (topk_length is not None and topk_length.shape[0] != T):
        raise ValueError("topk_idxs / topk_length must have T rows")
    if attn_sink is not None and attn_sink.shape[0] != H:
        raise ValueError("attn_sink must have H entries")
    if o is None:
        o = torch.empty((T, H, d_v), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    _need(o, "o", torch.bfloat16, dev, 3)
    _need(lse, "lse", torch.float32, dev, 2)
    dims = _dims_from(q, kv, topk_idxs, scale, d_v)
    _check(LIB.smla_fwd(ctypes.byref(dims), _ptr(q), _ptr(kv), _ptr(topk_idxs), _ptr(topk_length),
                        _ptr(attn_sink), _ptr(o), _ptr(lse), _stream(dev, stream)), "smla_fwd")
    return o, lse


def smla_fwd_splitkv_workspace_size(T, S_kv, H, d_qk, d_v, W, scale=1.0) -> int:
    dims = make_dims(T, S_kv, H, d_qk, d_v, W, scale)
    return int(LIB.smla_fwd_splitkv_workspace_size(ctypes.byref(dims)))


def smla_fwd_splitkv(q, kv, topk_idxs, topk_length, attn_sink, scale, o=None, lse=None, workspace=None,
                     stream=None, d_v=512):
    """Forward with the token's slot blocks split over several workgroups
    when few tokens would leave the GPU idle; returns (o, lse) as smla_fwd.
    ``workspace``: uint8 device tensor, or None to allocate
    smla_fwd_splitkv_workspace_size bytes here."""
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 3)
    _need(kv, "kv", torch.bfloat16, dev, 2)
    _need(topk_idxs, "topk_idxs", torch.int32, dev, 2)
    _need(topk_length, "topk_length", torch.int32, dev, 1)
    _need(attn_sink, "attn_sink", torch.float32, dev, 1)
    T, H, _ = q.shape
    if topk_idxs.shape[0] != T or (topk_length is not None and topk_length.shape[0] != T):
        raise ValueError("topk_idxs / topk_length must have T rows")
    if attn_sink is not None and attn_sink.shape[0] != H:
        raise ValueError("attn_sink must have H entries")
    if o is None:
        o = torch.empty((T, H, d_v), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    _need(o, "o", torch.bfloat16, dev, 3)
    _need(lse, "lse", torch.float32, dev, 2)
    dims = _dims_from(q, kv, topk_idxs, scale, d_v)
    if workspace is None:
        need = int(LIB.smla_fwd_splitkv_workspace_size(ctypes.byref(dims)))
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev, 1)
    _check(LIB.smla_fwd_splitkv(ctypes.byref(dims), _ptr(q), _ptr(kv), _ptr(topk_idxs), _ptr(topk_length),
                                _ptr(attn_sink), _ptr(o), _ptr(lse), _ptr(workspace),
                                ctypes.c_size_t(workspace.numel()), _stream(dev, stream)),
           "smla_fwd_splitkv")
    return o, lse


def smla_bwd_preprocess(o, dO, delta=None, stream=None, scale=1.0):
    """Delta = rowsum(o * dO) in fp32; returns delta [T,H]."""
    dev = o.device
    _need(o, "o", torch.bfloat16, dev, 3)
    _need(dO, "dO", torch.bfloat16, dev, 3)
    if o.shape != dO.shape:
        raise ValueError("o and dO must have the same shape")
    T, H, d_v = o.shape
    if delta is None:
        delta = torch.empty((T, H), dtype=torch.float32, device=dev)
    _need(delta, "delta", torch.float32, dev, 2)
    dims = make_dims(T, 1, H, 576, d_v, 1, scale)
    _check(LIB.smla_bwd_preprocess(ctypes.byref(dims), _ptr(o), _ptr(dO), _ptr(delta),
                                   _stream(dev, stream)), "smla_bwd_preprocess")
    return delta


def smla_bwd_delta_exact(q, kv, dO, lse, topk_idxs, topk_length, attn_sink, scale, delta=None,
                         stream=None):
    """Exact Delta = sum_j P_j dP_j in fp32 (no bf16 O); returns delta [T,H]."""
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 3)
    _need(kv, "kv", torch.bfloat16, dev, 2)
    _need(dO, "dO", torch.bfloat16, dev, 3)
    _need(lse, "lse", torch.float32, dev, 2)
    _need(topk_idxs, "topk_idxs", torch.int32, dev, 2)
    _need(topk_length, "topk_length", torch.int32, dev, 1)
    _need(attn_sink, "attn_sink", torch.float32, dev, 1)
    T, H, _ = q.shape
    d_v = dO.shape[2]
    if dO.shape[:2] != (T, H) or lse.shape != (T, H):
        raise ValueError("dO and lse must match q's [T, H]")
    if topk_idxs.shape[0] != T or (topk_length is not None and topk_length.shape[0] != T):
        raise ValueError("topk_idxs / topk_length must have T rows")
    if attn_sink is not None and attn_sink.shape[0] != H:
        raise ValueError("attn_sink must have H entries")
    if delta is None:
        delta = torch.empty((T, H), dtype=torch.float32, device=dev)
    _need(delta, "delta", torch.float32, dev, 2)
    dims = _dims_from(q, kv, topk_idxs, scale, d_v)
    _check(LIB.smla_bwd_delta_exact(ctypes.byref(dims), _ptr(q), _ptr(kv), _ptr(dO), _ptr(lse),
                                    _ptr(topk_idxs), _ptr(topk_length), _ptr(attn_sink), _ptr(delta),
                                    _stream(dev, stream)), "smla_bwd_delta_exact")
    return delta


def smla_bwd_workspace_size(T, S_kv, H, d_qk, d_v, W, scale=1.0) -> int:
    dims = make_dims(T, S_kv, H, d_qk, d_v, W, scale)
    return int(LIB.smla_bwd_workspace_size(ctypes.byref(dims)))


def smla_bwd_chunk_tokens(T, S_kv, H, d_qk, d_v, W, workspace_bytes, scale=1.0) -> int:
    dims = make_dims(T, S_kv, H, d_qk, d_v, W, scale)
    return int(LIB.smla_bwd_chunk_tokens(ctypes.byref(dims), ctypes.c_size_t(int(workspace_bytes))))


def smla_bwd(q, kv, dO, lse, delta, topk_idxs, topk_length, attn_sink, scale, dq=None, dkv=None,
             d_sink=None, workspace=None, stream=None, stage_events=None):
    """Backward; returns (dq bf16 [T,H,d_qk], dkv fp32 [S_kv,d_qk], d_sink fp32 [H] or None).

    With ``stage_events`` (len(BWD_STAGES) + 1 torch.cuda.Event objects that
    have been recorded once), smla_bwd_profiled runs instead and records them
    at the stage boundaries."""
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 3)
    _need(kv, "kv", torch.bfloat16, dev, 2)
    _need(dO, "dO", torch.bfloat16, dev, 3)
    _need(lse, "lse", torch.float32, dev, 2)
    _need(delta, "delta", torch.float32, dev, 2)
    _need(topk_idxs, "topk_idxs", torch.int32, dev, 2)
    _need(topk_length, "topk_length", torch.int32, dev, 1)
    _need(attn_sink, "attn_sink", torch.float32, dev, 1)
    T, H, d_qk = q.shape
    d_v = dO.shape[2]
    dims = _dims_from(q, kv, topk_idxs, scale, d_v)
    if dq is None:
        dq = torch.empty_like(q)
    if dkv is None:
        dkv = torch.empty((kv.shape[0], d_qk), dtype=torch.float32, device=dev)
    if attn_sink is not None and d_sink is None:
        d_sink = torch.empty((H,), dtype=torch.float32, device=dev)
    _need(dq, "dq", torch.bfloat16, dev, 3)
    _need(dkv, "dkv", torch.float32, dev, 2)
    _need(d_sink, "d_sink", torch.float32, dev, 1)
    need = int(LIB.smla_bwd_workspace_size(ctypes.byref(dims)))
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev, 1)
    args = (ctypes.byref(dims), _ptr(q), _ptr(kv), _ptr(dO), _ptr(lse), _ptr(delta),
            _ptr(topk_idxs), _ptr(topk_length), _ptr(attn_sink), _ptr(dq), _ptr(dkv),
            _ptr(d_sink), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
            _stream(dev, stream))
    if stage_events is None:
        _check(LIB.smla_bwd(*args), "smla_bwd")
    else:
        handles = (ctypes.c_void_p * len(stage_events))(
            *[ctypes.c_void_p(e.cuda_event) for e in stage_events])
        _check(LIB.smla_bwd_profiled(*args, handles, len(stage_events)), "smla_bwd_profiled")
    return dq, dkv, d_sink


def smla_bwd_from_o(q, kv, dO, o, lse, topk_idxs, topk_length, attn_sink, scale, delta=None, dq=None,
                    dkv=None, d_sink=None, workspace=None, stream=None):
    """smla_bwd_preprocess + smla_bwd in one call (Delta formed inside the
    backward from ``o``); returns (dq, dkv, d_sink or None, delta fp32 [T,H])."""
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 3)
    _need(kv, "kv", torch.bfloat16, dev, 2)
    _need(dO, "dO", torch.bfloat16, dev, 3)
    _need(o, "o", torch.bfloat16, dev, 3)
    _need(lse, "lse", torch.float32, dev, 2)
    _need(topk_idxs, "topk_idxs", torch.int32, dev, 2)
    _need(topk_length, "topk_length", torch.int32, dev, 1)
    _need(attn_sink, "attn_sink", torch.float32, dev, 1)
    T, H, d_qk = q.shape
    d_v = dO.shape[2]
    dims = _dims_from(q, kv, topk_idxs, scale, d_v)
    if delta is None:
        delta = torch.empty((T, H), dtype=torch.float32, device=dev)
    if dq is None:
        dq = torch.empty_like(q)
    if dkv is None:
        dkv = torch.empty((kv.shape[0], d_qk), dtype=torch.float32, device=dev)
    if attn_sink is not None and d_sink is None:
        d_sink = torch.empty((H,), dtype=torch.float32, device=dev)
    _need(delta, "delta", torch.float32, dev, 2)
    _need(dq, "dq", torch.bfloat16, dev, 3)
    _need(dkv, "dkv", torch.float32, dev, 2)
    _need(d_sink, "d_sink", torch.float32, dev, 1)
    need = int(LIB.smla_bwd_workspace_size(ctypes.byref(dims)))
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev, 1)
    _check(LIB.smla_bwd_from_o(ctypes.byref(dims), _ptr(q), _ptr(kv), _ptr(dO), _ptr(o), _ptr(lse),
                               _ptr(delta), _ptr(topk_idxs), _ptr(topk_length), _ptr(attn_sink),
                               _ptr(dq), _ptr(dkv), _ptr(d_sink), _ptr(workspace),
                               ctypes.c_size_t(workspace.numel()), _stream(dev, stream)),
           "smla_bwd_from_o")
    return dq, dkv, d_sink, delta


def smla_bwd_profiled(*args, stage_events, **kw):
    """smla_bwd recording ``stage_events`` at its stage boundaries."""
    return smla_bwd(*args, stage_events=stage_events, **kw)


def smla_bwd_noalloc(q, kv, dO, lse, delta, topk_idxs, topk_length, attn_sink, scale, dq=None, dkv=None,
                     d_sink=None, stream=None):
    """smla_bwd on the library's fixed per-GPU scratch (no workspace, nothing
    allocated by the call when the outputs are given); returns (dq, dkv,
    d_sink or None).  Calls that overlap on one GPU share the scratch."""
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 3)
    _need(kv, "kv", torch.bfloat16, dev, 2)
    _need(dO, "dO", torch.bfloat16, dev, 3)
    _need(lse, "lse", torch.float32, dev, 2)
    _need(delta, "delta", torch.float32, dev, 2)
    _need(topk_idxs, "topk_idxs", torch.int32, dev, 2)
    _need(topk_length, "topk_length", torch.int32, dev, 1)
    _need(attn_sink, "attn_sink", torch.float32, dev, 1)
    T, H, d_qk = q.shape
    d_v = dO.shape[2]
    dims = _dims_from(q, kv, topk_idxs, scale, d_v)
    if dq is None:
        dq = torch.empty_like(q)
    if dkv is None:
        dkv = torch.empty((kv.shape[0], d_qk), dtype=torch.float32, device=dev)
    if attn_sink is not None and d_sink is None:
        d_sink = torch.empty((H,), dtype=torch.float32, device=dev)
    _need(dq, "dq", torch.bfloat16, dev, 3)
    _need(dkv, "dkv", torch.float32, dev, 2)
    _need(d_sink, "d_sink", torch.float32, dev, 1)
    _check(LIB.smla_bwd_noalloc(ctypes.byref(dims), _ptr(q), _ptr(kv), _ptr(dO), _ptr(lse), _ptr(delta),
                                _ptr(topk_idxs), _ptr(topk_length), _ptr(attn_sink), _ptr(dq), _ptr(dkv),
                                _ptr(d_sink), _stream(dev, stream)), "smla_bwd_noalloc")
    return dq, dkv, d_sink
