"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same bit patterns, and compare with the stated bars.

Bars (applied per output tensor):
  O, dQ, dKV   max|gpu - ref| <= 2e-2 * max|ref| and cosine >= 0.9995, all GPU
               entries finite; an all-zero reference needs max|gpu| <= 1e-6
  LSE          finite entries within 1e-3 absolute, non-finite entries equal
  d_sink       max|gpu - ref| <= 1e-2 * max|ref| over the head vector
               (<= 1e-6 absolute when the reference is all zero)
  dKV rows     the set of rows with any nonzero value is identical
With the exact Delta (smla_bwd_delta_exact), against the fp64 reference:
  Delta        max|gpu - ref| <= 1e-4 * max|ref| (fp32 sums of fp32 terms),
               and below the error of the bf16-O Delta
  d_sink       max|gpu - ref| <= 1e-4 * max|ref|
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

REL_TOL = 2e-2
COS_MIN = 0.9995
LSE_TOL = 1e-3
DSINK_TOL = 1e-2
# Outputs are fp32 and the kernels' fp32 exponentials return no subnormal
# results: a d_sink reference below the smallest normal fp32 is 0 at the
# kernel's precision.
FP32_TINY = float(np.finfo(np.float32).tiny)
# Whether a dKV row is nonzero is decided at the kernel's precision: P below
# 2^-126 is 0 there, and the 16-bit partials keep each slot's contribution to
# 2^-127 absolute, so a row whose reference lies wholly below 2^26 such
# contributions (more slots than any problem here names one row with) may be
# exactly 0; only rows above that, and rows the reference leaves exactly 0,
# are decided.
DKV_ROW_FLOOR = 2.0 ** -100


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(p, dev):
    return dict(
        q=p.q.to(dev), kv=p.kv.to(dev), dO=p.dO.to(dev), idx=p.topk_idxs.to(dev),
        length=None if p.topk_length is None else p.topk_length.to(dev),
        sink=None if p.attn_sink is None else p.attn_sink.to(dev),
    )


def run_gpu(p, dev, nan_prefill=True, ws_tokens=None):
    """Forward + preprocess + backward on the GPU; returns host numpy arrays.
    ``ws_tokens``: give the backward the workspace of that many tokens, so it
    runs in token chunks of (about) that size."""
    from sparse_top_attention_topk_amd import _lib
    d = to_dev(p, dev)
    ws = None
    if ws_tokens is not None:
        nb = _lib.smla_bwd_workspace_size(ws_tokens, p.S_kv, p.H, p.d_qk, p.d_v, p.W, p.scale)
        ws = torch.empty((nb,), dtype=torch.uint8, device=dev)
    T, H = p.T, p.H
    o = torch.empty((T, H, p.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    dq = torch.empty((T, H, p.d_qk), dtype=torch.bfloat16, device=dev)
    dkv = torch.empty((p.S_kv, p.d_qk), dtype=torch.float32, device=dev)
    if nan_prefill:
        for x in (o, lse, dq, dkv):
            x.fill_(float("nan"))
    o, lse = _lib.smla_fwd(d["q"], d["kv"], d["idx"], d["length"], d["sink"], p.scale, o=o, lse=lse)
    delta = _lib.smla_bwd_preprocess(o, d["dO"])
    d_sink = None
    if d["sink"] is not None:
        d_sink = torch.full((H,), float("nan"), dtype=torch.float32, device=dev)
    dq, dkv, d_sink = _lib.smla_bwd(d["q"], d["kv"], d["dO"], lse, delta, d["idx"], d["length"],
                                    d["sink"], p.scale, dq=dq, dkv=dkv, d_sink=d_sink, workspace=ws)
    torch.cuda.synchronize()
    out = dict(o=o.float().cpu().numpy(), lse=lse.cpu().numpy(), dq=dq.float().cpu().numpy(),
               dkv=dkv.cpu().numpy(), delta=delta.cpu().numpy(),
               d_sink=None if d_sink is None else d_sink.cpu().numpy())
    return out


def run_gpu_from_o(p, dev):
    """Forward, then smla_bwd_from_o (Delta formed inside the backward); the
    preprocess Delta is returned too (delta_pre) for comparison."""
    from sparse_top_attention_topk_amd import _lib
    d = to_dev(p, dev)
    T, H = p.T, p.H
    o, lse = _lib.smla_fwd(d["q"], d["kv"], d["idx"], d["length"], d["sink"], p.scale)
    delta_pre = _lib.smla_bwd_preprocess(o, d["dO"])
    delta = torch.full((T, H), float("nan"), dtype=torch.float32, device=dev)
    dq = torch.full((T, H, p.d_qk), float("nan"), dtype=torch.bfloat16, device=dev)
    dkv = torch.full((p.S_kv, p.d_qk), float("nan"), dtype=torch.float32, device=dev)
    d_sink = None if d["sink"] is None else torch.full((H,), float("nan"), dtype=torch.float32, device=dev)
    dq, dkv, d_sink, delta = _lib.smla_bwd_from_o(d["q"], d["kv"], d["dO"], o, lse, d["idx"], d["length"],
                                                  d["sink"], p.scale, delta=delta, dq=dq, dkv=dkv,
                                                  d_sink=d_sink)
    torch.cuda.synchronize()
    return dict(o=o.float().cpu().numpy(), lse=lse.cpu().numpy(), dq=dq.float().cpu().numpy(),
                dkv=dkv.cpu().numpy(), delta=delta.cpu().numpy(), delta_pre=delta_pre.cpu().numpy(),
                d_sink=None if d_sink is None else d_sink.cpu().numpy())


def run_gpu_exact(p, dev):
    """Forward, then the exact Delta (sum_j P_j dP_j) and the backward fed with
    it; the preprocess Delta (bf16 O . dO) is returned too for comparison."""
    from sparse_top_attention_topk_amd import _lib
    d = to_dev(p, dev)
    T, H = p.T, p.H
    o, lse = _lib.smla_fwd(d["q"], d["kv"], d["idx"], d["length"], d["sink"], p.scale)
    delta_pre = _lib.smla_bwd_preprocess(o, d["dO"])
    delta = torch.full((T, H), float("nan"), dtype=torch.float32, device=dev)
    _lib.smla_bwd_delta_exact(d["q"], d["kv"], d["dO"], lse, d["idx"], d["length"], d["sink"],
                              p.scale, delta=delta)
    d_sink = None if d["sink"] is None else torch.empty((H,), dtype=torch.float32, device=dev)
    dq, dkv, d_sink = _lib.smla_bwd(d["q"], d["kv"], d["dO"], lse, delta, d["idx"], d["length"],
                                    d["sink"], p.scale, d_sink=d_sink)
    torch.cuda.synchronize()
    return dict(o=o.float().cpu().numpy(), lse=lse.cpu().numpy(), dq=dq.float().cpu().numpy(),
                dkv=dkv.cpu().numpy(), delta=delta.cpu().numpy(), delta_pre=delta_pre.cpu().numpy(),
                d_sink=None if d_sink is None else d_sink.cpu().numpy())


def oracle_delta_exact(p, tokens=None):
    """The oracle's exact Delta on all tokens or on a token subset (only those
    tokens' rows are widened to fp64)."""
    tk = torch.arange(p.T) if tokens is None else torch.from_numpy(np.asarray(tokens, dtype=np.int64))
    return oracle.oracle_delta_exact(
        p.q[tk].double().numpy(), p.kv.double().numpy(), p.dO[tk].double().numpy(),
        p.topk_idxs[tk].numpy(), None if p.topk_length is None else p.topk_length[tk].numpy(),
        None if p.attn_sink is None else p.attn_sink.double().numpy(), p.scale, p.d_v)


def run_oracle(p, tokens=None, delta_from="bf16"):
    """The oracle on all tokens, or on a token subset (only those tokens' rows
    are widened to fp64; dKV and d_sink then sum over the subset only).

    The backward's Delta is taken from the forward output rounded to bf16 by
    default: smla_bwd_preprocess is defined on the bf16 O the forward returns,
    which is where the pages place the kernel's Delta ([cuDNN-FE #785] Not
    addressed).  ``delta_from="fp64"`` gives the exact-O reference."""
    if tokens is None:
        x = p.np_inputs()
    else:
        tk = torch.from_numpy(np.asarray(tokens, dtype=np.int64))
        x = dict(q=p.q[tk].double().numpy(), kv=p.kv.double().numpy(),
                 dO=p.dO[tk].double().numpy(), topk_idxs=p.topk_idxs[tk].numpy(),
                 topk_length=None if p.topk_length is None else p.topk_length[tk].numpy(),
                 attn_sink=None if p.attn_sink is None else p.attn_sink.double().numpy(),
                 scale=p.scale, d_v=p.d_v)
    O, lse, aux = oracle.oracle_fwd(x["q"], x["kv"], x["topk_idxs"], x["topk_length"],
                                    x["attn_sink"], x["scale"], x["d_v"])
    dq, dkv, ds, delta = oracle.oracle_bwd(x["q"], x["kv"], x["dO"], x["topk_idxs"],
                                           x["topk_length"], x["attn_sink"], x["scale"], x["d_v"],
                                           delta_from=delta_from)
    return dict(o=O, lse=lse, dq=dq, dkv=dkv, d_sink=ds, delta=delta, p_sink=aux["p_sink"])


def cosine(a, b):
    a = a.ravel().astype(np.float64)
    b = b.ravel().astype(np.float64)
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    if na == 0 or nb == 0:
        return 0.0
    return float(a @ b / (na * nb))


def check_tensor(name, gpu, ref, errors):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if gpu.shape != ref.shape:
        errors.append(f"{name}: shape {gpu.shape} vs {ref.shape}")
        return
    if not np.all(np.isfinite(gpu)):
        errors.append(f"{name}: {np.count_nonzero(~np.isfinite(gpu))} non-finite GPU entries")
        return
    mref = np.abs(ref).max() if ref.size else 0.0
    err = np.abs(gpu - ref).max() if ref.size else 0.0
    if mref == 0.0:
        if err > 1e-6:
            errors.append(f"{name}: reference is zero, max|gpu| = {err:.3e}")
        return
    cos = cosine(gpu, ref)
    if err > REL_TOL * mref or cos < COS_MIN:
        errors.append(f"{name}: max err {err:.3e} (rel {err / mref:.3e}), cos {cos:.6f}")


def check_lse(gpu, ref, errors):
    fin = np.isfinite(ref)
    if not np.array_equal(np.isfinite(gpu), fin):
        errors.append(f"lse: finiteness differs in {np.count_nonzero(np.isfinite(gpu) != fin)} entries")
        return
    if not np.array_equal(gpu[~fin], ref[~fin]):
        errors.append("lse: non-finite entries differ")
    if fin.any():
        e = np.abs(gpu[fin] - ref[fin]).max()
        if e > LSE_TOL:
            errors.append(f"lse: max abs err {e:.3e}")


def check_dsink(gpu, ref, errors):
    if ref is None:
        return
    if gpu is None or not np.all(np.isfinite(gpu)):
        errors.append("d_sink: missing or non-finite")
        return
    ref = np.where(np.abs(ref) < FP32_TINY, 0.0, ref)
    m = np.abs(ref).max()
    e = np.abs(gpu - ref).max()
    if (m == 0 and e > 1e-6) or (m > 0 and e > DSINK_TOL * m):
        errors.append(f"d_sink: max err {e:.3e} vs max|ref| {m:.3e}")


def check_dkv_rows(gpu_dkv, ref_dkv, errors):
    """Rows the reference leaves exactly 0 are exactly 0; rows whose reference
    reaches DKV_ROW_FLOOR are nonzero; rows in between are not decided."""
    g = np.any(gpu_dkv != 0, axis=1)
    m = np.abs(ref_dkv).max(axis=1)
    decided = (m == 0) | (m >= DKV_ROW_FLOOR)
    r = m >= DKV_ROW_FLOOR
    bad = decided & (g != r)
    if np.any(bad):
        errors.append(f"dkv rows: nonzero row sets differ ({np.count_nonzero(bad)} rows)")


def compare_exact_delta(gpu, ref64, errors):
    """Against the exact-O (fp64 Delta) reference the backward must still be
    aligned: cosine >= 0.9995 on dQ and dKV."""
    for k in ("dq", "dkv"):
        c = cosine(gpu[k], ref64[k])
        if c < COS_MIN and np.abs(ref64[k]).max() > 0:
            errors.append(f"{k} vs exact-Delta reference: cos {c:.6f}")


def compare_full(gpu, ref):
    errors = []
    check_tensor("o", gpu["o"], ref["o"], errors)
    check_lse(gpu["lse"], ref["lse"], errors)
    check_tensor("dq", gpu["dq"], ref["dq"], errors)
    check_tensor("dkv", gpu["dkv"], ref["dkv"], errors)
    check_dkv_rows(gpu["dkv"], ref["dkv"], errors)
    check_dsink(gpu["d_sink"], ref["d_sink"], errors)
    return errors


def referenced_rows(p):
    idx = p.topk_idxs.numpy()
    ok = (idx >= 0) & (idx < p.S_kv)
    if p.topk_length is not None:
        ln = np.clip(p.topk_length.numpy().astype(np.int64), 0, p.W)
        ok &= np.arange(p.W)[None, :] < ln[:, None]
    rows = np.zeros(p.S_kv, dtype=bool)
    rows[idx[ok]] = True
    return rows


def tokens_referencing(p, rows):
    idx = p.topk_idxs.numpy()
    ok = (idx >= 0) & (idx < p.S_kv)
    if p.topk_length is not None:
        ln = np.clip(p.topk_length.numpy().astype(np.int64), 0, p.W)
        ok &= np.arange(p.W)[None, :] < ln[:, None]
    hit = ok & np.isin(idx, np.asarray(rows))
    return np.nonzero(hit.any(axis=1))[0]
