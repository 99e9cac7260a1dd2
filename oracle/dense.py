"""Dense masked attention in torch fp64: an independent formulation that pins
the per-slot oracle.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Instead of gathering the valid slots of each token, this builds one boolean
mask over all (token, KV row) pairs and runs ordinary dense softmax attention
over every KV row, with the sink appended as an extra logit column that has no
value row.  The mask is built by indexing with the valid (token, index) pairs
only; a -1 sentinel is never clamped to a row number, so row 0 is marked only
when a valid slot names it ([cuDNN-FE #298], the test-reference fix: clamping
-1 to 0 had marked row 0 as attended).

Gradients come from torch autograd, so none of the oracle's hand-written
backward formulas is reused.  A row named twice in one token's slots is marked
once here (the per-slot oracle would count it twice); inputs used to compare
the two hold distinct indices per row.
"""
from __future__ import annotations

import torch

__all__ = ["dense_mask", "dense_attention", "dense_loss_grads"]


def dense_mask(topk_idxs: torch.Tensor, topk_length, S_kv: int) -> torch.Tensor:
    """Boolean [T, S_kv]: token t attends KV row r."""
    T, W = topk_idxs.shape
    idx = topk_idxs.to(torch.int64)
    pos = torch.arange(W).unsqueeze(0).expand(T, W)
    if topk_length is None:
        cand = torch.ones(T, W, dtype=torch.bool)
    else:
        ln = torch.as_tensor(topk_length, dtype=torch.int64).clamp(0, W)
        cand = pos < ln.unsqueeze(1)
    valid = cand & (idx >= 0) & (idx < S_kv)
    t_ids = torch.arange(T).unsqueeze(1).expand(T, W)[valid]
    r_ids = idx[valid]
    mask = torch.zeros(T, S_kv, dtype=torch.bool)
    mask[t_ids, r_ids] = True
    return mask


def dense_attention(q, kv, mask, attn_sink, scale, d_v):
    """O [T,H,d_v] and sink-free LSE [T,H] of dense masked attention (fp64)."""
    T, H, d_qk = q.shape
    S = scale * torch.einsum("thc,rc->thr", q, kv[:, :d_qk])          # [T,H,S_kv]
    neg = torch.tensor(float("-inf"), dtype=S.dtype)
    S = torch.where(mask.unsqueeze(1), S, neg)
    lse_cols = torch.logsumexp(S, dim=-1)                                # -inf if empty
    if attn_sink is not None:
        sink_col = attn_sink.view(1, H, 1).expand(T, H, 1)
        logits = torch.cat([S, sink_col], dim=-1)
    else:
        logits = S
    lse_tot = torch.logsumexp(logits, dim=-1, keepdim=True)
    safe = torch.where(torch.isfinite(lse_tot), lse_tot, torch.zeros_like(lse_tot))
    P = torch.exp(logits - safe)
    P = torch.where(torch.isposinf(lse_tot), torch.zeros_like(P), P)
    O = torch.einsum("thr,rc->thc", P[..., : kv.shape[0]], kv[:, :d_v])
    return O, lse_cols


def dense_loss_grads(q, kv, dO, mask, attn_sink, scale, d_v):
    """Gradients of L = sum(dO * O) by autograd: (dq, dkv, d_sink or None)."""
    q = q.detach().clone().requires_grad_(True)
    kv = kv.detach().clone().requires_grad_(True)
    sink = None
    if attn_sink is not None:
        sink = attn_sink.detach().clone().requires_grad_(True)
    O, _ = dense_attention(q, kv, mask, sink, scale, d_v)
    L = (O * dO).sum()
    grads = torch.autograd.grad(L, [x for x in (q, kv, sink) if x is not None])
    dq, dkv = grads[0], grads[1]
    ds = grads[2] if sink is not None else None
    return dq, dkv, ds
