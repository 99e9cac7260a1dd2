"""Central finite differences of L = sum(dO * O) through the oracle forward.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

A pin for the oracle backward that uses only the oracle forward: along a random
direction (u_q, u_kv, u_sink) the directional derivative of L must equal the
inner product of that direction with (dQ, dKV, d_sink).
"""
from __future__ import annotations

from .smla import oracle_fwd

__all__ = ["loss", "directional_fd"]


def loss(q, kv, dO, topk_idxs, topk_length, attn_sink, scale, d_v):
    O, _, _ = oracle_fwd(q, kv, topk_idxs, topk_length, attn_sink, scale, d_v)
    return float((O * dO).sum())


def directional_fd(q, kv, dO, topk_idxs, topk_length, attn_sink, scale, d_v,
                   u_q, u_kv, u_sink=None, eps=1e-5):
    """(L(x + eps u) - L(x - eps u)) / (2 eps), with x = (q, kv, sink)."""
    def at(sign):
        s = None if attn_sink is None else attn_sink + sign * eps * u_sink
        return loss(q + sign * eps * u_q, kv + sign * eps * u_kv, dO, topk_idxs,
                    topk_length, s, scale, d_v)
    return (at(+1.0) - at(-1.0)) / (2.0 * eps)
