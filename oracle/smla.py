"""fp64 oracle: sparse top-k MLA attention, forward and backward, by definition.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Sources (the pages, cited by title and section):

* [cuDNN-FE #785] "DSA backward SM90: fix three top-k and attention-sink
  boundary failures" -- Summary items 1-3, Why 1-3, Testing, Not addressed.
* [cuDNN-FE #298] "DSA bwd SM100 fix dropped dKV gradients when topk width >
  total_S_kv" -- description and the test-reference fix.
* [flash-attn #2882] "[CuTe, SM100] Support 1..128 Q heads in sparse MLA via
  in-kernel TMA padding" -- Agent Notes, Mechanism, Performance.
* [Automodel #3467] "Fix DeepSeek-V4 TileLang sparse-MLA backward compilation
  on Blackwell" -- the review's statement of the validity mask.

What is computed (plain definition; the method is exact, not approximate):
for every token t and head h, softmax attention over the KV rows listed in the
token's valid top-k slots, with an optional per-head sink logit that joins the
softmax denominator and carries no value row.  Query heads share one latent KV
row set (MQA): K = kv[:, :d_qk], V = kv[:, :d_v].

Readings of points the pages leave open:

* the forward returns the sink-free natural-log LSE of the valid scores;
  O carries the sink's normalisation (the backward folds the sink into the LSE
  itself, [cuDNN-FE #785] Summary 3);
* an empty row has LSE = -inf, O = 0, dQ = 0;
* an index outside [0, S_kv) is invalid in both layouts; a negative length is
  an empty row; a length above the width is clamped to the width;
* duplicate indices in a row count once per slot (a slot-based gather).

Every array here is float64 unless stated.  Inputs arrive as the exact values
the GPU receives (bf16 / fp32 bit patterns widened to fp64).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "valid_slots",
    "glae",
    "p_sink",
    "round_to_bf16",
    "oracle_fwd",
    "oracle_bwd",
    "oracle_delta_exact",
    "oracle_dsink",
]


# --------------------------------------------------------------------------
# Validity of a slot
# --------------------------------------------------------------------------
def valid_slots(idx_row: np.ndarray, length, S_kv: int):
    """Slot positions and KV rows of the valid slots of one token.

    Two index layouts ([cuDNN-FE #785] Why 2, quoting the SM100 contract that a
    missing length means non-compact with -1 entries; [cuDNN-FE #298]):

    * compact (``length`` given): slots j < length are the candidates, the tail
      is ignored whatever it holds;
    * non-compact (``length is None``): every slot of the row is a candidate and
      -1 marks padding anywhere in the row.

    A candidate is valid iff 0 <= idx < S_kv (the TileLang interface's mask,
    [Automodel #3467] review).  Validity is decided by the index *value* and the
    slot position, never by comparing the slot position with S_kv: a column
    >= S_kv in a row wider than S_kv is still valid ([cuDNN-FE #298]).
    """
    W = idx_row.shape[0]
    if length is None:
        n = W
    else:
        # nonpositive length = empty row ([cuDNN-FE #785] Summary 1); a length
        # above the width has no defined meaning and is clamped to it.
        n = min(max(int(length), 0), W)
    cand = np.arange(n, dtype=np.int64)
    ids = idx_row[:n].astype(np.int64)
    ok = (ids >= 0) & (ids < S_kv)
    return cand[ok], ids[ok]


# --------------------------------------------------------------------------
# Sink folding ([cuDNN-FE #785] Summary 3 and Why 3)
# --------------------------------------------------------------------------
def glae(a, b):
    """Finite-max-guarded logaddexp, elementwise: ln(e^a + e^b).

    Shift by the maximum only while that maximum is finite; an infinite
    maximum is already the answer ([cuDNN-FE #785] Why 3).
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    m = np.maximum(a, b)
    out = np.array(m, dtype=np.float64, copy=True)
    fin = np.isfinite(m)
    with np.errstate(over="ignore", invalid="ignore"):
        out[fin] = m[fin] + np.log(np.exp(a[fin] - m[fin]) + np.exp(b[fin] - m[fin]))
    return out


def p_sink(lse_cols, sink):
    """Probability mass that the sink takes: e^sink / (e^sink + sum_j e^{s_j}).

    Written as the sigmoid sigma(sink - lse_cols), which the page states is
    algebraically the same as exp(sink - logaddexp(lse, sink)) but stays finite
    when either term saturates ([cuDNN-FE #785] Why 3).  The limits:
    sink = -inf (or no sink) -> 0; lse = -inf with sink > -inf -> 1;
    sink = lse = +inf -> 1/2 (the review thread on the same page).
    """
    lse_cols = np.asarray(lse_cols, dtype=np.float64)
    if sink is None:
        return np.zeros_like(lse_cols)
    sink = np.broadcast_to(np.asarray(sink, dtype=np.float64), lse_cols.shape)
    out = np.empty_like(lse_cols)
    both_inf = np.isposinf(sink) & np.isposinf(lse_cols)
    sink_neg_inf = np.isneginf(sink)
    lse_neg_inf = np.isneginf(lse_cols) & ~sink_neg_inf
    rest = ~(both_inf | sink_neg_inf | lse_neg_inf)
    out[both_inf] = 0.5
    out[sink_neg_inf] = 0.0
    out[lse_neg_inf] = 1.0
    x = sink[rest] - lse_cols[rest]
    # sigma(x) without overflow for either sign of x
    with np.errstate(over="ignore"):
        pos = x >= 0
        r = np.empty_like(x)
        r[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
        ex = np.exp(x[~pos])
        r[~pos] = ex / (1.0 + ex)
    out[rest] = r
    return out


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (round to nearest, ties to even), as fp64.

    Used only to mirror the pages' statement that the backward's Delta comes
    from the bf16-stored O ([cuDNN-FE #785] Not addressed, first item).  The
    value goes fp64 -> fp32 (RNE by NumPy) -> bf16 (RNE on the bit pattern).
    NaN is not expected here (O is finite by construction).
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Forward
# --------------------------------------------------------------------------
def _token_probs(q_t, kv, rows, scale, sink, d_qk):
    """Scores, LSE of the valid scores, LSE with the sink, and probabilities.

    s_j = scale * <q[t,h,:d_qk], kv[idx_j,:d_qk]> over the valid slots only: a
    padded or invalid slot never enters the softmax (it is masked before the
    exponential, [cuDNN-FE #785] Summary 2 and Why 2).
    """
    H = q_t.shape[0]
    K = kv[rows, :d_qk]                     # [K_t, d_qk]
    s = scale * (q_t[:, :d_qk] @ K.T)       # [H, K_t]
    if rows.size == 0:
        lse_cols = np.full(H, -np.inf)
    else:
        m = s.max(axis=1)
        lse_cols = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    if sink is None:
        lse_tot = lse_cols.copy()
    else:
        lse_tot = glae(lse_cols, sink)
    # p_j = e^{s_j} / (sum_k e^{s_k} + e^{sink}) = exp(s_j - lse_tot); zero
    # where the total is +inf (a saturating positive sink takes all the mass).
    with np.errstate(invalid="ignore", over="ignore"):
        p = np.exp(s - lse_tot[:, None])
    p[~np.isfinite(lse_tot), :] = 0.0
    return s, lse_cols, lse_tot, p


def oracle_fwd(q, kv, topk_idxs, topk_length, attn_sink, scale, d_v, tokens=None):
    """Forward: O[t,h,:] and the sink-free LSE[t,h] (natural log).

    Parameters are NumPy arrays: q [T,H,d_qk], kv [S_kv,d_qk], topk_idxs [T,W]
    int, topk_length [T] int or None, attn_sink [H] or None; d_v <= d_qk.
    ``tokens`` restricts the computation to a subset of token indices (the
    returned arrays are then indexed by position in that subset).

    Returns (O [T',H,d_v], lse [T',H], aux) where aux holds lse_tot and
    p_sink [T',H] for diagnostics.
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    T, H, d_qk = q.shape
    S_kv = kv.shape[0]
    sink = None if attn_sink is None else np.asarray(attn_sink, dtype=np.float64)
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    O = np.zeros((len(toks), H, d_v))
    lse = np.empty((len(toks), H))
    lse_tot_all = np.empty((len(toks), H))
    ps = np.empty((len(toks), H))
    for i, t in enumerate(toks):
        ln = None if topk_length is None else topk_length[t]
        _, rows = valid_slots(topk_idxs[t], ln, S_kv)
        _, lse_cols, lse_tot, p = _token_probs(q[t], kv, rows, scale, sink, d_qk)
        O[i] = p @ kv[rows, :d_v]
        lse[i] = lse_cols
        lse_tot_all[i] = lse_tot
        ps[i] = p_sink(lse_cols, sink)
    return O, lse, {"lse_tot": lse_tot_all, "p_sink": ps}


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------
def oracle_bwd(q, kv, dO, topk_idxs, topk_length, attn_sink, scale, d_v,
               delta_from="fp64", tokens=None):
    """Backward of L = sum(dO * O): dQ, dKV, d_sink (and Delta).

    Steps per token, after the forward's probabilities p_j are recomputed:

    * Delta[h] = sum_c dO[t,h,c] * O[t,h,c]  (the FlashAttention identity the
      pages name; [cuDNN-FE #785] Not addressed).  ``delta_from="fp64"`` uses
      the oracle's own fp64 O; ``"bf16"`` rounds that O to bf16 first, which is
      what the pages say the kernel does.
    * dP_j = <dO[t,h,:], kv[idx_j,:d_v]>,  dS_j = p_j (dP_j - Delta).
    * dQ[t,h,:] = scale * sum_j dS_j kv[idx_j,:d_qk]
    * dKV[idx_j,:d_qk] += scale * sum_h dS_j q[t,h,:];
      dKV[idx_j,:d_v]  += sum_h p_j dO[t,h,:]   (scatter over valid slots only;
      a -1 never lands on row 0, [cuDNN-FE #298]).
    * d_sink[h] = -sum_t p_sink[t,h] * Delta[t,h]: dp_j/dsink = -p_j p_sink,
      which gives -Delta at p_sink = 1 ([cuDNN-FE #785] Testing: a saturating
      positive sink gives d_sink = -sum(dP_sum)).

    ``tokens`` restricts dQ and Delta to a token subset; dKV and d_sink then
    sum over that subset only.
    Returns (dq [T',H,d_qk], dkv [S_kv,d_qk], d_sink [H] or None, delta [T',H]).
    """
    if delta_from not in ("fp64", "bf16"):
        raise ValueError(delta_from)
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    T, H, d_qk = q.shape
    S_kv = kv.shape[0]
    sink = None if attn_sink is None else np.asarray(attn_sink, dtype=np.float64)
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    dq = np.zeros((len(toks), H, d_qk))
    dkv = np.zeros((S_kv, d_qk))
    d_sink = np.zeros(H)
    delta = np.zeros((len(toks), H))
    for i, t in enumerate(toks):
        ln = None if topk_length is None else topk_length[t]
        _, rows = valid_slots(topk_idxs[t], ln, S_kv)
        if rows.size == 0:
            # empty row: dQ = 0, no contribution anywhere ([cuDNN-FE #785]
            # Summary 1 and Why 1: an empty row needs no Q, dO, LSE or Delta)
            continue
        _, lse_cols, _, p = _token_probs(q[t], kv, rows, scale, sink, d_qk)
        o_t = p @ kv[rows, :d_v]
        if delta_from == "bf16":
            o_t = round_to_bf16(o_t)
        dl = (dO[t] * o_t).sum(axis=1)                  # [H]
        dP = dO[t] @ kv[rows, :d_v].T                    # [H, K_t]
        dS = p * (dP - dl[:, None])                      # [H, K_t]
        dq[i] = scale * (dS @ kv[rows, :d_qk])
        gk = scale * (dS.T @ q[t][:, :d_qk])             # [K_t, d_qk]
        gv = p.T @ dO[t]                                 # [K_t, d_v]
        contrib = gk
        contrib[:, :d_v] += gv
        if np.unique(rows).size == rows.size:
            dkv[rows] += contrib
        else:
            np.add.at(dkv, rows, contrib)
        delta[i] = dl
        if sink is not None:
            d_sink -= p_sink(lse_cols, sink) * dl
    return dq, dkv, (d_sink if sink is not None else None), delta


def oracle_delta_exact(q, kv, dO, topk_idxs, topk_length, attn_sink, scale, d_v, tokens=None):
    """Delta[t,h] = sum_j p_j dP_j over the token's valid slots.

    The second delta source of the table in [cuDNN-FE #785] Not addressed:
    the probabilities p_j (with the sink in the denominator) times
    dP_j = <dO[t,h,:], kv[idx_j,:d_v]>, summed over the valid slots, instead
    of the product of dO with the stored output.  By the FlashAttention
    identity it equals dO . O for the exact O.  An empty row gives 0.
    Returns delta [T',H] (``tokens`` as in oracle_fwd).
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    T, H, d_qk = q.shape
    S_kv = kv.shape[0]
    sink = None if attn_sink is None else np.asarray(attn_sink, dtype=np.float64)
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    delta = np.zeros((len(toks), H))
    for i, t in enumerate(toks):
        ln = None if topk_length is None else topk_length[t]
        _, rows = valid_slots(topk_idxs[t], ln, S_kv)
        if rows.size == 0:
            continue
        _, _, _, p = _token_probs(q[t], kv, rows, scale, sink, d_qk)
        dP = dO[t] @ kv[rows, :d_v].T                    # [H, K_t]
        delta[i] = (p * dP).sum(axis=1)
    return delta


def oracle_dsink(q, kv, dO, topk_idxs, topk_length, attn_sink, scale, d_v, delta_from="fp64",
                 tokens=None):
    """d_sink[h] = -sum_t p_sink[t,h] * Delta[t,h] on its own.

    The sink gradient of oracle_bwd (the same passages: [cuDNN-FE #785]
    Testing for the limit -sum(dP_sum) at p_sink = 1, Not addressed for
    Delta), without the dQ and dKV products, so that it can run over every
    token of a large problem: per token the probabilities, O = P V, Delta =
    dO . O (O rounded to bf16 first for ``delta_from="bf16"``) and the
    token's term.  Empty rows add nothing.  Returns d_sink [H] (None without
    a sink).
    """
    if delta_from not in ("fp64", "bf16"):
        raise ValueError(delta_from)
    if attn_sink is None:
        return None
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    T, H, d_qk = q.shape
    S_kv = kv.shape[0]
    sink = np.asarray(attn_sink, dtype=np.float64)
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    d_sink = np.zeros(H)
    for t in toks:
        ln = None if topk_length is None else topk_length[t]
        _, rows = valid_slots(topk_idxs[t], ln, S_kv)
        if rows.size == 0:
            continue
        _, lse_cols, _, p = _token_probs(q[t], kv, rows, scale, sink, d_qk)
        o_t = p @ kv[rows, :d_v]
        if delta_from == "bf16":
            o_t = round_to_bf16(o_t)
        dl = (dO[t] * o_t).sum(axis=1)
        d_sink -= p_sink(lse_cols, sink) * dl
    return d_sink
