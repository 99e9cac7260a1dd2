"""Seeded synthetic problems for sparse top-k MLA attention.

This module only draws inputs: random tensors, index lists and lengths.  It
holds none of the attention arithmetic, and both the GPU library's callers and
the CPU oracle consume the same bit patterns from it.

Recipe (fixed generation order per problem): q, kv, dO as fp32 N(0, 1) from
``numpy.random.default_rng(seed)`` rounded to bf16 (round to nearest even, by
torch), then the sink (fp32 N(0, 1)), then the indices.  Index lists are int32
in sampled (unsorted) order.

Shapes follow the workloads of the pages: DeepSeek-V4-like sliding window of
128 recent positions followed by causal top-k slots, -1 padded
([flash-attn #2882] Performance at DeepSeek-V4 shapes; the [window | compressed]
slot order of [cuDNN-FE #298]); compact layouts with a length per token and
non-compact layouts wider than S_kv ([cuDNN-FE #785] Testing; [cuDNN-FE #298]);
saturating sinks ([cuDNN-FE #785] Summary 3).  They stand in for the indexer
output of a trained model, which is not available.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

__all__ = ["Problem", "make_problem", "make_batched", "make_degenerate", "make_block_gaps",
           "pack_live_blocks", "segment", "make_spiky", "head_slice", "PROBLEMS", "EDGE_HEADS",
           "EXTRA_HEADS", "DEGENERATE_KINDS"]

EDGE_HEADS = (1, 24, 64, 96, 128)
# head counts that leave the last group of 32 heads partly filled (the pages'
# in-kernel padding validation set includes 72, 100 and 120)
EXTRA_HEADS = (72, 80, 90, 100, 120)


def _edge_seed(base, H):
    """Seed of an edge-suite problem: base + position of H in EDGE_HEADS, or
    base + 5 + position in EXTRA_HEADS."""
    if H in EDGE_HEADS:
        return base + EDGE_HEADS.index(H)
    return base + len(EDGE_HEADS) + EXTRA_HEADS.index(H)


@dataclass
class Problem:
    name: str
    T: int
    S_kv: int
    H: int
    d_qk: int
    d_v: int
    W: int
    scale: float
    q: torch.Tensor                      # bf16 [T, H, d_qk] (CPU)
    kv: torch.Tensor                     # bf16 [S_kv, d_qk]
    dO: torch.Tensor                     # bf16 [T, H, d_v]
    topk_idxs: torch.Tensor              # int32 [T, W]
    topk_length: Optional[torch.Tensor]  # int32 [T] or None
    attn_sink: Optional[torch.Tensor]    # fp32 [H] or None
    meta: dict = field(default_factory=dict)

    # fp64 NumPy views of the exact values, for the oracle
    def np_inputs(self):
        return dict(
            q=self.q.double().numpy(),
            kv=self.kv.double().numpy(),
            dO=self.dO.double().numpy(),
            topk_idxs=self.topk_idxs.numpy(),
            topk_length=None if self.topk_length is None else self.topk_length.numpy(),
            attn_sink=None if self.attn_sink is None else self.attn_sink.double().numpy(),
            scale=self.scale,
            d_v=self.d_v,
        )

    def valid_count(self) -> int:
        """Number of valid (token, slot) pairs (the FLOP convention's K summed)."""
        idx = self.topk_idxs.numpy()
        ok = (idx >= 0) & (idx < self.S_kv)
        if self.topk_length is not None:
            ln = np.clip(self.topk_length.numpy().astype(np.int64), 0, self.W)
            ok &= np.arange(self.W)[None, :] < ln[:, None]
        return int(ok.sum())


def _bf16(rng, shape):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(a).to(torch.bfloat16)


def _dense(rng, T, S_kv, H, d_qk, d_v, with_sink):
    q = _bf16(rng, (T, H, d_qk))
    kv = _bf16(rng, (S_kv, d_qk))
    dO = _bf16(rng, (T, H, d_v))
    sink = None
    if with_sink:
        sink = torch.from_numpy(rng.standard_normal(size=(H,), dtype=np.float32))
    return q, kv, dO, sink


def _causal_tiny_idxs(rng, T, W):
    """Row t: min(W, t+1) distinct indices drawn from [0, t], then -1."""
    idx = np.full((T, W), -1, dtype=np.int32)
    for t in range(T):
        n = min(W, t + 1)
        idx[t, :n] = rng.choice(t + 1, size=n, replace=False)
    return idx


def _window_topk_idxs(rng, T, window, topk):
    """[window | top-k] rows: slots [0, window) hold max(0,t-window+1)..t
    ascending then -1; slots [window, window+topk) hold min(topk, t-window+1)
    distinct indices from [0, t-window] (the causal prefix before the window),
    then -1."""
    W = window + topk
    idx = np.full((T, W), -1, dtype=np.int32)
    for t in range(T):
        lo = max(0, t - window + 1)
        idx[t, : t - lo + 1] = np.arange(lo, t + 1, dtype=np.int32)
        n_before = lo  # positions 0 .. lo-1 lie before the window
        k = min(topk, n_before)
        if k > 0:
            idx[t, window: window + k] = rng.choice(n_before, size=k, replace=False)
    return idx


def make_tiny(seed=0, sink=True, compact=False):
    """T=64, S_kv=64 causal, H=4, d_qk=576, d_v=512, width 32, scale 1/sqrt(576)."""
    rng = np.random.default_rng(seed)
    T, S, H, dqk, dv, W = 64, 64, 4, 576, 512, 32
    q, kv, dO, s = _dense(rng, T, S, H, dqk, dv, sink)
    idx = _causal_tiny_idxs(rng, T, W)
    length = None
    if compact:
        length = torch.from_numpy((idx >= 0).sum(axis=1).astype(np.int32))
    return Problem("tiny", T, S, H, dqk, dv, W, 1.0 / math.sqrt(dqk), q, kv, dO,
                   torch.from_numpy(idx), length, s,
                   meta=dict(seed=seed, compact=compact, sink=sink))


def make_edge_compact(H, seed=None):
    """Compact layout: T=128, S_kv=128, width 64, length ~ U{0..64} with 10% of
    rows forced to 0; slots < length hold distinct indices from [0,128); the
    tail holds random in-range indices that must be ignored by position."""
    if seed is None:
        seed = _edge_seed(10, H)
    rng = np.random.default_rng(seed)
    T, S, dqk, dv, W = 128, 128, 576, 512, 64
    q, kv, dO, s = _dense(rng, T, S, H, dqk, dv, True)
    length = rng.integers(0, W + 1, size=T).astype(np.int32)
    zero = rng.random(T) < 0.10
    length[zero] = 0
    length[0] = 0          # at least one empty row, next to a full one
    length[1] = W
    idx = rng.integers(0, S, size=(T, W)).astype(np.int32)   # tail: in-range garbage
    for t in range(T):
        n = int(length[t])
        idx[t, :n] = rng.choice(S, size=n, replace=False)
    return Problem(f"edge_compact_h{H}", T, S, H, dqk, dv, W, 1.0 / math.sqrt(dqk),
                   q, kv, dO, torch.from_numpy(idx), torch.from_numpy(length), s,
                   meta=dict(seed=seed))


def make_edge_wide(H, seed=None, T=128, S=256, W=1024):
    """Non-compact layout wider than S_kv: W=1024 > S_kv=256; n_valid[t] ~
    U{0..256} distinct indices at random slot positions, -1 elsewhere; one row
    with 0 valid and one with 256.  No sink."""
    if seed is None:
        seed = _edge_seed(20, H)
    rng = np.random.default_rng(seed)
    dqk, dv = 576, 512
    q, kv, dO, s = _dense(rng, T, S, H, dqk, dv, False)
    nval = rng.integers(0, S + 1, size=T)
    nval[0] = 0
    nval[1] = S
    idx = np.full((T, W), -1, dtype=np.int32)
    for t in range(T):
        n = int(nval[t])
        pos = rng.choice(W, size=n, replace=False)
        idx[t, pos] = rng.choice(S, size=n, replace=False)
    return Problem(f"edge_wide_h{H}", T, S, H, dqk, dv, W, 1.0 / math.sqrt(dqk),
                   q, kv, dO, torch.from_numpy(idx), None, s, meta=dict(seed=seed))


def make_edge_width118(H, seed=40, T=64, S=128):
    """Non-compact width 118 = 100 valid indices at random positions + 18 -1
    entries per row (a 54-slot partial last block, [cuDNN-FE #785] review)."""
    rng = np.random.default_rng(seed)
    W, dqk, dv = 118, 576, 512
    q, kv, dO, s = _dense(rng, T, S, H, dqk, dv, True)
    idx = np.full((T, W), -1, dtype=np.int32)
    for t in range(T):
        pos = rng.choice(W, size=100, replace=False)
        idx[t, pos] = rng.choice(S, size=100, replace=False)
    return Problem(f"edge_w118_h{H}", T, S, H, dqk, dv, W, 1.0 / math.sqrt(dqk), q, kv, dO,
                   torch.from_numpy(idx), None, s, meta=dict(seed=seed))


def make_deep_rows(T, seed=130, S=8, H=16, W=512):
    """Every slot of every token names one of a few KV rows (drawn with
    replacement from S = 8 rows, non-compact, with a sink): each row's list
    holds about T * W / S entries, cut into several reduce parts, and a token
    names each row dozens of times."""
    rng = np.random.default_rng(seed + T)
    dqk, dv = 576, 512
    q, kv, dO, s = _dense(rng, T, S, H, dqk, dv, True)
    idx = rng.integers(0, S, size=(T, W)).astype(np.int32)
    return Problem(f"deep_rows_T{T}", T, S, H, dqk, dv, W, 1.0 / math.sqrt(dqk), q, kv, dO,
                   torch.from_numpy(idx), None, s, meta=dict(seed=seed + T))


DEGENERATE_KINDS = ("single", "all_invalid", "out_of_range", "duplicates")


def make_degenerate(kind, seed=80):
    """Small problems at the edges of the argument contract, with a sink.

    single        T = S_kv = H = W = 1, d_qk = d_v = 512: one token whose one
                  slot names the one KV row
    all_invalid   T = 5, S_kv = 8, H = 3, width 70 (a full and a 6-slot
                  block), every slot -1: every row is empty
    out_of_range  T = 16, S_kv = 40, H = 8, width 96: per row 20 distinct
                  valid indices, 20 indices in [S_kv, S_kv + 1000), 20 below -1
                  and -1 elsewhere, at random positions (only the valid ones
                  name a row)
    duplicates    T = 16, S_kv = 50, H = 8, width 64: per row 40 slots drawn
                  with replacement from [0, 50) (so rows repeat), -1 after;
                  a row named twice by one token counts twice, as the
                  slot-wise definition gives
    """
    rng = np.random.default_rng(seed + DEGENERATE_KINDS.index(kind))
    if kind == "single":
        T, S, H, dqk, dv, W = 1, 1, 1, 512, 512, 1
        q, kv, dO, s = _dense(rng, T, S, H, dqk, dv, True)
        idx = np.zeros((T, W), dtype=np.int32)
    elif kind == "all_invalid":
        T, S, H, dqk, dv, W = 5, 8, 3, 576, 512, 70
        q, kv, dO, s = _dense(rng, T, S, H, dqk, dv, True)
        idx = np.full((T, W), -1, dtype=np.int32)
    elif kind == "out_of_range":
        T, S, H, dqk, dv, W = 16, 40, 8, 576, 512, 96
        q, kv, dO, s = _dense(rng, T, S, H, dqk, dv, True)
        idx = np.full((T, W), -1, dtype=np.int32)
        for t in range(T):
            pos = rng.permutation(W)
            idx[t, pos[:20]] = rng.choice(S, size=20, replace=False)
            idx[t, pos[20:40]] = rng.integers(S, S + 1000, size=20)
            idx[t, pos[40:60]] = rng.integers(-(2 ** 31), -1, size=20)
    elif kind == "duplicates":
        T, S, H, dqk, dv, W = 16, 50, 8, 576, 512, 64
        q, kv, dO, s = _dense(rng, T, S, H, dqk, dv, True)
        idx = np.full((T, W), -1, dtype=np.int32)
        idx[:, :40] = rng.integers(0, S, size=(T, 40))
    else:
        raise ValueError(f"unknown degenerate problem {kind!r}")
    return Problem(f"degenerate_{kind}", T, S, H, dqk, dv, W, 1.0 / math.sqrt(dqk), q, kv, dO,
                   torch.from_numpy(idx), None, s, meta=dict(seed=seed, kind=kind))


def make_block_gaps(H=64, seed=90, T=96, S=200, nblocks=8):
    """Non-compact rows of nblocks 64-slot blocks, each block either all -1
    or live: per token a random set of 0..4 live blocks anywhere in the row
    (so whole blocks of padding sit before, between and after them), each
    live block with 1..64 valid slots at random positions (-1 elsewhere);
    a token's indices are distinct."""
    rng = np.random.default_rng(seed)
    dqk, dv, W = 576, 512, 64 * nblocks
    q, kv, dO, s = _dense(rng, T, S, H, dqk, dv, True)
    idx = np.full((T, W), -1, dtype=np.int32)
    for t in range(T):
        live = rng.choice(nblocks, size=int(rng.integers(0, 5)), replace=False)
        cnt = [int(rng.integers(1, 65)) for _ in live]
        rows = rng.choice(S, size=sum(cnt), replace=False)
        k = 0
        for b, c in zip(live, cnt):
            pos = 64 * int(b) + rng.choice(64, size=c, replace=False)
            idx[t, pos] = rows[k:k + c]
            k += c
    return Problem(f"block_gaps_h{H}", T, S, H, dqk, dv, W, 1.0 / math.sqrt(dqk), q, kv, dO,
                   torch.from_numpy(idx), None, s, meta=dict(seed=seed))


def pack_live_blocks(p):
    """The same problem with each token's blocks that hold a valid slot moved,
    in order and unchanged, to the front of its row (the rest all -1)."""
    idx = p.topk_idxs.numpy()
    T, W = idx.shape
    out = np.full_like(idx, -1)
    for t in range(T):
        blocks = [idx[t, j:j + 64] for j in range(0, W, 64)]
        live = [b for b in blocks if ((b >= 0) & (b < p.S_kv)).any()]
        for i, b in enumerate(live):
            out[t, 64 * i: 64 * i + b.size] = b
    return Problem(p.name + "_packed", p.T, p.S_kv, p.H, p.d_qk, p.d_v, p.W, p.scale, p.q, p.kv, p.dO,
                   torch.from_numpy(out), None, p.attn_sink, meta=dict(p.meta, packed=True))


SATURATING_SINKS = (3.0e38, -3.0e38, float("inf"), float("-inf"))


def make_edge_sink(H, seed=None, sink_cycle_offset=0):
    """Saturating sinks: T=128, S_kv=128, width 64, causal non-compact;
    sink[h] = (+3e38, -3e38, +inf, -inf)[(h + offset) mod 4].  Every 4th token
    (t % 4 == 0) has q scaled by 1e-3; tokens t % 4 == 1 are anti-aligned with
    their gathered rows so that their scores (and LSE) are strongly negative:
    q[t,h] = -g * m / |m| with m the sum of the token's gathered kv rows and g
    chosen so that the largest score is -100 (rows whose projections are not
    all positive are redrawn)."""
    if seed is None:
        seed = _edge_seed(30, H)
    rng = np.random.default_rng(seed)
    T, S, dqk, dv, W = 128, 128, 576, 512, 64
    scale = 1.0 / math.sqrt(dqk)
    q32 = rng.standard_normal(size=(T, H, dqk), dtype=np.float32)
    kv = _bf16(rng, (S, dqk))
    dO = _bf16(rng, (T, H, dv))
    sink = torch.tensor([SATURATING_SINKS[(h + sink_cycle_offset) % 4] for h in range(H)],
                        dtype=torch.float32)
    idx = _causal_tiny_idxs(rng, T, W)
    kvf = kv.double().numpy()
    anti = []
    for t in range(T):
        if t % 4 == 0:
            q32[t] *= np.float32(1e-3)
        elif t % 4 == 1:
            for _attempt in range(100):
                rows = idx[t][idx[t] >= 0]
                m = kvf[rows].sum(axis=0)
                mhat = m / np.linalg.norm(m)
                proj = kvf[rows] @ mhat
                if proj.min() > 0:
                    break
                # redraw this row's index set
                n = rows.size
                idx[t] = -1
                idx[t, :n] = rng.choice(t + 1, size=n, replace=False)
            else:
                continue
            g = 100.0 / (scale * proj.min())
            q32[t, :, :] = (-g * mhat).astype(np.float32)
            anti.append(t)
    q = torch.from_numpy(q32).to(torch.bfloat16)
    return Problem(f"edge_sink_h{H}_o{sink_cycle_offset}", T, S, H, dqk, dv, W, scale,
                   q, kv, dO, torch.from_numpy(idx), None, sink,
                   meta=dict(seed=seed, anti_aligned_tokens=anti))


def make_dsv4(T, H, d_qk, d_v, topk, seed, window=128, sink=True, compact=False,
              scale=None, name=None):
    """DeepSeek-V4-like: S_kv = T causal, window 128 + top-k distinct causal
    indices from before the window, -1 padded; fp32 sink N(0,1).  ``compact``
    packs the same index sets to the front with a length per token."""
    rng = np.random.default_rng(seed)
    q, kv, dO, s = _dense(rng, T, T, H, d_qk, d_v, sink)
    idx = _window_topk_idxs(rng, T, window, topk)
    length = None
    if compact:
        valid = idx >= 0
        length = valid.sum(axis=1).astype(np.int32)
        packed = np.full_like(idx, -1)
        for t in range(T):
            packed[t, : length[t]] = idx[t][valid[t]]
        idx = packed
        length = torch.from_numpy(length)
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    return Problem(name or f"dsv4_T{T}_H{H}_d{d_qk}_k{topk}", T, T, H, d_qk, d_v,
                   window + topk, scale, q, kv, dO, torch.from_numpy(idx), length, s,
                   meta=dict(seed=seed, window=window, topk=topk, compact=compact))


def make_batched(H=64, lengths=(300, 77, 650), window=64, topk=128, d_qk=576, d_v=512, seed=70,
                 compact=False):
    """Several sequences packed into one problem (the varlen / batched case):
    the tokens and KV rows of the sequences are concatenated and every index
    is global.  Each sequence has S_kv = its length, causal [window | top-k]
    rows of its own (the dsv4 recipe at a smaller window and top-k), shifted
    by the sequence's first KV row; -1 stays -1.  ``meta["segments"]`` holds
    the [start, end) token (and KV row) range of each sequence."""
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    q, kv, dO, s = _dense(rng, T, T, H, d_qk, d_v, True)
    W = window + topk
    idx = np.full((T, W), -1, dtype=np.int32)
    segs, t0 = [], 0
    for n in lengths:
        part = _window_topk_idxs(rng, n, window, topk)
        idx[t0:t0 + n] = np.where(part >= 0, part + t0, -1)
        segs.append((t0, t0 + n))
        t0 += n
    length = None
    if compact:
        valid = idx >= 0
        ln = valid.sum(axis=1).astype(np.int32)
        packed = np.full_like(idx, -1)
        for t in range(T):
            packed[t, : ln[t]] = idx[t][valid[t]]
        idx, length = packed, torch.from_numpy(ln)
    return Problem(f"batched_H{H}_{'_'.join(map(str, lengths))}", T, T, H, d_qk, d_v, W,
                   1.0 / math.sqrt(d_qk), q, kv, dO, torch.from_numpy(idx), length, s,
                   meta=dict(seed=seed, segments=segs, window=window, topk=topk, compact=compact))


def segment(p: Problem, i: int) -> Problem:
    """Sequence i of a batched problem as a problem of its own (local indices)."""
    a, b = p.meta["segments"][i]
    idx = p.topk_idxs[a:b].clone()
    idx = torch.where(idx >= 0, idx - a, idx)
    return Problem(f"{p.name}_seg{i}", b - a, b - a, p.H, p.d_qk, p.d_v, p.W, p.scale,
                   p.q[a:b].clone(), p.kv[a:b].clone(), p.dO[a:b].clone(), idx,
                   None if p.topk_length is None else p.topk_length[a:b].clone(),
                   p.attn_sink, meta=dict(parent=p.name, segment=i))


def make_spiky(H, d_qk=576, seed=100, T=256, window=64, topk=128, frac=0.25, d_v=512,
               spike=(80.0, 120.0)):
    """DeepSeek-V4-like rows (window, then causal top-k; [window | top-k]
    order) where some tokens hold one KV row whose score rises far above
    everything in the token's first 64-slot block.

    For a fraction ``frac`` of the tokens that have top-k slots past the
    first block, one top-k slot j >= 64 is picked and its row r = idx[t, j];
    for every other head h of that token q[t, h] is replaced by
    g_h * kv[r] / |kv[r]| + 0.25 N(0, 1) with g_h drawn so that the score
    scale * <q[t, h], kv[r]> lands near a value drawn from ``spike`` (in
    nats), i.e. 60-100 nats above the N(0, 1)-scale scores of the first
    block.  A further set of tokens (the same count) gets the spike in the
    first block instead (window slot 0), which makes every later score tiny
    next to it.  meta["late_spike"] / meta["early_spike"] list the tokens."""
    rng = np.random.default_rng(seed)
    q32 = rng.standard_normal(size=(T, H, d_qk), dtype=np.float32)
    kv = _bf16(rng, (T, d_qk))
    dO = _bf16(rng, (T, H, d_v))
    sink = torch.from_numpy(rng.standard_normal(size=(H,), dtype=np.float32))
    idx = _window_topk_idxs(rng, T, window, topk)
    scale = 1.0 / math.sqrt(d_qk)
    kvf = kv.double().numpy()
    cand = np.nonzero((idx[:, 64:] >= 0).any(axis=1))[0]
    n = max(1, int(round(frac * cand.size)))
    picked = rng.choice(cand, size=min(2 * n, cand.size), replace=False)
    late, early = sorted(int(t) for t in picked[:n]), sorted(int(t) for t in picked[n:])
    for t in late + early:
        if t in late:
            slots = np.nonzero(idx[t, 64:] >= 0)[0] + 64
            j = int(rng.choice(slots))
        else:
            j = 0
        r = int(idx[t, j])
        u = kvf[r] / np.linalg.norm(kvf[r])
        for h in range(0, H, 2):
            target = rng.uniform(*spike)
            g = target / (scale * np.linalg.norm(kvf[r]))
            q32[t, h] = (g * u + 0.25 * rng.standard_normal(d_qk)).astype(np.float32)
    q = torch.from_numpy(q32).to(torch.bfloat16)
    return Problem(f"spiky_h{H}_d{d_qk}", T, T, H, d_qk, d_v, window + topk, scale, q, kv, dO,
                   torch.from_numpy(idx), None, sink,
                   meta=dict(seed=seed, window=window, topk=topk, late_spike=late, early_spike=early))


def head_slice(p: Problem, H: int) -> Problem:
    """The first H heads of a problem (q, dO and the sink sliced)."""
    return Problem(f"{p.name}_heads{H}", p.T, p.S_kv, H, p.d_qk, p.d_v, p.W, p.scale,
                   p.q[:, :H].clone(), p.kv, p.dO[:, :H].clone(), p.topk_idxs, p.topk_length,
                   None if p.attn_sink is None else p.attn_sink[:H].clone(),
                   meta=dict(p.meta, head_slice=H))


def with_zero_dO_past(p: Problem, H: int) -> Problem:
    """The same problem with dO = 0 for every head h >= H."""
    dO = p.dO.clone()
    dO[:, H:] = 0
    return Problem(p.name + f"_dO0from{H}", p.T, p.S_kv, p.H, p.d_qk, p.d_v, p.W, p.scale, p.q, p.kv,
                   dO, p.topk_idxs, p.topk_length, p.attn_sink, meta=dict(p.meta, dO_zero_from=H))


def make_spiky_dsv4(T=4096, H=128, d_qk=576, topk=512, seed=2, frac=0.10, name=None):
    """The DeepSeek-V4-like problem of the same seed (make_dsv4) where a
    fraction ``frac`` of the tokens that have top-k slots past the first
    block get a late score spike as in make_spiky (every other head's query
    aligned with one of the token's top-k rows, 80-120 nats)."""
    p = make_dsv4(T, H, d_qk, 512, topk, seed=seed)
    rng = np.random.default_rng(seed + 1000)
    idx = p.topk_idxs.numpy()
    q32 = p.q.float().numpy().copy()
    kvf = p.kv.double().numpy()
    cand = np.nonzero((idx[:, 64:] >= 0).any(axis=1))[0]
    late = sorted(int(t) for t in rng.choice(cand, size=int(round(frac * cand.size)), replace=False))
    for t in late:
        slots = np.nonzero(idx[t, 64:] >= 0)[0] + 64
        r = int(idx[t, int(rng.choice(slots))])
        u = kvf[r] / np.linalg.norm(kvf[r])
        g = rng.uniform(80.0, 120.0, size=(H + 1) // 2) / (p.scale * np.linalg.norm(kvf[r]))
        q32[t, 0::2] = (g[:, None] * u[None, :] +
                        0.25 * rng.standard_normal((g.size, d_qk))).astype(np.float32)
    q = torch.from_numpy(q32).to(torch.bfloat16)
    return Problem(name or f"{p.name}_spiky", p.T, p.S_kv, H, d_qk, 512, p.W, p.scale, q, p.kv, p.dO,
                   p.topk_idxs, None, p.attn_sink, meta=dict(p.meta, late_spike=late))


def make_decode(T, S_kv=16384, H=128, d_qk=576, topk=1024, window=128, seed=110, name=None, scale=None):
    """Few query tokens at the end of a long KV set (decode, or a short
    prefill chunk): query i sits at position S_kv - T + i and holds the
    DeepSeek-V4-like [window | top-k] row of that position (the window of
    the <= 128 latest positions, then top-k distinct positions from before
    the window), -1 padded.  d_v = 512, fp32 sink N(0, 1); scale
    1/sqrt(d_qk) unless given."""
    rng = np.random.default_rng(seed)
    q, kv, dO, s = _dense(rng, T, S_kv, H, d_qk, 512, True)
    W = window + topk
    idx = np.full((T, W), -1, dtype=np.int32)
    for i in range(T):
        pos = S_kv - T + i
        lo = max(0, pos - window + 1)
        idx[i, : pos - lo + 1] = np.arange(lo, pos + 1, dtype=np.int32)
        k = min(topk, lo)
        if k > 0:
            idx[i, window: window + k] = rng.choice(lo, size=k, replace=False)
    return Problem(name or f"decode_T{T}_S{S_kv}_H{H}_k{topk}", T, S_kv, H, d_qk, 512, W,
                   1.0 / math.sqrt(d_qk) if scale is None else scale, q, kv, dO, torch.from_numpy(idx), None, s,
                   meta=dict(seed=seed, window=window, topk=topk))


def make_random(seed):
    """A small problem with every size and index property drawn at random
    (seeded): T in [1, 300], S_kv in [1, 2000], H in [1, 128], d_qk 512 or
    576, W in [1, 1500], compact or non-compact layout, no sink, a finite
    sink or saturating ones, rows whose valid slots sit anywhere among -1,
    indices >= S_kv and below -1, some rows empty and some with duplicate
    indices.  meta["ws_tokens"]: a workspace size (in tokens) to run the
    backward with, sometimes smaller than T (token chunks)."""
    rng = np.random.default_rng(10_000 + seed)
    T = int(rng.integers(1, 301))
    S = int(rng.integers(1, 2001))
    H = int(rng.choice([1, 2, 7, 16, 23, 32, 33, 48, 64, 65, 80, 96, 100, 127, 128]))
    dqk = int(rng.choice([512, 576]))
    W = int(rng.integers(1, 1501))
    compact = bool(rng.random() < 0.4)
    sink_kind = rng.choice(["none", "finite", "finite", "saturating"])
    q, kv, dO, _ = _dense(rng, T, S, H, dqk, 512, False)
    sink = None
    if sink_kind == "finite":
        sink = torch.from_numpy(rng.standard_normal(size=(H,), dtype=np.float32))
    elif sink_kind == "saturating":
        sink = torch.tensor([SATURATING_SINKS[h % 4] if h % 3 == 0 else float(rng.standard_normal())
                             for h in range(H)], dtype=torch.float32)
    idx = np.full((T, W), -1, dtype=np.int32)
    length = np.zeros(T, dtype=np.int32) if compact else None
    for t in range(T):
        if rng.random() < 0.05:
            continue                                   # empty row
        n = int(rng.integers(1, min(W, S) + 1))
        rows = rng.choice(S, size=n, replace=bool(rng.random() < 0.1)).astype(np.int32)
        if compact:
            length[t] = n + int(rng.integers(0, 3)) if rng.random() < 0.1 else n
            idx[t, :n] = rows
            idx[t, n:] = rng.integers(-5, S + 5, size=W - n)   # tail: ignored by position
        else:
            pos = rng.choice(W, size=n, replace=False)
            idx[t, pos] = rows
            bad = rng.random(W) < 0.03                 # out-of-range values among the padding
            idx[t, bad & (idx[t] < 0)] = rng.integers(S, S + 100, size=int((bad & (idx[t] < 0)).sum()))
    ws_tokens = T if rng.random() < 0.7 else int(rng.integers(1, T + 1))
    return Problem(f"random_{seed}", T, S, H, dqk, 512, W, 1.0 / math.sqrt(dqk), q, kv, dO,
                   torch.from_numpy(idx), None if length is None else torch.from_numpy(length), sink,
                   meta=dict(seed=seed, ws_tokens=ws_tokens, sink_kind=str(sink_kind)))


def make_problem(name: str, **kw) -> Problem:
    return PROBLEMS[name](**kw)


# The five workloads: tiny, the edge suite, and three DeepSeek-V4-like shapes.
PROBLEMS = {
    "tiny": make_tiny,
    "edge_compact": make_edge_compact,
    "edge_wide": make_edge_wide,
    "edge_sink": make_edge_sink,
    "batched": make_batched,
    "dsv4_flash_h64": lambda **kw: make_dsv4(4096, 64, 512, 512, 512, seed=1,
                                             name="dsv4_flash_h64_T4096", **kw),
    "dsv4_flash_h128": lambda **kw: make_dsv4(4096, 128, 576, 512, 512, seed=2,
                                              name="dsv4_flash_h128_T4096", **kw),
    "dsv4_pro": lambda **kw: make_dsv4(16384, 128, 512, 512, 1024, seed=3,
                                       name="dsv4_pro_h128_T16384", **kw),
    # the grid of the pages' DeepSeek-V4 timing table (D_qk = D_v = 512 in every row):
    # flash H=64 and H=128 (top-k 512), pro H=128 (top-k 1024), T = 4096 / 8192 / 16384
    **{f"grid_flash_h64_T{T}": (lambda T: lambda **kw: make_dsv4(T, 64, 512, 512, 512, seed=40 + T // 4096,
                                                                  name=f"grid_flash_h64_T{T}", **kw))(T)
       for T in (4096, 8192, 16384)},
    **{f"grid_flash_h128_T{T}": (lambda T: lambda **kw: make_dsv4(T, 128, 512, 512, 512, seed=50 + T // 4096,
                                                                   name=f"grid_flash_h128_T{T}", **kw))(T)
       for T in (4096, 8192, 16384)},
    **{f"grid_pro_h128_T{T}": (lambda T: lambda **kw: make_dsv4(T, 128, 512, 512, 1024, seed=60 + T // 4096,
                                                                 name=f"grid_pro_h128_T{T}", **kw))(T)
       for T in (4096, 8192, 16384)},
    # the pages' T = 2048 comparison (flash H = 64 / H = 128, top-k 512, D = 512)
    "grid_flash_h64_T2048": lambda **kw: make_dsv4(2048, 64, 512, 512, 512, seed=45,
                                                   name="grid_flash_h64_T2048", **kw),
    "grid_flash_h128_T2048": lambda **kw: make_dsv4(2048, 128, 512, 512, 512, seed=55,
                                                    name="grid_flash_h128_T2048", **kw),
    # the headline shape at small head counts (the in-kernel head padding of
    # one 16-head MFMA tile)
    **{f"dsv4_flash_h{H}": (lambda H: lambda **kw: make_dsv4(4096, H, 576, 512, 512, seed=80 + H,
                                                             name=f"dsv4_flash_h{H}_T4096", **kw))(H)
       for H in (1, 8, 24)},
    # few queries against a 16384-row KV set (window 128 + top-k 1024)
    **{f"decode_T{T}": (lambda T: lambda **kw: make_decode(T, seed=110 + T, **kw))(T) for T in (1, 16, 64)},
    # the headline with 10 % of its tokens holding a late score spike
    "dsv4_flash_h128_spiky": lambda **kw: make_spiky_dsv4(name="dsv4_flash_h128_T4096_spiky", **kw),
    # the headline's index sets packed to the front with topk_length
    "dsv4_flash_h128_compact": lambda **kw: make_dsv4(4096, 128, 576, 512, 512, seed=2, compact=True,
                                                      name="dsv4_flash_h128_T4096_compact", **kw),
}
