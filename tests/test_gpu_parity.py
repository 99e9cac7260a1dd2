"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small problems are compared element by element on every output.  The three
DeepSeek-V4-like workloads run at their full size in the same launch
configuration as bench.py and are compared on sampled tokens (O, LSE, dQ) and
sampled KV rows (dKV, computed exactly from every token that names the row),
plus identities that hold at any size.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import (compare_full, compare_exact_delta, run_gpu, run_gpu_exact, run_gpu_from_o, run_oracle,
                    oracle_delta_exact, say, check_tensor, check_lse, check_dsink, check_dkv_rows,
                    referenced_rows, tokens_referencing, cosine, to_dev)
from sparse_top_attention_topk_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _dq_close(a, b):
    """dQ of two runs whose backward split the blocks differently (fewer than
    128 tokens per chunk): the same fp32 terms summed in other groups, then
    rounded to bf16, so elements may differ by a bf16 rounding step."""
    m = np.abs(b).max()
    return np.abs(a - b).max() <= 2.0 ** -7 * m and cosine(a, b) >= 0.99999


def _run_and_compare(p, label):
    """The default path against the oracle (Delta from the bf16 O, as the
    kernel forms it) at the full bars, and against the exact-O oracle
    (cosine of dQ and dKV).  In the saturating-sink problems the
    anti-aligned tokens make dS = P (dP - Delta) cancel, so the bf16
    rounding of O reaches dKV beyond that cosine ([cuDNN-FE #785] Not
    addressed: the table of Delta sources); there the exact-Delta backward,
    the page's remedy, is held to the exact-O oracle at the full bars."""
    say(f"[gpu] case {label}: T={p.T} S_kv={p.S_kv} H={p.H} d_qk={p.d_qk} W={p.W} "
        f"compact={p.topk_length is not None} sink={p.attn_sink is not None}")
    gpu = run_gpu(p, DEV)
    ref = run_oracle(p)
    errors = compare_full(gpu, ref)
    ref64 = run_oracle(p, delta_from="fp64")
    if p.meta.get("anti_aligned_tokens"):
        say(f"[gpu] case {label}: exact-Delta backward against the exact-O oracle")
        errors += [f"exact-Delta path: {e}" for e in compare_full(run_gpu_exact(p, DEV), ref64)]
    else:
        compare_exact_delta(gpu, ref64, errors)
    assert not errors, f"{label}: " + "; ".join(errors)
    return gpu, ref


@pytest.mark.parametrize("variant", ["sink", "nosink", "compact"])
def test_tiny(variant):
    p = wl.make_tiny(seed=0, sink=variant != "nosink", compact=variant == "compact")
    _run_and_compare(p, f"tiny-{variant}")


@pytest.mark.parametrize("H", wl.EDGE_HEADS)
def test_edge_compact(H):
    p = wl.make_edge_compact(H)
    gpu, ref = _run_and_compare(p, f"edge-compact-h{H}")
    ln = p.topk_length.numpy()
    empty = np.nonzero(ln == 0)[0]
    assert empty.size > 0
    assert np.all(gpu["o"][empty] == 0) and np.all(np.isneginf(gpu["lse"][empty]))
    assert np.all(gpu["dq"][empty] == 0)


@pytest.mark.parametrize("H", wl.EDGE_HEADS)
def test_edge_wide_noncompact(H):
    p = wl.make_edge_wide(H)
    gpu, ref = _run_and_compare(p, f"edge-wide-h{H}")
    # rows named only at columns >= S_kv still receive dKV
    idx = p.topk_idxs.numpy()
    late = np.unique(idx[:, p.S_kv:][idx[:, p.S_kv:] >= 0])
    assert late.size > 0 and np.all(np.any(gpu["dkv"][late] != 0, axis=1))
    # rows never named (row 0 included when unnamed) are exactly 0
    unnamed = ~referenced_rows(p)
    assert np.all(gpu["dkv"][unnamed] == 0)


@pytest.mark.parametrize("H", wl.EDGE_HEADS)
def test_edge_saturating_sinks(H):
    offsets = range(4) if H == 1 else (0,)
    for off in offsets:
        p = wl.make_edge_sink(H, sink_cycle_offset=off)
        gpu, ref = _run_and_compare(p, f"edge-sink-h{H}-o{off}")
        anti = np.array(p.meta["anti_aligned_tokens"])
        assert ref["lse"][anti].max() < -80        # the case exercises the overflow
        s = p.attn_sink.numpy()
        pos = s > 2.36e38                            # +3e38 and +inf heads take all mass
        assert np.all(gpu["o"][:, pos] == 0) and np.all(gpu["dq"][:, pos] == 0)


@pytest.mark.parametrize("H", (24, 128))
def test_width_118_tail(H):
    """Non-compact width 118 = 100 valid + 18 padding: a partial last block."""
    _run_and_compare(wl.make_edge_width118(H), f"width-118-h{H}")


@pytest.mark.parametrize("H,d_qk", [(48, 576), (128, 576), (64, 512), (96, 512)])
def test_forward_rerun_pass(H, d_qk):
    """Tokens whose scores rise far (60-100 nats) above everything in their
    first 64-slot block: the forward's fixed reference max is exceeded by
    more than its slack, the first pass overflows, and the token is run
    again with the exact maximum.  Other tokens have the spike in the first
    block instead (later probabilities underflow) or none.  Every output is
    compared with the oracle element by element; H <= 64 and H > 64 run the
    two head tilings of the forward."""
    p = wl.make_spiky(H, d_qk=d_qk)
    x = p.np_inputs()
    # the case reaches the rerun: some head's late maximum exceeds the first
    # block's maximum by more than 64 log2 units (44.4 nats)
    rise = []
    for t in p.meta["late_spike"]:
        idx = x["topk_idxs"][t]
        ok = idx >= 0
        s = p.scale * (x["q"][t] @ x["kv"][np.where(ok, idx, 0)].T)
        s[:, ~ok] = -np.inf
        rise.append((s[:, 64:].max(axis=1) - s[:, :64].max(axis=1)).max())
    assert min(rise) > 50.0, min(rise)
    gpu, ref = _run_and_compare(p, f"rerun-h{H}-d{d_qk}")
    for k in ("o", "lse", "dq", "dkv"):
        assert np.all(np.isfinite(gpu[k][p.meta["late_spike"]] if k != "dkv" else gpu[k])), k


@pytest.mark.parametrize("H", wl.EXTRA_HEADS)
@pytest.mark.parametrize("kind", ["compact", "wide", "sink"])
def test_edge_partial_head_groups(kind, H):
    """Head counts whose last group of 32 heads is partly filled (the backward's
    dKV kernel stages rows past H and zeroes their P / dS tiles)."""
    make = {"compact": wl.make_edge_compact, "wide": wl.make_edge_wide, "sink": wl.make_edge_sink}[kind]
    _run_and_compare(make(H), f"edge-{kind}-h{H}")


@pytest.mark.parametrize("H", (72, 96, 120))
def test_d512_partial_head_groups(H):
    """d_qk = d_v = 512 (no rotary columns) at head counts of 3 and 4 groups of
    32 heads, some partly filled."""
    p = wl.make_dsv4(320, H, 512, 512, 96, seed=73 + H, window=64)
    _run_and_compare(p, f"dsv4-512-h{H}")


HEAD_SLICE_H = (1, 8, 16, 24, 48, 64, 72, 96, 100, 120)


def test_head_slice_invariance():
    """In-kernel head padding against a full 128-head run ([flash-attn #2882]
    Validation): the first H heads of a 128-head problem whose heads >= H
    have dO = 0 give, run with H heads, the same O, LSE, dQ, Delta and d_sink
    bits as the 128-head run's first H heads, and the same dKV (the extra
    heads add exact zeros to it)."""
    for H in HEAD_SLICE_H:
        p128 = wl.with_zero_dO_past(wl.make_dsv4(256, 128, 576, 512, 96, seed=74, window=64), H)
        say(f"[gpu] head slice H={H}: 128-head run with dO = 0 past head {H}")
        g128 = run_gpu(p128, DEV)
        say(f"[gpu] head slice H={H}: {H}-head run")
        gh = run_gpu(wl.head_slice(p128, H), DEV)
        for k in ("o", "lse", "dq", "delta", "d_sink"):
            a, b = gh[k], g128[k][..., :H] if k in ("lse", "delta", "d_sink") else g128[k][:, :H]
            assert np.array_equal(a, b), f"H={H}: {k} differs from the 128-head run's first {H} heads"
        d = np.abs(gh["dkv"] - g128["dkv"]).max()
        m = np.abs(g128["dkv"]).max()
        say(f"[gpu] head slice H={H}: dkv max diff {d:.3e} (max {m:.3e})")
        assert d <= 1e-6 * m, f"H={H}: dkv differs by {d:.3e}"


@pytest.mark.parametrize("kind", wl.DEGENERATE_KINDS)
def test_degenerate_problems(kind):
    """Edges of the argument contract: one token with one slot over a one-row
    KV; every slot -1; indices >= S_kv and below -1 among valid ones; KV rows
    named more than once by one token (each naming counts).

    O, LSE, dQ and dKV meet the usual bars.  d_sink is checked through the
    exact Delta against the fp64 oracle (bar 1e-4): with 16 tokens whose
    Delta terms cancel, rounding O to bf16 alone moves the oracle's own
    d_sink by up to 0.9 % of its largest head, which leaves the 1e-2 bar of
    the bf16-O Delta no room for the kernels' rounding.  The default path's
    d_sink must still be -sum_t p_sink Delta of its own LSE and Delta."""
    p = wl.make_degenerate(kind)
    say(f"[gpu] case degenerate-{kind}: T={p.T} S_kv={p.S_kv} H={p.H} d_qk={p.d_qk} W={p.W}")
    gpu = run_gpu(p, DEV)
    ref = run_oracle(p)
    errors = []
    check_tensor("o", gpu["o"], ref["o"], errors)
    check_lse(gpu["lse"], ref["lse"], errors)
    check_tensor("dq", gpu["dq"], ref["dq"], errors)
    check_tensor("dkv", gpu["dkv"], ref["dkv"], errors)
    check_dkv_rows(gpu["dkv"], ref["dkv"], errors)
    # default path: d_sink from its own LSE and Delta (fp64 on the host)
    lse, dl = gpu["lse"].astype(np.float64), gpu["delta"].astype(np.float64)
    sk = p.attn_sink.double().numpy()[None, :]
    ps = np.where(np.isneginf(lse), 0.0, 1.0 / (1.0 + np.exp(-(sk - np.where(np.isneginf(lse), 0.0, lse)))))
    own = -(ps * dl).sum(axis=0)
    scale_h = np.abs(ps * dl).sum(axis=0)         # fp32 summation error is relative to this
    if np.any(np.abs(gpu["d_sink"] - own) > 1e-5 * scale_h + 1e-7):
        errors.append(f"d_sink: {gpu['d_sink']} vs its own -sum p_sink Delta {own}")
    # exact-Delta path against the fp64 oracle
    ge = run_gpu_exact(p, DEV)
    ref64 = run_oracle(p, delta_from="fp64")
    ms = np.abs(ref64["d_sink"]).max()
    es = np.abs(ge["d_sink"] - ref64["d_sink"]).max()
    say(f"[gpu] degenerate-{kind}: exact-Delta d_sink max err {es:.3e} vs max {ms:.3e}")
    if es > EXACT_TOL * ms + 1e-7:
        errors.append(f"exact-Delta d_sink: max err {es:.3e} vs max {ms:.3e}")
    assert not errors, f"degenerate-{kind}: " + "; ".join(errors)
    if kind == "all_invalid":
        assert np.all(gpu["o"] == 0) and np.all(np.isneginf(gpu["lse"]))
        assert np.all(gpu["dq"] == 0) and np.all(gpu["dkv"] == 0) and np.all(gpu["d_sink"] == 0)
    if kind == "out_of_range":
        assert np.all(gpu["dkv"][~referenced_rows(p)] == 0)
    if kind == "single":
        assert np.all(np.isfinite(gpu["lse"])) and np.any(gpu["dkv"] != 0)


@pytest.mark.parametrize("H", (64, 128))
def test_blocks_without_valid_slots_change_no_bit(H):
    """64-slot blocks holding no valid slot, before, between and after the
    live ones, are skipped; they would add exact zeros.  Moving each token's
    live blocks to the front of its row (the same blocks, in order) gives the
    same bits for every output, and the gapped problem meets the oracle."""
    p = wl.make_block_gaps(H)
    _run_and_compare(p, f"block-gaps-h{H}")
    a = run_gpu(p, DEV)
    b = run_gpu(wl.pack_live_blocks(p), DEV)
    for k in ("o", "lse", "dkv", "delta", "d_sink"):
        assert np.array_equal(a[k], b[k]), f"{k} differs between the gapped and packed rows"
    # 96 tokens: the backward splits each row's blocks into ranges, and the
    # live blocks fall into different ranges in the two layouts
    assert _dq_close(a["dq"], b["dq"]), "dq differs between the gapped and packed rows"


def test_nan_prefilled_outputs_fully_written_and_deterministic():
    p = wl.make_edge_compact(64)
    a = run_gpu(p, DEV, nan_prefill=True)
    b = run_gpu(p, DEV, nan_prefill=False)
    for k in ("o", "lse", "dq", "d_sink"):
        assert np.array_equal(a[k], b[k], equal_nan=False), k
    assert np.all(np.isfinite(a["o"])) and np.all(np.isfinite(a["dq"]))


def test_repeated_empty_and_mixed_rows():
    """Repeated launches of the empty-row path (all-empty and mixed rows),
    compared bit for bit across launches ([cuDNN-FE #785] Testing repeats the
    empty-row launch 800 times)."""
    p = wl.make_edge_compact(128)
    p_empty = wl.make_edge_compact(128)
    p_empty.topk_length = torch.zeros_like(p_empty.topk_length)
    ref_m = run_gpu(p, DEV)
    ref_e = run_gpu(p_empty, DEV)
    assert np.all(ref_e["o"] == 0) and np.all(ref_e["dq"] == 0) and np.all(ref_e["dkv"] == 0)
    # 400 rounds of the two problems: 800 launches of each entry point, in one
    # process, stopping at the first launch whose output differs
    for i in range(400):
        for pp, rr in ((p, ref_m), (p_empty, ref_e)):
            g = run_gpu(pp, DEV)
            for k in ("o", "lse", "dq", "dkv", "d_sink"):
                assert np.array_equal(g[k], rr[k]), f"launch {i}: {k} differs"


@pytest.mark.parametrize("compact", [False, True])
def test_batched_sequences(compact):
    """Three sequences packed with global indices: parity with the oracle, and
    each sequence's O, LSE, dQ and dKV rows are the bits of that sequence run
    alone (the same slots in the same order); d_sink is the sum over them."""
    p = wl.make_batched(compact=compact)
    gpu, ref = _run_and_compare(p, f"batched-compact{int(compact)}")
    ds_sum = np.zeros_like(gpu["d_sink"])
    for i, (a, b) in enumerate(p.meta["segments"]):
        g = run_gpu(wl.segment(p, i), DEV)
        for k in ("o", "lse", "dkv"):
            assert np.array_equal(gpu[k][a:b], g[k]), f"segment {i}: {k} differs"
        # a sequence of fewer than 128 tokens run alone splits its blocks
        # (the batch does not): dQ then sums its terms in other groups
        if b - a >= 128:
            assert np.array_equal(gpu["dq"][a:b], g["dq"]), f"segment {i}: dq differs"
        else:
            assert _dq_close(gpu["dq"][a:b], g["dq"]), f"segment {i}: dq differs"
        ds_sum += g["d_sink"]
    np.testing.assert_allclose(gpu["d_sink"], ds_sum, rtol=1e-5, atol=1e-5)


# ---------------------------------------------------------------------------
# the backward in token chunks (workspace smaller than all tokens need)
# ---------------------------------------------------------------------------
CHUNK_CASES = {
    "edge-compact-h24-c1": (lambda: wl.make_edge_compact(24), 1),
    "edge-wide-h128-c7": (lambda: wl.make_edge_wide(128), 7),
    "edge-sink-h90-c40": (lambda: wl.make_edge_sink(90), 40),
    "batched-c100": (lambda: wl.make_batched(), 100),
    "dsv4-512-h96-c64": (lambda: wl.make_dsv4(320, 96, 512, 512, 96, seed=76, window=64), 64),
}


@pytest.mark.parametrize("name", list(CHUNK_CASES))
def test_chunked_backward(name):
    """A workspace that holds only some tokens makes the backward run chunk by
    chunk (index inversion, S/dP, dQ, dKV partials and reduce per chunk,
    dKV accumulated over the chunks in token order; chunks of fewer than 128
    tokens also split each row's blocks).  The outputs meet the oracle; O,
    LSE, Delta and d_sink are the bits of the one-chunk run, dKV and dQ differ
    from it only by the summation grouping."""
    make, C = CHUNK_CASES[name]
    p = make()
    say(f"[gpu] chunked {name}: T={p.T} S_kv={p.S_kv} H={p.H} W={p.W}, workspace of {C} tokens")
    g = run_gpu(p, DEV, ws_tokens=C)
    errors = compare_full(g, run_oracle(p))
    one = run_gpu(p, DEV)
    for k in ("o", "lse", "delta", "d_sink"):
        if g[k] is not None and not np.array_equal(g[k], one[k]):
            errors.append(f"{k} differs from the one-chunk run")
    if not _dq_close(g["dq"], one["dq"]):
        errors.append("dq differs from the one-chunk run beyond a bf16 rounding step")
    m = np.abs(one["dkv"]).max()
    e = np.abs(g["dkv"] - one["dkv"]).max()
    say(f"[gpu] chunked {name}: dkv vs one chunk max diff {e:.3e} (max {m:.3e})")
    if e > 1e-5 * m:
        errors.append(f"dkv differs from the one-chunk run by {e:.3e}")
    assert not errors, f"{name}: " + "; ".join(errors)


@pytest.mark.parametrize("T", (1, 16, 48))
def test_deep_row_lists(T):
    """A few KV rows named by every slot (each row's list several reduce parts
    long, every token naming each row dozens of times), against the oracle:
    chunks of up to 16 tokens take the one-workgroup index inversion, larger
    ones the five-kernel one (T = 48, and T = 48 run in chunks of 16)."""
    p = wl.make_deep_rows(T)
    say(f"[gpu] deep rows T={T}: S_kv={p.S_kv} H={p.H} W={p.W}")
    ref = run_oracle(p)
    errors = compare_full(run_gpu(p, DEV), ref)
    if T > 16:
        errors += [f"chunks of 16: {e}" for e in compare_full(run_gpu(p, DEV, ws_tokens=16), ref)]
    assert not errors, f"deep rows T={T}: " + "; ".join(errors)


@pytest.mark.parametrize("T,W", ((40, 2600), (8, 5000)))
def test_wide_rows(T, W):
    """Rows wider than 2048 slots (the index inversion's fill walks a token's
    slots in a loop instead of holding them in registers) and, with few
    tokens, wider than the one-workgroup inversion takes (4096 slots): a
    non-compact layout much wider than S_kv, against the oracle."""
    p = wl.make_edge_wide(8, seed=150 + T, T=T, S=512, W=W)
    say(f"[gpu] wide rows T={T} W={W}: S_kv={p.S_kv} H={p.H}")
    errors = compare_full(run_gpu(p, DEV), run_oracle(p))
    assert not errors, f"wide rows T={T} W={W}: " + "; ".join(errors)


def test_batched_large_kv_set():
    """Three sequences whose concatenated KV set (43000 rows) is larger than
    one workgroup's inversion counters cover (32768 rows): O, LSE, dQ and
    Delta on sampled tokens and dKV on sampled rows against the oracle,
    d_sink over every token against the oracle's sink gradient; each
    sequence's outputs are the bits of that sequence run alone."""
    p = wl.make_batched(H=16, lengths=(20000, 15000, 8000), window=64, topk=64, seed=77)
    assert p.S_kv > 40960
    say(f"[gpu] batched large: T={p.T} S_kv={p.S_kv} H={p.H} W={p.W}")
    gpu = run_gpu(p, DEV)
    errors = []
    segs = p.meta["segments"]
    toks = np.unique(np.concatenate([[a, a + 1, b - 1] for a, b in segs] +
                                    [np.random.default_rng(9).integers(0, p.T, 24)]))
    ref = run_oracle(p, tokens=toks)
    check_tensor("o[sampled]", gpu["o"][toks], ref["o"], errors)
    check_lse(gpu["lse"][toks], ref["lse"], errors)
    check_tensor("dq[sampled]", gpu["dq"][toks], ref["dq"], errors)
    check_tensor("delta[sampled]", gpu["delta"][toks], ref["delta"], errors)
    rows = np.array([a for a, _ in segs] + [b - 1 for _, b in segs] + [32767, 32768, 40000])
    toks_r = tokens_referencing(p, rows)
    ref_r = run_oracle(p, tokens=toks_r)
    check_tensor("dkv[sampled rows]", gpu["dkv"][rows], ref_r["dkv"][rows], errors)
    x = p.np_inputs()
    ds_ref = oracle.oracle_dsink(x["q"], x["kv"], x["dO"], x["topk_idxs"], x["topk_length"], x["attn_sink"],
                                 x["scale"], x["d_v"], delta_from="bf16")
    check_dsink(gpu["d_sink"], ds_ref, errors)
    named = referenced_rows(p)
    if np.any(gpu["dkv"][~named] != 0) or not np.all(np.any(gpu["dkv"][named] != 0, axis=1)):
        errors.append("dkv: named / unnamed row structure")
    for i, (a, b) in enumerate(segs):
        g = run_gpu(wl.segment(p, i), DEV)
        for k in ("o", "lse", "dq", "dkv"):
            if not np.array_equal(gpu[k][a:b], g[k]):
                errors.append(f"segment {i}: {k} differs from the sequence run alone")
    assert not errors, "; ".join(errors)


def largest_kv_problem(d_qk, S_kv, T=48, H=24, W=200, R=4000, seed=None):
    """A problem over the largest KV set (S_kv rows) whose valid slots name R
    of its rows: the first 500, the last 1500 and 2000 in between.  Returns
    (p, rows, idx_big): p is the same problem over those R rows alone (row k
    of p is KV row rows[k]; indices renumbered, slots in the same order), and
    idx_big holds p's indices as KV rows of the large set, its padding -1 or
    values >= S_kv (S_kv itself, S_kv + 7, 2^31 - 1).  Rows that no valid
    slot names take no part in any output, so p's oracle results are the
    large problem's (dKV: rows[k] <-> row k; every other row 0)."""
    rng = np.random.default_rng(170 + d_qk if seed is None else seed)
    mid = rng.choice(S_kv - 2000, size=R - 2000, replace=False) + 500
    rows = np.sort(np.concatenate([np.arange(500), mid, np.arange(S_kv - 1500, S_kv)])).astype(np.int64)
    assert len(np.unique(rows)) == R and rows[-1] == S_kv - 1
    local = np.full((T, W), -1, dtype=np.int64)
    for t in range(T):
        n = int(rng.integers(W // 2, W + 1))
        local[t, rng.choice(W, size=n, replace=False)] = rng.choice(R, size=n, replace=False)
    local[0, 0], local[1, W - 1] = R - 1, 0                 # the last and the first row
    big = np.where(local >= 0, rows[np.clip(local, 0, None)], -1)
    pad = np.argwhere(local < 0)
    bad = np.array([S_kv, S_kv + 7, 2 ** 31 - 1])
    pick = pad[rng.random(len(pad)) < 0.3]
    big[pick[:, 0], pick[:, 1]] = bad[rng.integers(0, 3, len(pick))]

    def bf(shape, mul=1.0):
        return torch.from_numpy((rng.standard_normal(size=shape) * mul).astype(np.float32)).to(torch.bfloat16)

    p = wl.Problem(name=f"largest_kv_d{d_qk}", T=T, S_kv=R, H=H, d_qk=d_qk, d_v=512, W=W,
                   scale=1.0 / np.sqrt(d_qk), q=bf((T, H, d_qk)), kv=bf((R, d_qk)), dO=bf((T, H, 512)),
                   topk_idxs=torch.from_numpy(local.astype(np.int32)), topk_length=None,
                   attn_sink=torch.from_numpy(rng.standard_normal(H).astype(np.float32)))
    return p, rows, torch.from_numpy(big.astype(np.int32))


def test_tokens_past_2g_elements():
    """T = 32768 tokens at H = 128, d_qk = 576 (DeepSeek-V4-like rows, window
    128 + top-k 512): q, dO, O and dQ hold more than 2^31 elements, so the
    rows of the last ~3600 tokens start past 32-bit element offsets.  q, kv
    and dO are drawn on the GPU from a seeded generator.  O, LSE, Delta and dQ
    of sampled tokens (among them the first past 2^31 elements and the last),
    and dKV of rows near the end (every token that names them included),
    against the oracle on those tokens."""
    from sparse_top_attention_topk_amd import _lib
    T, H, d_qk = 32768, 128, 576
    assert T * H * d_qk > 2 ** 31
    g = torch.Generator(device=DEV).manual_seed(210)

    def draw(shape):
        return torch.randn(shape, generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)

    q, kv, dO = draw((T, H, d_qk)), draw((T, d_qk)), draw((T, H, 512))
    sink = torch.randn((H,), generator=g, device=DEV, dtype=torch.float32)
    idx_np = wl._window_topk_idxs(np.random.default_rng(210), T, 128, 512)
    idx = torch.from_numpy(idx_np).to(DEV)
    scale = 1.0 / np.sqrt(d_qk)
    say(f"[gpu] tokens past 2^31 elements: T={T} H={H} d_qk={d_qk} (q: {T * H * d_qk} elements)")
    o, lse = _lib.smla_fwd(q, kv, idx, None, sink, scale)
    delta = _lib.smla_bwd_preprocess(o, dO)
    dq, dkv, _ = _lib.smla_bwd(q, kv, dO, lse, delta, idx, None, sink, scale)
    torch.cuda.synchronize()
    first_past = -(-(2 ** 31) // (H * d_qk))
    rows = np.array([T - 1, T - 130, T - 300])
    valid = (idx_np >= 0) & (idx_np < T)
    namers = np.nonzero((valid & np.isin(idx_np, rows)).any(axis=1))[0]
    sampled = np.array([0, 1, 640, first_past - 1, first_past, first_past + 1, T - 2, T - 1])
    toks = np.unique(np.concatenate([sampled, namers]))
    tk = torch.from_numpy(toks).to(DEV)
    p = wl.Problem("tokens_past_2g_subset", len(toks), T, H, d_qk, 512, idx_np.shape[1], scale,
                   q[tk].cpu(), kv.cpu(), dO[tk].cpu(), torch.from_numpy(idx_np[toks]), None, sink.cpu())
    ref = run_oracle(p)
    errors = []
    check_tensor("o[sampled]", o[tk].float().cpu().numpy(), ref["o"], errors)
    check_lse(lse[tk].cpu().numpy(), ref["lse"], errors)
    check_tensor("dq[sampled]", dq[tk].float().cpu().numpy(), ref["dq"], errors)
    check_tensor("delta[sampled]", delta[tk].cpu().numpy(), ref["delta"], errors)
    check_tensor("dkv[rows near the end]", dkv[torch.from_numpy(rows).to(DEV)].cpu().numpy(), ref["dkv"][rows],
                 errors)
    assert not errors, "tokens past 2^31 elements: " + "; ".join(errors)


def lengths_out_of_range_problem(T=128):
    """The compact edge problem (H = 24, W = 64) with lengths outside [0, W]
    on its first tokens: -1, -2^31, W + 1, 2^31 - 1, then 0 and W (clamped
    to [0, W]: empty, empty, full, full); ``T`` < 128 keeps the first T
    tokens (split block ranges and the one-workgroup index inversion)."""
    p = wl.make_edge_compact(24)
    ln = p.topk_length.numpy().copy()
    ln[:6] = [-1, -2 ** 31, p.W + 1, 2 ** 31 - 1, 0, p.W]
    # tokens 6..9: invalid values inside the row's length (slots that do not
    # count), -1, -5, S_kv and 2^31 - 1 at every third slot
    idx = p.topk_idxs.numpy().copy()
    for k, t in enumerate(range(6, 10)):
        ln[t] = p.W
        idx[t, k::3] = (-1, -5, p.S_kv, 2 ** 31 - 1)[k]
    return wl.Problem(f"lengths_out_of_range_T{T}", T, p.S_kv, p.H, p.d_qk, p.d_v, p.W, p.scale, p.q[:T],
                      p.kv, p.dO[:T], torch.from_numpy(idx[:T].copy()), torch.from_numpy(ln[:T].copy()),
                      p.attn_sink)


@pytest.mark.parametrize("T", (128, 16))
def test_lengths_out_of_range(T):
    """Compact lengths below 0 and above W, up to the int32 extremes, are
    clamped to [0, W] by every kernel that reads them, and invalid values
    inside a row's length are slots that do not count (forward, backward,
    index inversion; with 16 tokens the split paths), against the oracle."""
    p = lengths_out_of_range_problem(T)
    say(f"[gpu] lengths out of range: T={p.T} W={p.W} lengths {p.topk_length[:6].tolist()}")
    gpu = run_gpu(p, DEV)
    errors = compare_full(gpu, run_oracle(p))
    if T < 128:
        _, o_s, lse_s = _fwd_split(p)
        ref = run_oracle(p)
        check_tensor("o (split fwd)", o_s, ref["o"], errors)
        check_lse(lse_s, ref["lse"], errors)
    assert not errors, f"lengths out of range T={T}: " + "; ".join(errors)


@pytest.mark.parametrize("scale", (0.0, -1.0 / 24, 1e-30, 0.5, 2.0))
def test_softmax_scales(scale):
    """Finite scales away from 1/sqrt(d_qk), all inside the boundary's
    contract: 0 (uniform weights), negative (the scores' order reversed), tiny,
    and 12x / 48x the usual (scores spread over hundreds of nats, so that many
    rows outgrow their first block's reference and the forward reruns them),
    on DeepSeek-V4-like rows (window 64 + top-k 128, three blocks), H = 48,
    compact and with a sink, against the oracle."""
    p = wl.make_dsv4(160, 48, 576, 512, 128, seed=190, window=64, compact=True, scale=scale,
                     name=f"scale_{scale:g}")
    say(f"[gpu] softmax scale {scale:g}: T={p.T} H={p.H} W={p.W}")
    errors = compare_full(run_gpu(p, DEV), run_oracle(p))
    assert not errors, f"scale {scale:g}: " + "; ".join(errors)


def partial_rows_past_2g_problem(T, W, S=2048, H=8, n_valid=1500, seed=None):
    """Non-compact rows so wide that one token's dKV partial rows (W slots of
    2 d_qk = 1152 bytes) span more than 2^31 bytes: n_valid distinct KV rows at
    random slot positions over the whole width, -1 elsewhere; token 0 also
    names the last slot and, when W reaches it, the first slot whose partial
    row starts past 2^31 bytes.  A finite sink."""
    rng = np.random.default_rng(180 + T if seed is None else seed)
    d_qk = 576
    idx = np.full((T, W), -1, dtype=np.int32)
    for t in range(T):
        pos = rng.choice(W, size=n_valid, replace=False)
        idx[t, pos] = rng.choice(S, size=n_valid, replace=False)
    first_past = -(-(2 ** 31) // (2 * d_qk))
    idx[0, W - 1] = 5
    if W > first_past:
        idx[0, first_past] = 7

    def bf(shape):
        return torch.from_numpy(rng.standard_normal(size=shape).astype(np.float32)).to(torch.bfloat16)

    return wl.Problem(name=f"partial_rows_past_2g_T{T}_W{W}", T=T, S_kv=S, H=H, d_qk=d_qk, d_v=512, W=W,
                      scale=1.0 / np.sqrt(d_qk), q=bf((T, H, d_qk)), kv=bf((S, d_qk)), dO=bf((T, H, 512)),
                      topk_idxs=torch.from_numpy(idx), topk_length=None,
                      attn_sink=torch.from_numpy(rng.standard_normal(H).astype(np.float32)))


@pytest.mark.parametrize("T,W", ((2, 2 ** 21 + 100), (1, 2 ** 24)))
def test_partial_rows_past_2g(T, W):
    """Rows whose dKV partial rows span more than 2^31 bytes per token, up to
    the widest rows the boundary accepts (2^24 slots): every output against
    the oracle (the partial rows are addressed per block from a 64-bit base)."""
    p = partial_rows_past_2g_problem(T, W)
    say(f"[gpu] partial rows past 2^31 bytes: T={T} W={W} S_kv={p.S_kv} H={p.H} valid={p.valid_count()}")
    errors = compare_full(run_gpu(p, DEV), run_oracle(p))
    assert not errors, f"partial rows past 2^31 bytes T={T} W={W}: " + "; ".join(errors)


@pytest.mark.parametrize("d_qk,S_kv", ((576, 1864135), (512, 2097151)))
def test_largest_kv_set(d_qk, S_kv):
    """The largest KV set the boundary accepts (KV rows are addressed with
    32-bit byte offsets: S_kv * d_qk * 2 just under 2^31), with valid slots
    on its first and last rows and padding values at and past S_kv, through
    forward, preprocess and backward (48 tokens: the backward's split block
    ranges): O, LSE, Delta, dQ and d_sink on every token, and dKV on every
    named row, against the oracle on the same problem over the named rows
    alone; every other dKV row exactly 0 (the outputs start as NaN)."""
    from sparse_top_attention_topk_amd import _lib
    p, rows, idx_big = largest_kv_problem(d_qk, S_kv)
    say(f"[gpu] largest kv set: S_kv={S_kv} d_qk={d_qk} T={p.T} H={p.H} W={p.W} named rows={len(rows)}")
    rows_d = torch.from_numpy(rows).to(DEV)
    kv = torch.zeros((S_kv, d_qk), dtype=torch.bfloat16, device=DEV)
    kv[rows_d] = p.kv.to(DEV)
    q, dO, idx, sink = p.q.to(DEV), p.dO.to(DEV), idx_big.to(DEV), p.attn_sink.to(DEV)
    o = torch.full((p.T, p.H, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((p.T, p.H), float("nan"), dtype=torch.float32, device=DEV)
    dq = torch.full((p.T, p.H, d_qk), float("nan"), dtype=torch.bfloat16, device=DEV)
    dkv = torch.full((S_kv, d_qk), float("nan"), dtype=torch.float32, device=DEV)
    d_sink = torch.full((p.H,), float("nan"), dtype=torch.float32, device=DEV)
    o, lse = _lib.smla_fwd(q, kv, idx, None, sink, p.scale, o=o, lse=lse)
    delta = _lib.smla_bwd_preprocess(o, dO)
    dq, dkv, d_sink = _lib.smla_bwd(q, kv, dO, lse, delta, idx, None, sink, p.scale, dq=dq, dkv=dkv,
                                    d_sink=d_sink)
    named = torch.zeros((S_kv,), dtype=torch.bool, device=DEV)
    named[rows_d] = True
    stray = int(torch.count_nonzero((dkv != 0).any(dim=1) & ~named))
    gpu = dict(o=o.float().cpu().numpy(), lse=lse.cpu().numpy(), dq=dq.float().cpu().numpy(),
               delta=delta.cpu().numpy(), dkv=dkv[rows_d].cpu().numpy(), d_sink=d_sink.cpu().numpy())
    del kv, dkv, named
    ref = run_oracle(p)
    errors = compare_full(gpu, ref)
    check_tensor("delta", gpu["delta"], ref["delta"], errors)
    if stray:
        errors.append(f"dkv: {stray} rows that no valid slot names are not 0")
    assert not errors, f"largest kv set d_qk={d_qk}: " + "; ".join(errors)


# ---------------------------------------------------------------------------
# few tokens: the blocks of each row split over several workgroups
# ---------------------------------------------------------------------------
SPLIT_CASES = {
    "decode-T1": lambda: wl.make_problem("decode_T1"),
    "decode-T16": lambda: wl.make_problem("decode_T16"),
    "decode-T64": lambda: wl.make_problem("decode_T64"),
    "decode-T16-h64-d512": lambda: wl.make_decode(16, H=64, d_qk=512, seed=140),
    "decode-T5-h24-k2048": lambda: wl.make_decode(5, S_kv=8192, H=24, topk=2048, seed=141),
    "spiky-T96-h64": lambda: wl.make_spiky(64, T=96, window=32, topk=160, frac=0.5),
    "decode-T1-k8064": lambda: wl.make_decode(1, H=128, topk=8064, seed=142),   # 128 blocks: 64 splits
    # scores spread over hundreds of nats: block ranges rerun with their own exact max
    "decode-T16-h64-scale2": lambda: wl.make_decode(16, S_kv=4096, H=64, seed=143, scale=2.0),
    "edge-wide-h128-T64": lambda: wl.make_edge_wide(128, T=64),
}


def _fwd_split(p):
    from sparse_top_attention_topk_amd import _lib
    d = to_dev(p, DEV)
    ws_n = _lib.smla_fwd_splitkv_workspace_size(p.T, p.S_kv, p.H, p.d_qk, p.d_v, p.W, p.scale)
    o = torch.full((p.T, p.H, p.d_v), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((p.T, p.H), float("nan"), dtype=torch.float32, device=DEV)
    o, lse = _lib.smla_fwd_splitkv(d["q"], d["kv"], d["idx"], d["length"], d["sink"], p.scale, o=o, lse=lse)
    torch.cuda.synchronize()
    return ws_n, o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_split_kv(name):
    """Few tokens against long rows: smla_fwd_splitkv runs each token's blocks
    in up to ceil(W / 64) workgroups and merges them; the backward splits
    its S/dP, dQ and dKV kernels over block ranges (dQ through fp32
    partials).  Both meet the oracle element by element; the split forward
    agrees with smla_fwd to its tolerance."""
    p = SPLIT_CASES[name]()
    say(f"[gpu] split kv {name}: T={p.T} S_kv={p.S_kv} H={p.H} d_qk={p.d_qk} W={p.W}")
    ws_n, o_s, lse_s = _fwd_split(p)
    assert ws_n > 0, "the case should split"
    gpu = run_gpu(p, DEV)                    # smla_fwd + the (split) backward
    ref = run_oracle(p)
    errors = compare_full(gpu, ref)
    check_tensor("o (split fwd)", o_s, ref["o"], errors)
    check_lse(lse_s, ref["lse"], errors)
    if not np.all(np.isfinite(o_s)):
        errors.append("split fwd: O not fully written")
    m = np.abs(gpu["o"]).max()
    if np.abs(o_s - gpu["o"]).max() > 2.0 ** -7 * m:
        errors.append(f"split fwd: O differs from smla_fwd by {np.abs(o_s - gpu['o']).max():.3e}")
    assert not errors, f"{name}: " + "; ".join(errors)


# ---------------------------------------------------------------------------
# exact Delta (smla_bwd_delta_exact) and the backward fed with it
# ---------------------------------------------------------------------------
EXACT_TOL = 1e-4
EXACT_CASES = {
    "tiny-sink": lambda: wl.make_tiny(seed=0, sink=True),
    "tiny-compact": lambda: wl.make_tiny(seed=0, sink=True, compact=True),
    "edge-compact-h24": lambda: wl.make_edge_compact(24),
    "edge-compact-h128": lambda: wl.make_edge_compact(128),
    "edge-wide-h64": lambda: wl.make_edge_wide(64),
    "edge-sink-h24": lambda: wl.make_edge_sink(24),
    "width-118-h128": lambda: wl.make_edge_width118(128),
}


@pytest.mark.parametrize("name", list(EXACT_CASES))
def test_exact_delta(name):
    p = EXACT_CASES[name]()
    say(f"[gpu] exact delta {name}: T={p.T} H={p.H} W={p.W} compact={p.topk_length is not None}")
    g = run_gpu_exact(p, DEV)
    ref = run_oracle(p, delta_from="fp64")
    d_ref = oracle_delta_exact(p)
    errors = compare_full(g, ref)
    m = np.abs(d_ref).max()
    e = np.abs(g["delta"] - d_ref).max()
    e_pre = np.abs(g["delta_pre"] - d_ref).max()
    say(f"[gpu] exact delta {name}: max err {e:.3e}, bf16-O delta {e_pre:.3e}, max|delta| {m:.3e}")
    if not np.all(np.isfinite(g["delta"])):
        errors.append("delta: non-finite entries")
    elif e > EXACT_TOL * m + 1e-7:
        errors.append(f"delta: max err {e:.3e} vs max {m:.3e}")
    if e_pre > 0 and e >= e_pre:
        errors.append(f"delta: exact {e:.3e} not below bf16-O {e_pre:.3e}")
    if g["d_sink"] is not None:
        ms = np.abs(ref["d_sink"]).max()
        es = np.abs(g["d_sink"] - ref["d_sink"]).max()
        say(f"[gpu] exact delta {name}: d_sink max err {es:.3e} vs max {ms:.3e}")
        if es > EXACT_TOL * ms + 1e-7:
            errors.append(f"d_sink: max err {es:.3e} vs max {ms:.3e}")
    if p.topk_length is not None:
        empty = np.nonzero(p.topk_length.numpy() <= 0)[0]
        if empty.size and not np.all(g["delta"][empty] == 0):
            errors.append("delta: empty rows are not 0")
    assert not errors, f"{name}: " + "; ".join(errors)


FROM_O_CASES = {
    "tiny-sink": lambda: wl.make_tiny(seed=0, sink=True, compact=False),
    "tiny-compact": lambda: wl.make_tiny(seed=0, sink=True, compact=True),
    "edge-compact-h24": lambda: wl.make_edge_compact(24),
    "edge-wide-h128-T64": lambda: wl.make_edge_wide(128, T=64),
    "edge-sink-h64": lambda: wl.make_edge_sink(64),
    "width-118-h128": lambda: wl.make_edge_width118(128),
    "batched": lambda: wl.make_batched(),
    "dsv4-512-h128": lambda: wl.make_dsv4(320, 128, 512, 512, 96, seed=71, window=64),
    "dsv4-512-h64-compact": lambda: wl.make_dsv4(320, 64, 512, 512, 96, seed=72, window=64, compact=True),
}


@pytest.mark.parametrize("name", list(FROM_O_CASES))
def test_bwd_from_o(name):
    """smla_bwd_from_o against the oracle (the smla_bwd bars), and its Delta
    against smla_bwd_preprocess's (same fp32 sums in another order)."""
    p = FROM_O_CASES[name]()
    say(f"[gpu] bwd from o {name}: T={p.T} H={p.H} W={p.W} compact={p.topk_length is not None}")
    g = run_gpu_from_o(p, DEV)
    errors = compare_full(g, run_oracle(p))
    m = np.abs(g["delta_pre"]).max()
    e = np.abs(g["delta"] - g["delta_pre"]).max()
    say(f"[gpu] bwd from o {name}: delta vs preprocess max diff {e:.3e}, max|delta| {m:.3e}")
    if not np.all(np.isfinite(g["delta"])):
        errors.append("delta: non-finite entries")
    elif e > 1e-5 * m + 1e-7:
        errors.append(f"delta: max diff {e:.3e} vs preprocess, max {m:.3e}")
    assert not errors, f"{name}: " + "; ".join(errors)


def test_bwd_from_o_full_size():
    """The headline workload (the launch configuration bench.py times):
    smla_bwd_from_o against preprocess + smla_bwd on the same forward output,
    which test_full_size_sampled holds to the oracle.  Delta to fp32 rounding;
    dq, dkv, d_sink within the oracle bars (a Delta difference in the last
    places can move a bf16 rounding of dS)."""
    from sparse_top_attention_topk_amd import _lib
    p = wl.make_problem("dsv4_flash_h128")
    say(f"[gpu] bwd from o, full size: T={p.T} H={p.H} W={p.W}")
    d = {k: None if v is None else v.to(DEV) for k, v in
         dict(q=p.q, kv=p.kv, dO=p.dO, idx=p.topk_idxs, length=p.topk_length, sink=p.attn_sink).items()}
    o, lse = _lib.smla_fwd(d["q"], d["kv"], d["idx"], d["length"], d["sink"], p.scale)
    delta = _lib.smla_bwd_preprocess(o, d["dO"])
    dq2, dkv2, ds2 = _lib.smla_bwd(d["q"], d["kv"], d["dO"], lse, delta, d["idx"], d["length"], d["sink"],
                                   p.scale)
    dq1, dkv1, ds1, delta1 = _lib.smla_bwd_from_o(d["q"], d["kv"], d["dO"], o, lse, d["idx"], d["length"],
                                                  d["sink"], p.scale)
    torch.cuda.synchronize()
    m = delta.abs().max().item()
    e = (delta1 - delta).abs().max().item()
    say(f"[gpu] bwd from o, full size: delta max diff {e:.3e} (max {m:.3e})")
    assert torch.isfinite(delta1).all() and e <= 1e-5 * m + 1e-7
    for name, a, b in (("dq", dq1.float(), dq2.float()), ("dkv", dkv1, dkv2), ("d_sink", ds1, ds2)):
        mb = b.abs().max().item()
        err = (a - b).abs().max().item()
        cos = torch.nn.functional.cosine_similarity(a.flatten().double(), b.flatten().double(), dim=0).item()
        say(f"[gpu] bwd from o, full size: {name} max diff {err:.3e} (max {mb:.3e}), cos {cos:.8f}")
        assert torch.isfinite(a).all() and err <= 2e-2 * mb and cos >= 0.9995, name


def test_exact_delta_full_size_sampled():
    """The headline workload: exact Delta on sampled tokens against the oracle."""
    from sparse_top_attention_topk_amd import _lib
    p = wl.make_problem("dsv4_flash_h128")
    say(f"[gpu] exact delta full-size: T={p.T} H={p.H}")
    q, kv, dO, idx = p.q.to(DEV), p.kv.to(DEV), p.dO.to(DEV), p.topk_idxs.to(DEV)
    sink = p.attn_sink.to(DEV)
    _, lse = _lib.smla_fwd(q, kv, idx, None, sink, p.scale)
    delta = _lib.smla_bwd_delta_exact(q, kv, dO, lse, idx, None, sink, p.scale).cpu().numpy()
    toks = np.unique(np.concatenate([[0, 1, 127, 128, p.T // 2, p.T - 1],
                                     np.random.default_rng(8).integers(0, p.T, 6)]))
    d_ref = oracle_delta_exact(p, tokens=toks)
    m = np.abs(d_ref).max()
    e = np.abs(delta[toks] - d_ref).max()
    say(f"[gpu] exact delta full-size: max err {e:.3e} vs max {m:.3e}")
    assert np.all(np.isfinite(delta)) and e <= EXACT_TOL * m


# ---------------------------------------------------------------------------
# full-size workloads, as bench.py runs them
# ---------------------------------------------------------------------------
FULL = ["dsv4_flash_h64", "dsv4_flash_h128", "dsv4_flash_h128_compact", "dsv4_pro"]


# rows whose dKV is checked against the oracle: the most-named rows (row 0 is
# named by every causal top-k set that can reach it: about 1800 tokens at
# T = 4096 and 3850 at T = 16384, the longest lists of the reduce), a row
# just past the first window, and rows named by few tokens
def _heavy_rows(p):
    T = p.T
    if T > 8192:
        return np.array([0, T // 2, T - 1])
    return np.array([0, 1, 130, T // 2, T - 64, T - 1])


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    """Sampled tokens (O, LSE, dQ, Delta) and sampled KV rows (dKV, from every
    token that names them) against the oracle; d_sink over all tokens (the
    oracle's sink gradient over every token for T = 4096; for T = 16384,
    where that would take minutes, d_sink against the fp64 sum of the GPU's
    own p_sink * Delta over every token, whose terms are checked on the
    sampled tokens); structural dKV properties."""
    p = wl.make_problem(name)
    say(f"[gpu] full-size {name}: T={p.T} H={p.H} d_qk={p.d_qk} W={p.W}")
    gpu = run_gpu(p, DEV, nan_prefill=False)
    T = p.T
    errors = []
    for k in ("o", "dq", "dkv"):
        if not np.all(np.isfinite(gpu[k])):
            errors.append(f"{k}: non-finite entries")
    # sampled tokens: first, last, and spread over the range
    toks = np.unique(np.concatenate([[0, 1, 127, 128, 640, T // 2, T - 2, T - 1],
                                     np.random.default_rng(7).integers(0, T, 8)]))
    ref = run_oracle(p, tokens=toks)
    check_tensor("o[sampled]", gpu["o"][toks], ref["o"], errors)
    check_lse(gpu["lse"][toks], ref["lse"], errors)
    check_tensor("dq[sampled]", gpu["dq"][toks], ref["dq"], errors)
    check_tensor("delta[sampled]", gpu["delta"][toks], ref["delta"], errors)
    # sampled KV rows: exact dKV from every token that names them
    rows = _heavy_rows(p)
    toks_r = tokens_referencing(p, rows)
    say(f"[gpu] full-size {name}: dKV rows {rows.tolist()} named by {toks_r.size} tokens")
    ref_r = run_oracle(p, tokens=toks_r)
    check_tensor("dkv[sampled rows]", gpu["dkv"][rows], ref_r["dkv"][rows], errors)
    # d_sink over every token
    lse, dl = gpu["lse"].astype(np.float64), gpu["delta"].astype(np.float64)
    sk = p.attn_sink.double().numpy()[None, :]
    fin = ~np.isneginf(lse)
    ps = np.where(fin, 1.0 / (1.0 + np.exp(-(sk - np.where(fin, lse, 0.0)))), 0.0)
    own = -(ps * dl).sum(axis=0)
    scale_h = np.abs(ps * dl).sum(axis=0)
    if np.any(np.abs(gpu["d_sink"] - own) > 1e-5 * scale_h + 1e-6):
        errors.append("d_sink: differs from -sum_t p_sink * Delta of the GPU's own LSE and Delta")
    if T <= 8192:
        x = p.np_inputs()
        ds_ref = oracle.oracle_dsink(x["q"], x["kv"], x["dO"], x["topk_idxs"], x["topk_length"],
                                     x["attn_sink"], x["scale"], x["d_v"], delta_from="bf16")
        m, e = np.abs(ds_ref).max(), np.abs(gpu["d_sink"] - ds_ref).max()
        say(f"[gpu] full-size {name}: d_sink max err {e:.3e} vs max|ref| {m:.3e}")
        check_dsink(gpu["d_sink"], ds_ref, errors)
    # structural: rows never named are exactly zero, named rows are nonzero
    named = referenced_rows(p)
    if np.any(gpu["dkv"][~named] != 0):
        errors.append("dkv: unnamed rows are not zero")
    if not np.all(np.any(gpu["dkv"][named] != 0, axis=1)):
        errors.append("dkv: a named row received nothing")
    assert not errors, f"{name}: " + "; ".join(errors)


def test_full_size_layout_invariance():
    """The headline's index sets in the compact layout (packed, with
    topk_length) give the same results as the non-compact layout, up to the
    summation order that the slot positions change."""
    a = wl.make_problem("dsv4_flash_h128")
    b = wl.make_problem("dsv4_flash_h128_compact")
    say("[gpu] layout invariance: headline non-compact vs compact")
    ga = run_gpu(a, DEV, nan_prefill=False)
    gb = run_gpu(b, DEV, nan_prefill=False)
    errors = []
    for k in ("o", "dq", "dkv"):
        x, y = ga[k].astype(np.float64), gb[k].astype(np.float64)
        scale = np.abs(x).max()
        if np.abs(x - y).max() > 1e-2 * scale:
            errors.append(f"{k}: max diff {np.abs(x - y).max():.3g} vs max {scale:.3g}")
        cos = float((x * y).sum() / (np.linalg.norm(x) * np.linalg.norm(y)))
        if cos < 0.99999:
            errors.append(f"{k}: cosine {cos:.7f}")
    fin = np.isfinite(ga["lse"])
    if not np.array_equal(fin, np.isfinite(gb["lse"])) or np.abs(ga["lse"][fin] - gb["lse"][fin]).max() > 1e-4:
        errors.append("lse differs")
    if np.abs(ga["d_sink"] - gb["d_sink"]).max() > 1e-3 * np.abs(ga["d_sink"]).max():
        errors.append("d_sink differs")
    assert not errors, "; ".join(errors)
