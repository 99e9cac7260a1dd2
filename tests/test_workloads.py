"""The seeded input generators: shapes, index structure and determinism."""
import numpy as np
import pytest
import torch

from sparse_top_attention_topk_amd import workloads as wl


def test_tiny_structure():
    p = wl.make_tiny()
    assert p.q.shape == (64, 4, 576) and p.kv.shape == (64, 576) and p.dO.shape == (64, 4, 512)
    assert p.q.dtype == torch.bfloat16 and p.topk_idxs.dtype == torch.int32
    idx = p.topk_idxs.numpy()
    for t in range(64):
        n = min(32, t + 1)
        row = idx[t]
        assert np.all(row[n:] == -1)
        assert len(set(row[:n].tolist())) == n
        assert row[:n].min() >= 0 and row[:n].max() <= t
    assert p.valid_count() == sum(min(32, t + 1) for t in range(64))
    assert abs(p.scale - 1 / 24) < 1e-15


def test_determinism():
    a, b = wl.make_tiny(), wl.make_tiny()
    assert torch.equal(a.q, b.q) and torch.equal(a.topk_idxs, b.topk_idxs)
    assert torch.equal(a.attn_sink, b.attn_sink)
    c = wl.make_tiny(seed=1)
    assert not torch.equal(a.q, c.q)


def test_window_topk_rows():
    # same recipe as the 4096-token workloads, shorter so it runs fast
    p = wl.make_dsv4(900, 2, 64, 32, 512, seed=5)
    idx = p.topk_idxs.numpy()
    assert idx.shape == (900, 640)
    for t in (0, 1, 127, 128, 129, 639, 640, 899):
        row = idx[t]
        win = row[:128]
        lo = max(0, t - 127)
        assert np.array_equal(win[: t - lo + 1], np.arange(lo, t + 1))
        assert np.all(win[t - lo + 1:] == -1)
        top = row[128:]
        k = min(512, lo)
        assert np.all(top[k:] == -1)
        assert len(set(top[:k].tolist())) == k
        if k:
            assert top[:k].min() >= 0 and top[:k].max() <= t - 128
        assert (row >= 0).sum() == min(t + 1, 640)


def test_headline_valid_count_closed_form():
    # sum_t min(t+1, 640) for T = 4096
    assert sum(min(t + 1, 640) for t in range(4096)) == 2416960


def test_compact_packing_keeps_sets():
    a = wl.make_dsv4(300, 2, 64, 32, 64, seed=6)
    b = wl.make_dsv4(300, 2, 64, 32, 64, seed=6, compact=True)
    ia, ib, lb = a.topk_idxs.numpy(), b.topk_idxs.numpy(), b.topk_length.numpy()
    for t in range(300):
        assert sorted(ia[t][ia[t] >= 0].tolist()) == sorted(ib[t, : lb[t]].tolist())


@pytest.mark.parametrize("H", wl.EDGE_HEADS)
def test_edge_compact(H):
    p = wl.make_edge_compact(H)
    ln = p.topk_length.numpy()
    assert ln[0] == 0 and ln[1] == 64 and ln.min() >= 0 and ln.max() <= 64
    assert (ln == 0).mean() >= 0.05
    idx = p.topk_idxs.numpy()
    for t in range(128):
        assert len(set(idx[t, : ln[t]].tolist())) == ln[t]
    assert idx.min() >= 0 and idx.max() < 128     # the tail holds in-range garbage


@pytest.mark.parametrize("H", (1, 24))
def test_edge_wide(H):
    p = wl.make_edge_wide(H)
    idx = p.topk_idxs.numpy()
    assert idx.shape == (128, 1024) and p.S_kv == 256 and p.topk_length is None
    nv = (idx >= 0).sum(axis=1)
    assert nv[0] == 0 and nv[1] == 256
    assert (idx[:, 256:] >= 0).any()
    for t in range(128):
        v = idx[t][idx[t] >= 0]
        assert len(set(v.tolist())) == v.size and (v < 256).all()


def test_edge_sink_values():
    p = wl.make_edge_sink(24)
    s = p.attn_sink.numpy()
    assert s[0] == np.float32(3.0e38) and s[1] == np.float32(-3.0e38)
    assert np.isposinf(s[2]) and np.isneginf(s[3])
    assert len(p.meta["anti_aligned_tokens"]) > 20


def test_edge_sink_anti_aligned_rows_have_very_negative_lse():
    """Self-validating, as the pages' padded-column test is: the anti-aligned
    tokens must really drive the LSE below -80 (natural log), else the case
    would stop exercising exp(-LSE) overflow."""
    import oracle
    p = wl.make_edge_sink(1)
    toks = np.array(p.meta["anti_aligned_tokens"])
    x = p.np_inputs()
    _, lse, _ = oracle.oracle_fwd(x["q"], x["kv"], x["topk_idxs"], None, None, x["scale"],
                                  x["d_v"], tokens=toks)
    assert lse.max() < -80


def test_degenerate_problems_have_their_stated_structure():
    p = wl.make_degenerate("single")
    assert (p.T, p.S_kv, p.H, p.W, p.d_qk) == (1, 1, 1, 1, 512) and p.valid_count() == 1
    p = wl.make_degenerate("all_invalid")
    assert p.valid_count() == 0 and p.W == 70 and (p.topk_idxs.numpy() == -1).all()
    p = wl.make_degenerate("out_of_range")
    idx = p.topk_idxs.numpy()
    assert ((idx >= p.S_kv).sum(axis=1) == 20).all() and ((idx < -1).sum(axis=1) == 20).all()
    assert p.valid_count() == 20 * p.T
    p = wl.make_degenerate("duplicates")
    idx = p.topk_idxs.numpy()
    assert all(len(set(r[r >= 0].tolist())) < (r >= 0).sum() for r in idx)


def test_block_gaps_structure_and_packing():
    p = wl.make_block_gaps(64)
    idx = p.topk_idxs.numpy()
    blocks = idx.reshape(p.T, -1, 64)
    live = (blocks >= 0).any(axis=2)
    assert live.sum(axis=1).max() <= 4 and (live.sum(axis=1) == 0).any()
    # some row has a dead block before one of its live blocks
    assert any(live[t].any() and not live[t][: np.nonzero(live[t])[0][-1]].all() for t in range(p.T))
    for t in range(p.T):
        v = idx[t][idx[t] >= 0]
        assert len(set(v.tolist())) == v.size
    q = wl.pack_live_blocks(p)
    qb = q.topk_idxs.numpy().reshape(p.T, -1, 64)
    for t in range(p.T):
        n = int(live[t].sum())
        assert np.array_equal(qb[t, :n], blocks[t][live[t]]) and (qb[t, n:] == -1).all()
