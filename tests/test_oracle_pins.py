"""Pins of the fp64 oracle against things other than itself.

Each check below ties the oracle to an independent fact: a second formulation
(dense masked attention with torch autograd), central finite differences,
closed forms, invariants the pages state, and values the pages print.  A set of
planted mistakes at the end shows that plausible bugs in the oracle fail them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import smla
from oracle.dense import dense_attention, dense_loss_grads, dense_mask
from oracle.fd import directional_fd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# small random problems (fp64, tiny dims so brute force and FD are cheap)
# ---------------------------------------------------------------------------
def small_problem(seed, T=7, S_kv=10, H=3, d_qk=8, d_v=4, W=6, layout="noncompact",
                  sink="finite", empty_rows=True, wide=False):
    rng = np.random.default_rng(seed)
    if wide:
        W = S_kv + 5           # a non-compact row wider than S_kv
    q = rng.standard_normal((T, H, d_qk))
    kv = rng.standard_normal((S_kv, d_qk))
    dO = rng.standard_normal((T, H, d_v))
    idx = np.full((T, W), -1, dtype=np.int32)
    length = None
    if layout == "noncompact":
        for t in range(T):
            n = int(rng.integers(0 if empty_rows else 1, min(W, S_kv) + 1))
            pos = rng.choice(W, size=n, replace=False)
            idx[t, pos] = rng.choice(S_kv, size=n, replace=False)
        if empty_rows:
            idx[0, :] = -1
    else:
        length = np.zeros(T, dtype=np.int32)
        for t in range(T):
            n = int(rng.integers(0 if empty_rows else 1, min(W, S_kv) + 1))
            length[t] = n
            idx[t, :n] = rng.choice(S_kv, size=n, replace=False)
            idx[t, n:] = rng.integers(0, S_kv, size=W - n)      # in-range garbage tail
        if empty_rows:
            length[0] = 0
    if sink == "finite":
        s = rng.standard_normal(H)
    elif sink is None:
        s = None
    else:
        s = np.asarray(sink, dtype=np.float64)
    scale = 1.0 / math.sqrt(d_qk)
    return dict(q=q, kv=kv, dO=dO, topk_idxs=idx, topk_length=length, attn_sink=s,
                scale=scale, d_v=d_v)


def run_fwd(p, **kw):
    return oracle.oracle_fwd(p["q"], p["kv"], p["topk_idxs"], p["topk_length"],
                             p["attn_sink"], p["scale"], p["d_v"], **kw)


def run_bwd(p, **kw):
    return oracle.oracle_bwd(p["q"], p["kv"], p["dO"], p["topk_idxs"], p["topk_length"],
                             p["attn_sink"], p["scale"], p["d_v"], **kw)


def dense_of(p):
    mask = dense_mask(torch.from_numpy(p["topk_idxs"]),
                      None if p["topk_length"] is None else torch.from_numpy(p["topk_length"]),
                      p["kv"].shape[0])
    sink = None if p["attn_sink"] is None else torch.from_numpy(p["attn_sink"])
    O, lse = dense_attention(torch.from_numpy(p["q"]), torch.from_numpy(p["kv"]), mask, sink,
                             p["scale"], p["d_v"])
    return O.numpy(), lse.numpy(), mask, sink


CASES = [
    dict(layout="noncompact", sink="finite"),
    dict(layout="noncompact", sink=None, empty_rows=False),
    dict(layout="compact", sink="finite"),
    dict(layout="compact", sink=None, empty_rows=False),
    dict(layout="noncompact", sink="finite", wide=True),
]


def _fwd_agrees(p):
    O, lse, _ = run_fwd(p)
    Od, lsed, _, _ = dense_of(p)
    fin = np.isfinite(lsed)
    return (np.allclose(O, Od, rtol=0, atol=1e-12)
            and np.array_equal(np.isfinite(lse), fin)
            and np.allclose(lse[fin], lsed[fin], rtol=0, atol=1e-12)
            and np.array_equal(lse[~fin], lsed[~fin]))


def _bwd_agrees_dense(p):
    dq, dkv, ds, _ = run_bwd(p)
    _, _, mask, sink = dense_of(p)
    dqd, dkvd, dsd = dense_loss_grads(torch.from_numpy(p["q"]), torch.from_numpy(p["kv"]),
                                      torch.from_numpy(p["dO"]), mask, sink, p["scale"], p["d_v"])
    ok = np.allclose(dq, dqd.numpy(), rtol=0, atol=1e-10)
    ok &= np.allclose(dkv, dkvd.numpy(), rtol=0, atol=1e-10)
    if ds is not None:
        ok &= np.allclose(ds, dsd.numpy(), rtol=0, atol=1e-10)
    return bool(ok)


def _bwd_agrees_fd(p, seed=0):
    rng = np.random.default_rng(1000 + seed)
    dq, dkv, ds, _ = run_bwd(p)
    u_q = rng.standard_normal(p["q"].shape)
    u_kv = rng.standard_normal(p["kv"].shape)
    u_s = None if p["attn_sink"] is None else rng.standard_normal(p["attn_sink"].shape)
    fd = directional_fd(p["q"], p["kv"], p["dO"], p["topk_idxs"], p["topk_length"],
                        p["attn_sink"], p["scale"], p["d_v"], u_q, u_kv, u_s)
    an = (dq * u_q).sum() + (dkv * u_kv).sum() + (0.0 if ds is None else (ds * u_s).sum())
    return abs(fd - an) <= 1e-7 * max(1.0, abs(an))


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fwd_equals_dense_masked_attention(case, seed):
    p = small_problem(seed, **CASES[case])
    assert _fwd_agrees(p)


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("seed", [0, 1])
def test_bwd_equals_dense_autograd(case, seed):
    p = small_problem(seed, **CASES[case])
    assert _bwd_agrees_dense(p)


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("seed", [0, 1])
def test_bwd_equals_central_finite_differences(case, seed):
    p = small_problem(seed, **CASES[case])
    assert _bwd_agrees_fd(p, seed)


def test_fd_is_sharp_enough_to_see_a_small_error():
    # a gradient off by 1e-4 in one entry must be visible to the FD check
    p = small_problem(3)
    rng = np.random.default_rng(7)
    dq, dkv, ds, _ = run_bwd(p)
    u_q = rng.standard_normal(p["q"].shape)
    u_kv = rng.standard_normal(p["kv"].shape)
    u_s = rng.standard_normal(p["attn_sink"].shape)
    fd = directional_fd(p["q"], p["kv"], p["dO"], p["topk_idxs"], p["topk_length"],
                        p["attn_sink"], p["scale"], p["d_v"], u_q, u_kv, u_s)
    an = (dq * u_q).sum() + (dkv * u_kv).sum() + (ds * u_s).sum()
    assert abs(fd - an) < 1e-7
    assert abs(fd - (an + 1e-4 * u_q.flat[5])) > 1e-7


def test_single_slot_closed_form():
    """K_t = 1 and no sink: p = 1, O = v, LSE = s, dS = dP - Delta = 0 so dQ = 0
    and the K part of dKV is 0; the V part of the row receives sum_h dO."""
    p = small_problem(4, layout="noncompact", sink=None, empty_rows=False)
    T, W = p["topk_idxs"].shape
    S_kv = p["kv"].shape[0]
    rng = np.random.default_rng(5)
    rows = rng.choice(S_kv, size=T, replace=False) if T <= S_kv else rng.integers(0, S_kv, T)
    idx = np.full((T, W), -1, dtype=np.int32)
    for t in range(T):
        idx[t, rng.integers(0, W)] = rows[t]
    p["topk_idxs"] = idx
    O, lse, _ = run_fwd(p)
    dq, dkv, _, _ = run_bwd(p)
    dv = p["d_v"]
    for t in range(T):
        r = rows[t]
        np.testing.assert_allclose(O[t], np.broadcast_to(p["kv"][r, :dv], O[t].shape), atol=1e-14)
        s = p["scale"] * p["q"][t] @ p["kv"][r]
        np.testing.assert_allclose(lse[t], s, atol=1e-13)
    np.testing.assert_allclose(dq, 0.0, atol=1e-13)
    exp = np.zeros_like(dkv)
    for t in range(T):
        exp[rows[t], :dv] += p["dO"][t].sum(axis=0)
    np.testing.assert_allclose(dkv, exp, atol=1e-12)


@pytest.mark.parametrize("with_sink", [False, True])
def test_zero_query_closed_form(with_sink):
    """q = 0: every valid score is 0, so p_j = 1 / (K_t + e^sink) and LSE = ln K_t."""
    p = small_problem(6, sink="finite" if with_sink else None)
    p["q"] = np.zeros_like(p["q"])
    O, lse, aux = run_fwd(p)
    for t in range(p["q"].shape[0]):
        _, rows = oracle.valid_slots(p["topk_idxs"][t], None, p["kv"].shape[0])
        K = rows.size
        if K == 0:
            assert np.all(np.isneginf(lse[t]))
            assert np.all(O[t] == 0)
            continue
        np.testing.assert_allclose(lse[t], math.log(K), atol=1e-14)
        es = np.exp(p["attn_sink"]) if with_sink else np.zeros(p["q"].shape[1])
        pj = 1.0 / (K + es)
        exp = pj[:, None] * p["kv"][rows, : p["d_v"]].sum(axis=0)[None, :]
        np.testing.assert_allclose(O[t], exp, atol=1e-13)
        np.testing.assert_allclose(aux["p_sink"][t], es * pj, atol=1e-14)


@pytest.mark.parametrize("big", [float("inf"), 3.0e38, 2.4e38])
def test_positive_saturating_sink_takes_all_mass(big):
    """A sink at (or near) the top of the fp32 range takes the whole denominator:
    O = 0, dQ = 0, dKV = 0; with a self-consistent O, Delta = 0 and d_sink = 0
    (the page's limit d_sink = -sum(dP_sum) with dP_sum = 0)."""
    p = small_problem(8, sink=[big, big, big])
    O, lse, aux = run_fwd(p)
    assert np.all(O == 0)
    fin = np.isfinite(lse)
    assert np.all(aux["p_sink"][fin] == 1.0)
    dq, dkv, ds, delta = run_bwd(p)
    assert np.all(dq == 0) and np.all(dkv == 0)
    assert np.all(delta == 0) and np.all(ds == 0)


def test_positive_saturating_sink_dsink_limit_with_external_o():
    """With Delta taken from an O that does not come from this forward (the
    pages' test feeds the kernel its own stored O), a +inf sink gives
    d_sink[h] = -sum_t Delta[t,h] over the non-empty rows (p_sink = 1)."""
    p = small_problem(9, sink=[np.inf] * 3, empty_rows=False)
    rng = np.random.default_rng(11)
    O_ext = rng.standard_normal((p["q"].shape[0], 3, p["d_v"]))
    delta = (p["dO"] * O_ext).sum(axis=2)
    O, lse, aux = run_fwd(p)
    ps = aux["p_sink"]
    assert np.all(ps == 1.0)
    np.testing.assert_allclose(-(ps * delta).sum(axis=0), -delta.sum(axis=0), atol=0)


@pytest.mark.parametrize("neg", [float("-inf"), -3.0e38])
def test_negative_saturating_sink_equals_no_sink(neg):
    p = small_problem(10, sink=[neg] * 3)
    p0 = dict(p, attn_sink=None)
    O, lse, aux = run_fwd(p)
    O0, lse0, _ = run_fwd(p0)
    np.testing.assert_array_equal(O, O0)
    np.testing.assert_array_equal(lse, lse0)
    # a non-empty row gives the sink no mass; an empty row gives a finite sink
    # all of it (e^sink / e^sink), a -inf sink none
    fin = np.isfinite(lse)
    assert np.all(aux["p_sink"][fin] == 0.0)
    assert np.all(aux["p_sink"][~fin] == (0.0 if np.isinf(neg) else 1.0))
    dq, dkv, ds, _ = run_bwd(p)
    dq0, dkv0, _, _ = run_bwd(p0)
    np.testing.assert_array_equal(dq, dq0)
    np.testing.assert_array_equal(dkv, dkv0)
    assert np.all(ds == 0.0)


@pytest.mark.parametrize("layout", ["noncompact", "compact"])
def test_empty_row(layout):
    """An empty row gives O = 0, LSE = -inf, dQ = 0 and contributes nothing."""
    p = small_problem(12, layout=layout)
    O, lse, aux = run_fwd(p)
    dq, dkv, ds, _ = run_bwd(p)
    assert np.all(O[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(dq[0] == 0)
    assert np.all(aux["p_sink"][0] == 1.0)        # a finite sink takes all of an empty row
    # removing the empty row changes nothing else
    keep = np.arange(1, p["q"].shape[0])
    p1 = dict(p, q=p["q"][keep], dO=p["dO"][keep], topk_idxs=p["topk_idxs"][keep],
              topk_length=None if p["topk_length"] is None else p["topk_length"][keep])
    dq1, dkv1, ds1, _ = run_bwd(p1)
    np.testing.assert_allclose(dkv, dkv1, atol=1e-14)
    np.testing.assert_allclose(ds, ds1, atol=1e-14)


def test_negative_length_is_empty_and_long_length_is_clamped():
    p = small_problem(13, layout="compact")
    p["topk_length"] = p["topk_length"].copy()
    W = p["topk_idxs"].shape[1]
    O, lse, _ = run_fwd(p)
    pn = dict(p, topk_length=p["topk_length"].copy())
    pn["topk_length"][0] = -5
    On, lsen, _ = run_fwd(pn)
    assert np.all(On[0] == 0) and np.all(np.isneginf(lsen[0]))
    pw = dict(p, topk_length=p["topk_length"].copy())
    pw["topk_length"][1] = W + 7
    pf = dict(p, topk_length=p["topk_length"].copy())
    pf["topk_length"][1] = W
    np.testing.assert_array_equal(run_fwd(pw)[0], run_fwd(pf)[0])


def test_padding_contents_are_ignored():
    """Compact tail values and unreferenced kv rows change nothing; a -1
    sentinel never aliases row 0 (row 0 unreferenced gets exactly zero dKV)."""
    p = small_problem(14, layout="compact")
    O, lse, _ = run_fwd(p)
    dq, dkv, ds, _ = run_bwd(p)
    rng = np.random.default_rng(15)
    p2 = dict(p, topk_idxs=p["topk_idxs"].copy(), kv=p["kv"].copy())
    T, W = p2["topk_idxs"].shape
    for t in range(T):
        n = p["topk_length"][t]
        p2["topk_idxs"][t, n:] = rng.integers(-3, 40, size=W - n)
    used = set()
    for t in range(T):
        used |= set(oracle.valid_slots(p["topk_idxs"][t], p["topk_length"][t], p["kv"].shape[0])[1].tolist())
    for r in range(p["kv"].shape[0]):
        if r not in used:
            p2["kv"][r] = rng.standard_normal(p["kv"].shape[1]) * 100
    O2, lse2, _ = run_fwd(p2)
    dq2, dkv2, ds2, _ = run_bwd(p2)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(lse, lse2)
    np.testing.assert_array_equal(dq, dq2)
    np.testing.assert_array_equal(dkv, dkv2)
    # non-compact with -1 sentinels and row 0 never named: row 0 of dKV is exactly 0
    p3 = small_problem(16, layout="noncompact")
    p3["topk_idxs"] = np.where(p3["topk_idxs"] == 0, -1, p3["topk_idxs"]).astype(np.int32)
    assert (p3["topk_idxs"] == -1).any()
    _, dkv3, _, _ = run_bwd(p3)
    assert np.all(dkv3[0] == 0)


def test_columns_past_skv_still_receive_dkv():
    """A non-compact row wider than S_kv keeps valid indices at columns >= S_kv
    ([cuDNN-FE #298]); the result equals the same sets packed to the front."""
    p = small_problem(17, layout="noncompact", wide=True, empty_rows=False)
    S_kv = p["kv"].shape[0]
    T, W = p["topk_idxs"].shape
    # force each row to hold a valid index at a column >= S_kv
    rng = np.random.default_rng(18)
    for t in range(T):
        row = p["topk_idxs"][t]
        used = set(row[row >= 0].tolist())
        free = [r for r in range(S_kv) if r not in used]
        if row[S_kv:].max() < 0 and free:
            row[S_kv + int(rng.integers(0, W - S_kv))] = free[0]
    assert (p["topk_idxs"][:, S_kv:] >= 0).any()
    packed = np.full_like(p["topk_idxs"], -1)
    for t in range(T):
        v = p["topk_idxs"][t][p["topk_idxs"][t] >= 0]
        packed[t, : v.size] = v
    pp = dict(p, topk_idxs=packed)
    for a, b in zip(run_bwd(p), run_bwd(pp)):
        np.testing.assert_allclose(a, b, atol=1e-13)
    # the rows named only at columns >= S_kv do receive dKV
    _, dkv, _, _ = run_bwd(p)
    late = set(p["topk_idxs"][:, S_kv:][p["topk_idxs"][:, S_kv:] >= 0].tolist())
    assert all(np.any(dkv[r] != 0) for r in late)


def test_duplicate_slots_equal_copied_kv_rows():
    """By the slot-wise definition a KV row named twice by one token counts
    twice.  The same problem with each second naming pointed at an appended
    copy of the row has distinct indices; its outputs must match, with the
    copy's dKV added back to the row.  This ties the duplicate branch of the
    dKV scatter to the distinct one."""
    rng = np.random.default_rng(91)
    T, S, H, d_qk, d_v, W = 5, 6, 3, 8, 4, 6
    q = rng.standard_normal((T, H, d_qk))
    kv = rng.standard_normal((S, d_qk))
    dO = rng.standard_normal((T, H, d_v))
    idx = np.array([[2, 2, 0, -1, 3, 2],
                    [1, 4, 1, -1, -1, -1],
                    [-1, -1, -1, -1, -1, -1],
                    [5, 0, 5, 0, 5, 0],
                    [3, -1, 1, 2, 4, 0]], dtype=np.int32)
    sink = rng.standard_normal(H)
    dup = dict(q=q, kv=kv, dO=dO, topk_idxs=idx, topk_length=None, attn_sink=sink,
               scale=0.35, d_v=d_v)
    kv2, idx2, origin = [kv], idx.copy(), []
    for t in range(T):
        seen = set()
        for j in range(W):
            r = int(idx[t, j])
            if r < 0:
                continue
            if r in seen:
                idx2[t, j] = S + len(origin)
                origin.append(r)
                kv2.append(kv[r:r + 1])
            seen.add(r)
    assert origin, "the problem must hold duplicates"
    dist = dict(dup, kv=np.concatenate(kv2), topk_idxs=idx2)
    O1, l1, _ = run_fwd(dup)
    O2, l2, _ = run_fwd(dist)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isfinite(l1), np.isfinite(l2))
    np.testing.assert_allclose(l1[np.isfinite(l1)], l2[np.isfinite(l2)], rtol=0, atol=1e-12)
    dq1, dkv1, ds1, _ = run_bwd(dup)
    dq2, dkv2, ds2, _ = run_bwd(dist)
    folded = dkv2[:S].copy()
    for k, r in enumerate(origin):
        folded[r] += dkv2[S + k]
    np.testing.assert_allclose(dq1, dq2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dkv1, folded, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ds1, ds2, rtol=0, atol=1e-12)


def test_layout_and_slot_permutation_invariance():
    p = small_problem(19, layout="noncompact")
    T, W = p["topk_idxs"].shape
    rng = np.random.default_rng(20)
    perm = np.stack([rng.permutation(W) for _ in range(T)])
    pperm = dict(p, topk_idxs=np.take_along_axis(p["topk_idxs"], perm, axis=1))
    compact = np.full_like(p["topk_idxs"], 7)
    length = np.zeros(T, dtype=np.int32)
    for t in range(T):
        v = p["topk_idxs"][t][p["topk_idxs"][t] >= 0]
        compact[t, : v.size] = rng.permutation(v)
        length[t] = v.size
    pc = dict(p, topk_idxs=compact, topk_length=length)
    ref_f, ref_b = run_fwd(p), run_bwd(p)
    for other in (pperm, pc):
        f, b = run_fwd(other), run_bwd(other)
        np.testing.assert_allclose(f[0], ref_f[0], atol=1e-12)
        np.testing.assert_allclose(f[1], ref_f[1], atol=1e-12)
        for x, y in zip(b, ref_b):
            np.testing.assert_allclose(x, y, atol=1e-12)


def test_head_slice_invariance():
    """An H-head run equals heads [:H] of a larger run whose extra heads have
    dO = 0 and a finite sink; dKV is unchanged ([flash-attn #2882] Validation:
    in-kernel head padding against padding to 128 heads)."""
    p = small_problem(21, H=3)
    rng = np.random.default_rng(22)
    Hx = 8
    T, H, d = p["q"].shape
    qx = np.concatenate([p["q"], rng.standard_normal((T, Hx - H, d))], axis=1)
    dOx = np.concatenate([p["dO"], np.zeros((T, Hx - H, p["d_v"]))], axis=1)
    sx = np.concatenate([p["attn_sink"], rng.standard_normal(Hx - H)])
    px = dict(p, q=qx, dO=dOx, attn_sink=sx)
    O, lse, _ = run_fwd(p)
    Ox, lsex, _ = run_fwd(px)
    np.testing.assert_allclose(Ox[:, :H], O, atol=1e-14)
    fin = np.isfinite(lse)
    np.testing.assert_array_equal(np.isfinite(lsex[:, :H]), fin)
    np.testing.assert_allclose(lsex[:, :H][fin], lse[fin], atol=1e-14)
    dq, dkv, ds, _ = run_bwd(p)
    dqx, dkvx, dsx, _ = run_bwd(px)
    np.testing.assert_allclose(dqx[:, :H], dq, atol=1e-13)
    np.testing.assert_allclose(dkvx, dkv, atol=1e-12)
    np.testing.assert_allclose(dsx[:H], ds, atol=1e-13)
    assert np.all(dsx[H:] == 0) and np.all(dqx[:, H:] == 0)


def test_probability_mass_and_delta_identity():
    p = small_problem(23)
    T = p["q"].shape[0]
    for t in range(T):
        s_idx, rows = oracle.valid_slots(p["topk_idxs"][t], None, p["kv"].shape[0])
        _, lse_cols, lse_tot, pj = smla._token_probs(p["q"][t], p["kv"], rows, p["scale"],
                                                     p["attn_sink"], p["q"].shape[2])
        total = pj.sum(axis=1) + oracle.p_sink(lse_cols, p["attn_sink"])
        np.testing.assert_allclose(total, 1.0, atol=1e-14)
        if rows.size:
            O_t = pj @ p["kv"][rows, : p["d_v"]]
            dP = p["dO"][t] @ p["kv"][rows, : p["d_v"]].T
            np.testing.assert_allclose((p["dO"][t] * O_t).sum(1), (pj * dP).sum(1), atol=1e-13)


def test_glae_and_p_sink_special_values():
    inf = float("inf")
    assert oracle.glae(inf, inf) == inf
    assert oracle.glae(-inf, -inf) == -inf
    assert oracle.glae(3.0, -inf) == 3.0
    assert oracle.glae(inf, 1.0) == inf
    assert math.isclose(float(oracle.glae(1.0, 2.0)), math.log(math.e + math.e ** 2), rel_tol=1e-15)
    assert math.isclose(float(oracle.glae(1000.0, 1000.0)), 1000.0 + math.log(2.0), rel_tol=1e-15)
    ps = oracle.p_sink(np.array([inf, -inf, -inf, 0.0, 0.0, 5.0]),
                       np.array([inf, 2.0, -inf, -inf, 0.0, 5.0 + math.log(3.0)]))
    np.testing.assert_allclose(ps, [0.5, 1.0, 0.0, 0.0, 0.5, 0.75], atol=1e-15)
    assert np.all(oracle.p_sink(np.array([1.0, 2.0]), None) == 0.0)


def test_round_to_bf16_matches_torch():
    rng = np.random.default_rng(24)
    x = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-6, 6, 10000),
                        [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9]])
    ours = smla.round_to_bf16(x)
    theirs = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(ours, theirs)


def test_bf16_delta_mode_changes_only_by_o_rounding():
    p = small_problem(25)
    dq, dkv, ds, delta = run_bwd(p)
    dq2, dkv2, ds2, delta2 = run_bwd(p, delta_from="bf16")
    O, _, _ = run_fwd(p)
    exp = (p["dO"] * smla.round_to_bf16(O)).sum(axis=2)
    exp[0] = 0.0    # empty row contributes nothing
    np.testing.assert_allclose(delta2, exp, atol=1e-13)
    assert np.max(np.abs(delta2 - delta)) < 1e-2 * max(1.0, np.max(np.abs(delta)))


def test_token_subset_matches_full_run():
    p = small_problem(26)
    O, lse, _ = run_fwd(p)
    sub = np.array([5, 1, 3])
    Os, lses, _ = run_fwd(p, tokens=sub)
    np.testing.assert_array_equal(Os, O[sub])
    np.testing.assert_array_equal(lses, lse[sub])
    dq, _, _, _ = run_bwd(p)
    dqs, _, _, _ = run_bwd(p, tokens=sub)
    np.testing.assert_array_equal(dqs, dq[sub])


# ---------------------------------------------------------------------------
# exact Delta (sum_j p_j dP_j)
# ---------------------------------------------------------------------------
def run_delta_exact(p, **kw):
    return oracle.oracle_delta_exact(p["q"], p["kv"], p["dO"], p["topk_idxs"], p["topk_length"],
                                     p["attn_sink"], p["scale"], p["d_v"], **kw)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_delta_exact_equals_dense_output_dot_do(case):
    """Delta = dO . O with O from the dense masked brute force (a formulation
    that shares no code with the per-slot sum); empty rows give 0."""
    p = small_problem(40 + case, **CASES[case])
    d = run_delta_exact(p)
    Od, lsed, _, _ = dense_of(p)
    exp = (p["dO"] * Od).sum(axis=2)
    exp[~np.isfinite(lsed)] = 0.0          # empty rows: no slot, no Delta
    np.testing.assert_allclose(d, exp, rtol=0, atol=1e-12)


def test_delta_exact_closed_forms():
    # one valid slot, no sink: p = 1, Delta = dO . v
    p = small_problem(44, sink=None, empty_rows=False)
    T, W = p["topk_idxs"].shape
    rng = np.random.default_rng(45)
    idx = np.full((T, W), -1, dtype=np.int32)
    rows = rng.integers(0, p["kv"].shape[0], T)
    for t in range(T):
        idx[t, rng.integers(0, W)] = rows[t]
    p["topk_idxs"] = idx
    d = run_delta_exact(p)
    exp = (p["dO"] * p["kv"][rows, None, : p["d_v"]]).sum(axis=2)
    np.testing.assert_allclose(d, exp, rtol=0, atol=1e-13)
    # a saturating positive sink takes all the mass: Delta = 0
    p = small_problem(46, sink=[float("inf"), 3.0e38, 2.4e38], empty_rows=False)
    assert np.all(run_delta_exact(p) == 0)
    # a token subset gives the same rows
    p = small_problem(47)
    sub = np.array([6, 2, 3])
    np.testing.assert_array_equal(run_delta_exact(p, tokens=sub), run_delta_exact(p)[sub])


def test_delta_exact_vs_bf16_output_delta():
    """The bf16-rounded O of the default backward moves Delta by about 2^-9
    relative; the exact form agrees with the fp64-O backward's Delta."""
    p = small_problem(48)
    d = run_delta_exact(p)
    _, _, _, d64 = run_bwd(p, delta_from="fp64")
    _, _, _, d16 = run_bwd(p, delta_from="bf16")
    np.testing.assert_allclose(d, d64, rtol=0, atol=1e-12)
    assert np.abs(d16 - d).max() > 1e-6 * np.abs(d).max()


def test_planted_delta_mistakes_are_caught():
    """Sum over every slot position (sentinels aliased to row 0), or softmax
    without the sink: both must fail the dense pin."""
    p = small_problem(49)
    Od, lsed, _, _ = dense_of(p)
    exp = (p["dO"] * Od).sum(axis=2)
    exp[~np.isfinite(lsed)] = 0.0
    T, H, d_qk = p["q"].shape
    bad_alias = np.zeros((T, H))
    bad_nosink = np.zeros((T, H))
    for t in range(T):
        rows_all = np.clip(p["topk_idxs"][t].astype(np.int64), 0, None)
        _, _, _, pa = smla._token_probs(p["q"][t], p["kv"], rows_all, p["scale"], p["attn_sink"], d_qk)
        bad_alias[t] = (pa * (p["dO"][t] @ p["kv"][rows_all, : p["d_v"]].T)).sum(1)
        _, rows = smla.valid_slots(p["topk_idxs"][t], None, p["kv"].shape[0])
        if rows.size:
            _, _, _, pn = smla._token_probs(p["q"][t], p["kv"], rows, p["scale"], None, d_qk)
            bad_nosink[t] = (pn * (p["dO"][t] @ p["kv"][rows, : p["d_v"]].T)).sum(1)
    assert not np.allclose(bad_alias, exp, rtol=0, atol=1e-12)
    assert not np.allclose(bad_nosink, exp, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# batches as concatenated sequences with global indices
# ---------------------------------------------------------------------------
def test_batched_problem_equals_its_sequences():
    """Several sequences packed with global indices ([cuDNN-FE #298]: global
    row indices over total_S_kv) give, per sequence, exactly the results of
    that sequence alone; dKV rows of a sequence only receive its own tokens and
    d_sink is the sum over the sequences."""
    from sparse_top_attention_topk_amd import workloads as wl
    for compact in (False, True):
        p = wl.make_batched(H=2, lengths=(9, 4, 12), window=4, topk=6, seed=71, compact=compact)
        x = p.np_inputs()
        O, lse, _ = oracle.oracle_fwd(x["q"], x["kv"], x["topk_idxs"], x["topk_length"], x["attn_sink"],
                                      x["scale"], x["d_v"])
        dq, dkv, ds, _ = oracle.oracle_bwd(x["q"], x["kv"], x["dO"], x["topk_idxs"], x["topk_length"],
                                           x["attn_sink"], x["scale"], x["d_v"])
        ds_sum = np.zeros_like(ds)
        for i, (a, b) in enumerate(p.meta["segments"]):
            y = wl.segment(p, i).np_inputs()
            Oi, lsei, _ = oracle.oracle_fwd(y["q"], y["kv"], y["topk_idxs"], y["topk_length"],
                                            y["attn_sink"], y["scale"], y["d_v"])
            dqi, dkvi, dsi, _ = oracle.oracle_bwd(y["q"], y["kv"], y["dO"], y["topk_idxs"],
                                                  y["topk_length"], y["attn_sink"], y["scale"], y["d_v"])
            np.testing.assert_allclose(O[a:b], Oi, rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[a:b], lsei, rtol=0, atol=1e-13)
            np.testing.assert_allclose(dq[a:b], dqi, rtol=0, atol=1e-13)
            np.testing.assert_allclose(dkv[a:b], dkvi, rtol=0, atol=1e-13)
            ds_sum += dsi
        np.testing.assert_allclose(ds, ds_sum, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# values the pages print
# ---------------------------------------------------------------------------
def test_pages_sink_threshold_and_limits():
    """tests/golden/pages_sink_limits.json: the log2(e) rescale of an fp32 sink
    saturates above ~2.36e38; the saturating-sink test values; p_sink of two
    +inf terms is 1/2."""
    with open(os.path.join(GOLDEN, "pages_sink_limits.json")) as f:
        g = json.load(f)
    thr = np.float32(3.4e38) / np.float32(math.log2(math.e))
    assert abs(float(thr) - g["rescale_overflow_threshold"]) / g["rescale_overflow_threshold"] < 5e-3
    with np.errstate(over="ignore"):
        for v in g["test_sinks"]:
            if math.isfinite(v) and abs(v) > g["rescale_overflow_threshold"]:
                assert np.isinf(np.float32(v) * np.float32(math.log2(math.e)))
    assert float(oracle.p_sink(np.array([np.inf]), np.array([np.inf]))[0]) == g["p_sink_both_pos_inf"]
    # the saturating-sink limits hold in the oracle for each of the pages' values
    for v in g["test_sinks"]:
        p = small_problem(27, sink=[v] * 3, empty_rows=False)
        dq, dkv, ds, _ = run_bwd(p)
        if v > 0:
            assert np.all(dq == 0) and np.all(dkv == 0)
        else:
            p0 = dict(p, attn_sink=None)
            dq0, dkv0, _, _ = run_bwd(p0)
            np.testing.assert_array_equal(dq, dq0)
            np.testing.assert_array_equal(dkv, dkv0)


# ---------------------------------------------------------------------------
# the sink gradient alone (oracle_dsink)
# ---------------------------------------------------------------------------
def run_dsink(p, **kw):
    return oracle.oracle_dsink(p["q"], p["kv"], p["dO"], p["topk_idxs"], p["topk_length"],
                               p["attn_sink"], p["scale"], p["d_v"], **kw)


@pytest.mark.parametrize("case", [c for c in range(len(CASES)) if CASES[c]["sink"] is not None])
@pytest.mark.parametrize("seed", [0, 1])
def test_dsink_alone_equals_dense_autograd(case, seed):
    """oracle_dsink against the sink gradient of the dense formulation
    (torch fp64 autograd through a softmax with the sink as an extra column)."""
    p = small_problem(seed, **CASES[case])
    _, _, mask, sink = dense_of(p)
    _, _, dsd = dense_loss_grads(torch.from_numpy(p["q"]), torch.from_numpy(p["kv"]),
                                 torch.from_numpy(p["dO"]), mask, sink, p["scale"], p["d_v"])
    np.testing.assert_allclose(run_dsink(p), dsd.numpy(), rtol=0, atol=1e-10)


def test_dsink_alone_modes_and_limits():
    """No sink gives None; a +inf sink with its own O gives 0 (Delta = 0);
    the bf16-O mode moves d_sink only by the rounding of O; a token subset
    sums that subset's terms."""
    p = small_problem(12, T=9)
    assert run_dsink(dict(p, attn_sink=None)) is None
    assert np.all(run_dsink(dict(p, attn_sink=np.full(3, np.inf))) == 0.0)
    a, b = run_dsink(p), run_dsink(p, delta_from="bf16")
    assert np.abs(a - b).max() < 1e-2 * max(np.abs(a).max(), 1e-30) and not np.array_equal(a, b)
    part = run_dsink(p, tokens=np.arange(0, 4)) + run_dsink(p, tokens=np.arange(4, 9))
    np.testing.assert_allclose(part, a, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin
# ---------------------------------------------------------------------------
def _all_pins_pass(seed=30):
    ok = True
    for case in CASES:
        p = small_problem(seed, **case)
        ok &= _fwd_agrees(p)
        ok &= _bwd_agrees_dense(p)
        ok &= _bwd_agrees_fd(p)
    return bool(ok)


def test_pins_pass_on_the_real_oracle():
    assert _all_pins_pass()


def _mutant_bwd(bug):
    """The oracle backward with one plausible mistake planted."""
    def bwd(q, kv, dO, topk_idxs, topk_length, attn_sink, scale, d_v, delta_from="fp64",
            tokens=None):
        T, H, d_qk = q.shape
        S_kv = kv.shape[0]
        dq = np.zeros((T, H, d_qk))
        dkv = np.zeros((S_kv, d_qk))
        d_sink = np.zeros(H)
        for t in range(T):
            ln = None if topk_length is None else topk_length[t]
            _, rows = smla.valid_slots(topk_idxs[t], ln, S_kv)
            if rows.size == 0:
                continue
            _, lse_cols, _, p = smla._token_probs(q[t], kv, rows, scale, attn_sink, d_qk)
            o_t = p @ kv[rows, :d_v]
            dl = (dO[t] * o_t).sum(axis=1)
            dP = dO[t] @ kv[rows, :d_v].T
            dS = p * dP if bug == "no_delta" else p * (dP - dl[:, None])
            dq[t] = (1.0 if bug == "no_scale_dq" else scale) * (dS @ kv[rows, :d_qk])
            gk = scale * (dS.T @ q[t])
            if bug != "no_dv":
                gk[:, :d_v] += p.T @ dO[t]
            if bug == "dv_wrong_cols":
                gk[:, -d_v:] += p.T @ dO[t]
                gk[:, :d_v] -= p.T @ dO[t]
            dkv[rows] += gk
            if attn_sink is not None:
                sign = 1.0 if bug == "dsink_sign" else -1.0
                d_sink += sign * smla.p_sink(lse_cols, attn_sink) * dl
        return dq, dkv, (d_sink if attn_sink is not None else None), None
    return bwd


def _mutants():
    def glae_ignores_sink(a, b):
        return np.asarray(a, dtype=np.float64).copy()

    def valid_slots_clamps_minus_one(idx_row, length, S_kv):
        W = idx_row.shape[0]
        n = W if length is None else min(max(int(length), 0), W)
        ids = np.clip(idx_row[:n].astype(np.int64), 0, S_kv - 1)
        return np.arange(n), ids

    orig_valid = smla.valid_slots

    def valid_slots_position_vs_skv(idx_row, length, S_kv):
        cand, ids = orig_valid(idx_row, length, S_kv)
        keep = cand < S_kv
        return cand[keep], ids[keep]

    def valid_slots_ignores_length(idx_row, length, S_kv):
        return orig_valid(idx_row, None, S_kv)

    def p_sink_dropped(lse, sink):
        return np.zeros_like(np.asarray(lse, dtype=np.float64))

    return {
        "glae_ignores_sink": ("glae", glae_ignores_sink),
        "minus_one_aliases_row0": ("valid_slots", valid_slots_clamps_minus_one),
        "position_compared_with_skv": ("valid_slots", valid_slots_position_vs_skv),
        "compact_tail_not_ignored": ("valid_slots", valid_slots_ignores_length),
        "p_sink_dropped": ("p_sink", p_sink_dropped),
        "bwd_no_delta": ("oracle_bwd", _mutant_bwd("no_delta")),
        "bwd_no_scale_in_dq": ("oracle_bwd", _mutant_bwd("no_scale_dq")),
        "bwd_no_dv": ("oracle_bwd", _mutant_bwd("no_dv")),
        "bwd_dv_wrong_columns": ("oracle_bwd", _mutant_bwd("dv_wrong_cols")),
        "bwd_dsink_sign": ("oracle_bwd", _mutant_bwd("dsink_sign")),
    }


@pytest.mark.parametrize("name", list(_mutants().keys()))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = _mutants()[name]
    monkeypatch.setattr(smla, attr, fn)
    monkeypatch.setattr(oracle, attr, fn, raising=False)
    caught = False
    for seed in (30, 31):
        for case in CASES:
            p = small_problem(seed, **case)
            if attr == "position_compared_with_skv":
                p = small_problem(seed, layout="noncompact", wide=True, empty_rows=False)
            try:
                ok = _fwd_agrees(p) and _bwd_agrees_dense(p) and _bwd_agrees_fd(p)
            except Exception:
                ok = False
            if not ok:
                caught = True
                break
        if caught:
            break
    assert caught, f"planted mistake {name} was not caught by any pin"
