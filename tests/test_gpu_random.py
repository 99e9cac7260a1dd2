"""Seeded random problems against the oracle, element by element.

Each seed draws every size and index property (workloads.make_random): T,
S_kv, H (1..128, including partly filled groups of 16 and 32 heads), d_qk,
W (1..1500), the layout, the sink (none, finite, saturating on some heads),
empty rows, duplicate indices, out-of-range values among the padding, and a
workspace that sometimes holds only part of the tokens (token chunks, and
block splits below 128 tokens per chunk).  The forward with split KV runs as
well whenever the problem is small enough to split.  Every output meets the
oracle's bars; the split forward agrees with smla_fwd.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import (compare_full, run_gpu, run_gpu_exact, run_oracle, say, check_tensor, check_lse,
                    check_dsink, to_dev)
from sparse_top_attention_topk_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
SEEDS = range(128)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_problem(seed):
    from sparse_top_attention_topk_amd import _lib
    p = wl.make_random(seed)
    say(f"[gpu] random {seed}: T={p.T} S_kv={p.S_kv} H={p.H} d_qk={p.d_qk} W={p.W} "
        f"compact={p.topk_length is not None} sink={p.meta['sink_kind']} ws_tokens={p.meta['ws_tokens']}")
    gpu = run_gpu(p, DEV, ws_tokens=p.meta["ws_tokens"])
    ref = run_oracle(p)
    errors = [e for e in compare_full(gpu, ref) if not e.startswith("d_sink")]
    errors += _dsink_errors(p, gpu, ref, seed)
    fws = _lib.smla_fwd_splitkv_workspace_size(p.T, p.S_kv, p.H, p.d_qk, p.d_v, p.W, p.scale)
    if fws > 0:
        say(f"[gpu] random {seed}: split forward ({fws} bytes of workspace)")
        d = to_dev(p, DEV)
        o, lse = _lib.smla_fwd_splitkv(d["q"], d["kv"], d["idx"], d["length"], d["sink"], p.scale)
        torch.cuda.synchronize()
        o = o.float().cpu().numpy()
        check_tensor("o (split fwd)", o, ref["o"], errors)
        check_lse(lse.cpu().numpy(), ref["lse"], errors)
        m = np.abs(gpu["o"]).max()
        if m > 0 and np.abs(o - gpu["o"]).max() > 2.0 ** -7 * m:
            errors.append("split forward: O differs from smla_fwd beyond a bf16 rounding step")
    assert not errors, f"random {seed}: " + "; ".join(errors)


def _dsink_errors(p, gpu, ref, seed):
    """d_sink at the stated bar (1e-2 of the largest head) against the oracle
    with Delta from the bf16 O.  A sum over few tokens can cancel so far that
    the bf16 rounding of O alone moves the oracle's own d_sink by a sizeable
    share of it ([cuDNN-FE #785] Not addressed: the bf16-O Delta limits
    d_sink); there (a shift above 0.2 %) the exact-Delta path is held to the
    fp64 oracle at 1e-4 instead.  In every case the GPU's d_sink must be
    -sum_t p_sink Delta of its own LSE and Delta."""
    errors = []
    if ref["d_sink"] is None:
        return errors
    lse, dl = gpu["lse"].astype(np.float64), gpu["delta"].astype(np.float64)
    sk = p.attn_sink.double().numpy()[None, :]
    fin = ~np.isneginf(lse)
    with np.errstate(over="ignore", invalid="ignore"):
        ps = np.where(fin, 1.0 / (1.0 + np.exp(-(sk - np.where(fin, lse, 0.0)))), 0.0)
    ps = np.where(np.isneginf(sk), 0.0, ps)
    terms = np.where(ps == 0.0, 0.0, ps * dl)
    own = -terms.sum(axis=0)
    if np.any(np.abs(gpu["d_sink"] - own) > 1e-5 * np.abs(terms).sum(axis=0) + 1e-7):
        errors.append("d_sink: not -sum p_sink Delta of its own LSE and Delta")
    stated = []
    check_dsink(gpu["d_sink"], ref["d_sink"], stated)
    if not stated:
        return errors
    x = p.np_inputs()
    ds64 = oracle.oracle_dsink(x["q"], x["kv"], x["dO"], x["topk_idxs"], x["topk_length"], x["attn_sink"],
                               x["scale"], x["d_v"], delta_from="fp64")
    m64 = np.abs(ds64).max()
    shift = np.abs(ref["d_sink"] - ds64).max() / m64 if m64 > 0 else 0.0
    say(f"[gpu] random {seed}: {stated[0]}; bf16 O alone moves d_sink by {shift:.2%}")
    if shift <= 2e-3:
        return errors + stated
    ge = run_gpu_exact(p, DEV)
    e = np.abs(ge["d_sink"] - ds64).max()
    if not (e <= 1e-4 * m64 + 1e-7):
        errors.append(f"exact-Delta d_sink: max err {e:.3e} vs max {m64:.3e}")
    return errors
