"""smla_bwd_noalloc, the backward on the library's fixed per-GPU scratch,
against smla_bwd with a workspace of its own: two calls in a row through the
C ABI, the second on a smaller problem (the scratch keeps the first call's
contents, which the second must not depend on).

d_sink does not depend on how the tokens are chunked and must be the same
bits; dKV sums each row chunk by chunk and dQ sums block ranges when a chunk
has fewer than 128 tokens, so with a chunk size other than smla_bwd's they
may differ by the summation grouping only (and must be the same bits when
both run one chunk)."""
import pytest
import torch

from parity import say, to_dev
from sparse_top_attention_topk_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _inputs(p):
    from sparse_top_attention_topk_amd import _lib
    d = to_dev(p, DEV)
    o, lse = _lib.smla_fwd(d["q"], d["kv"], d["idx"], d["length"], d["sink"], p.scale)
    delta = _lib.smla_bwd_preprocess(o, d["dO"])
    return d, lse, delta


def _outputs(p, fill):
    dq = torch.full((p.T, p.H, p.d_qk), fill, dtype=torch.bfloat16, device=DEV)
    dkv = torch.full((p.S_kv, p.d_qk), fill, dtype=torch.float32, device=DEV)
    ds = None if p.attn_sink is None else torch.full((p.H,), fill, dtype=torch.float32, device=DEV)
    return dq, dkv, ds


def _compare(p, label, one_chunk):
    from sparse_top_attention_topk_amd import _lib
    d, lse, delta = _inputs(p)
    args = (d["q"], d["kv"], d["dO"], lse, delta, d["idx"], d["length"], d["sink"], p.scale)
    dq0, dkv0, ds0 = _outputs(p, 0.0)
    _lib.smla_bwd(*args, dq=dq0, dkv=dkv0, d_sink=ds0)
    dq1, dkv1, ds1 = _outputs(p, float("nan"))
    say(f"[gpu] noalloc {label}: T={p.T} S_kv={p.S_kv} H={p.H} W={p.W}")
    _lib.smla_bwd_noalloc(*args, dq=dq1, dkv=dkv1, d_sink=ds1)
    torch.cuda.synchronize()
    if one_chunk:
        assert torch.equal(dq1, dq0), f"{label}: dq differs from smla_bwd"
    else:
        md = dq0.float().abs().max().item()
        ed = (dq1.float() - dq0.float()).abs().max().item()
        say(f"[gpu] noalloc {label}: dq max diff {ed:.3e} (max {md:.3e})")
        assert ed <= 2.0 ** -7 * md, f"{label}: dq differs from smla_bwd by {ed:.3e}"
    if ds0 is not None:
        assert torch.equal(ds1, ds0), f"{label}: d_sink differs from smla_bwd"
    assert torch.isfinite(dkv1).all(), f"{label}: dkv not fully written"
    assert torch.equal((dkv1 != 0).any(1), (dkv0 != 0).any(1)), f"{label}: the rows receiving dKV differ"
    m = dkv0.abs().max().item()
    e = (dkv1 - dkv0).abs().max().item()
    say(f"[gpu] noalloc {label}: dkv max diff {e:.3e} (max {m:.3e})")
    if one_chunk:
        assert torch.equal(dkv1, dkv0), f"{label}: dkv differs from smla_bwd (both one chunk)"
    else:
        assert e <= 1e-5 * m, f"{label}: dkv differs from smla_bwd by {e:.3e}"


def test_noalloc_matches_bwd_on_two_calls():
    from sparse_top_attention_topk_amd import _lib
    big = wl.make_dsv4(1024, 128, 576, 512, 512, seed=78)
    small = wl.make_edge_compact(24)
    # the first problem needs more than the scratch at once (chunked), the
    # second fits in one chunk
    need_big = _lib.smla_bwd_workspace_size(big.T, big.S_kv, big.H, big.d_qk, big.d_v, big.W, big.scale)
    need_small = _lib.smla_bwd_workspace_size(small.T, small.S_kv, small.H, small.d_qk, small.d_v, small.W,
                                              small.scale)
    assert need_big > _lib.SMLA_NOALLOC_SCRATCH_BYTES >= need_small
    _compare(big, "dsv4-1024-h128", one_chunk=False)
    _compare(small, "edge-compact-h24", one_chunk=True)
