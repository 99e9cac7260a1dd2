"""One full step (smla_fwd, smla_bwd_preprocess, smla_bwd) captured in a HIP
graph through the C ABI and replayed: every replay, with eager work on the
outputs between replays, reproduces the eager step bit for bit (the library
enqueues kernels only, no memsets, and its results are deterministic)."""
import pytest
import torch

from parity import say, to_dev
from sparse_top_attention_topk_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

CASES = {
    "tiny-sink": lambda: wl.make_tiny(seed=0, sink=True, compact=False),
    "edge-compact-h64": lambda: wl.make_edge_compact(64),
    "edge-wide-h128": lambda: wl.make_edge_wide(128),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_matches_eager(name):
    from sparse_top_attention_topk_amd import _lib
    p = CASES[name]()
    say(f"[gpu] graph replay {name}: T={p.T} H={p.H} W={p.W} compact={p.topk_length is not None}")
    d = to_dev(p, DEV)
    T, H = p.T, p.H
    out = dict(
        o=torch.empty((T, H, p.d_v), dtype=torch.bfloat16, device=DEV),
        lse=torch.empty((T, H), dtype=torch.float32, device=DEV),
        delta=torch.empty((T, H), dtype=torch.float32, device=DEV),
        dq=torch.empty((T, H, p.d_qk), dtype=torch.bfloat16, device=DEV),
        dkv=torch.empty((p.S_kv, p.d_qk), dtype=torch.float32, device=DEV),
    )
    if d["sink"] is not None:
        out["d_sink"] = torch.empty((H,), dtype=torch.float32, device=DEV)
    need = _lib.smla_bwd_workspace_size(T, p.S_kv, H, p.d_qk, p.d_v, p.W, p.scale)
    ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=DEV)

    def step():
        _lib.smla_fwd(d["q"], d["kv"], d["idx"], d["length"], d["sink"], p.scale, o=out["o"], lse=out["lse"])
        _lib.smla_bwd_preprocess(out["o"], d["dO"], delta=out["delta"])
        _lib.smla_bwd(d["q"], d["kv"], d["dO"], out["lse"], out["delta"], d["idx"], d["length"], d["sink"],
                      p.scale, dq=out["dq"], dkv=out["dkv"], d_sink=out.get("d_sink"), workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # a warm-up on the capture stream's sibling
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in out.values():                   # eager work between replays
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in out.items():                 # (-inf LSE of empty rows compares equal)
            assert torch.equal(v, ref[k]), f"replay {rep}: {k} differs from the eager step"
    say(f"[gpu] graph replay {name}: 3 replays equal the eager step")
