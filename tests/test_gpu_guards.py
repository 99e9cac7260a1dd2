"""Guard regions around every buffer the library writes.

Each output (and the backward's workspace) is a view into a larger device
buffer whose bytes before and after the view hold a fixed pattern; the view
itself starts NaN-filled.  After the calls the guard bytes must be unchanged,
and the outputs must be the bits of an ordinary (unguarded) run.
"""
import numpy as np
import pytest
import torch

from parity import run_gpu, say, to_dev
from sparse_top_attention_topk_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
GUARD = 4096                       # bytes on each side of a view
PATTERN = 0x5A


class Guarded:
    """A view of ``shape`` / ``dtype`` inside a byte buffer with guards."""

    def __init__(self, shape, dtype, fill=float("nan"), nbytes=None):
        esz = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) if nbytes is None else nbytes // esz
        self.inner = n * esz
        self.buf = torch.full((GUARD + self.inner + GUARD,), PATTERN, dtype=torch.uint8, device=DEV)
        self.view = self.buf[GUARD:GUARD + self.inner].view(dtype)
        if nbytes is None:
            self.view = self.view.view(shape)
            self.view.fill_(fill)

    def intact(self):
        b = self.buf.cpu().numpy()
        return bool(np.all(b[:GUARD] == PATTERN) and np.all(b[GUARD + self.inner:] == PATTERN))


def _run_guarded(p):
    from sparse_top_attention_topk_amd import _lib
    d = to_dev(p, DEV)
    T, H = p.T, p.H
    g = {
        "o": Guarded((T, H, p.d_v), torch.bfloat16),
        "lse": Guarded((T, H), torch.float32),
        "delta": Guarded((T, H), torch.float32),
        "dq": Guarded((T, H, p.d_qk), torch.bfloat16),
        "dkv": Guarded((p.S_kv, p.d_qk), torch.float32),
        "delta_x": Guarded((T, H), torch.float32),
        "delta_o": Guarded((T, H), torch.float32),
        "dq_o": Guarded((T, H, p.d_qk), torch.bfloat16),
        "dkv_o": Guarded((p.S_kv, p.d_qk), torch.float32),
    }
    if d["sink"] is not None:
        g["d_sink"] = Guarded((H,), torch.float32)
        g["d_sink_o"] = Guarded((H,), torch.float32)
    need = _lib.smla_bwd_workspace_size(T, p.S_kv, H, p.d_qk, p.d_v, p.W, p.scale)
    ws = Guarded(None, torch.uint8, nbytes=max(need, 16))
    v = {k: x.view for k, x in g.items()}
    _lib.smla_fwd(d["q"], d["kv"], d["idx"], d["length"], d["sink"], p.scale, o=v["o"], lse=v["lse"])
    _lib.smla_bwd_preprocess(v["o"], d["dO"], delta=v["delta"])
    _lib.smla_bwd(d["q"], d["kv"], d["dO"], v["lse"], v["delta"], d["idx"], d["length"], d["sink"], p.scale,
                  dq=v["dq"], dkv=v["dkv"], d_sink=v.get("d_sink"), workspace=ws.view)
    _lib.smla_bwd_delta_exact(d["q"], d["kv"], d["dO"], v["lse"], d["idx"], d["length"], d["sink"], p.scale,
                              delta=v["delta_x"])
    _lib.smla_bwd_from_o(d["q"], d["kv"], d["dO"], v["o"], v["lse"], d["idx"], d["length"], d["sink"],
                         p.scale, delta=v["delta_o"], dq=v["dq_o"], dkv=v["dkv_o"], d_sink=v.get("d_sink_o"),
                         workspace=ws.view)
    torch.cuda.synchronize()
    g["workspace"] = ws
    return g


CASES = {
    "tiny": lambda: wl.make_tiny(seed=0),
    "edge-compact-h24": lambda: wl.make_edge_compact(24),
    "edge-wide-h128": lambda: wl.make_edge_wide(128),
    "width-118-h90": lambda: wl.make_edge_width118(90),
    "dsv4-512-h72": lambda: wl.make_dsv4(320, 72, 512, 512, 96, seed=75, window=64),
    "degenerate-all-invalid": lambda: wl.make_degenerate("all_invalid"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_guard_regions_untouched(name):
    p = CASES[name]()
    say(f"[gpu] guards {name}: T={p.T} S_kv={p.S_kv} H={p.H} d_qk={p.d_qk} W={p.W}")
    g = _run_guarded(p)
    bad = [k for k, x in g.items() if not x.intact()]
    assert not bad, f"{name}: guard bytes changed around {bad}"
    ref = run_gpu(p, DEV)
    for k in ("o", "lse", "delta", "dq", "dkv", "d_sink"):
        if k not in g:
            continue
        got = g[k].view.float().cpu().numpy() if g[k].view.dtype == torch.bfloat16 else g[k].view.cpu().numpy()
        assert np.array_equal(got, ref[k]), f"{name}: {k} differs from the unguarded run"
    # the one-call backward fills the same outputs
    for k, r in (("dq_o", "dq"), ("dkv_o", "dkv"), ("d_sink_o", "d_sink")):
        if k in g:
            got = g[k].view.float().cpu().numpy()
            assert np.all(np.isfinite(got)), f"{name}: {k} not fully written"
    assert np.all(np.isfinite(g["delta_x"].view.cpu().numpy())), f"{name}: exact delta not fully written"
