"""The C-ABI library: it loads, exports every symbol include/smla.h declares,
and rejects bad arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smla.h")


@pytest.fixture(scope="module")
def lib():
    from sparse_top_attention_topk_amd import build_lib
    if not os.path.exists(build_lib.LIB):
        build_lib.build()
    from sparse_top_attention_topk_amd import _lib
    return _lib


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:SMLA_API\s+)?(?:smla_status|size_t|int|const char\*)\s+(smla_\w+)\(",
                                 src, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(["smla_fwd", "smla_fwd_splitkv_workspace_size", "smla_fwd_splitkv",
                                           "smla_bwd_preprocess", "smla_bwd_delta_exact",
                                           "smla_bwd", "smla_bwd_from_o", "smla_bwd_workspace_size",
                                           "smla_bwd_chunk_tokens",
                                           "smla_bwd_profiled", "smla_bwd_noalloc", "smla_status_string"])
    from sparse_top_attention_topk_amd import _lib
    assert sorted(_lib.EXPORTED) == declared_functions()


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (smla_\w+)$", out, re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib.LIB, name)


def test_library_exports_no_other_functions(lib):
    """The library's exported functions are the header's entry points: its
    internal C++ functions (launchers, kernel stubs) stay hidden."""
    out = subprocess.run(["nm", "-D", "--defined-only", lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    functions = set(re.findall(r"^\S+ [TW] (\S+)$", out, re.M))
    assert functions == set(declared_functions())


def test_status_strings(lib):
    for code in range(8):
        assert lib.LIB.smla_status_string(code)
    assert lib.LIB.smla_status_string(0) == b"ok"


def _dims(lib, **kw):
    base = dict(T=4, S_kv=8, H=2, d_qk=576, d_v=512, W=4, scale=0.1)
    base.update(kw)
    return lib.make_dims(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(d_qk=128), 3), (dict(d_v=256), 3), (dict(H=129), 3), (dict(H=0), 2),
    (dict(S_kv=1864136), 3), (dict(S_kv=2097152, d_qk=512), 3), (dict(W=(1 << 24) + 1), 3),
    (dict(S_kv=40961), 1), (dict(S_kv=1864135), 1), (dict(S_kv=2097151, d_qk=512), 1),
    (dict(W=0), 2), (dict(S_kv=0), 2), (dict(T=-1), 2), (dict(scale=float("nan")), 2),
])
def test_fwd_rejects_bad_dims(lib, kw, code):
    d = _dims(lib, **kw)
    st = lib.LIB.smla_fwd(ctypes.byref(d), None, None, None, None, None, None, None, None)
    assert st == code


def test_null_pointers_and_alignment(lib):
    d = _dims(lib)
    assert lib.LIB.smla_fwd(None, None, None, None, None, None, None, None, None) == 1
    assert lib.LIB.smla_fwd(ctypes.byref(d), None, None, None, None, None, None, None, None) == 1
    p = ctypes.c_void_p(0x1000)
    q = ctypes.c_void_p(0x1008)       # not 16-byte aligned
    assert lib.LIB.smla_fwd(ctypes.byref(d), q, p, p, None, None, p, p, None) == 4
    assert lib.LIB.smla_bwd_preprocess(ctypes.byref(d), None, p, p, None) == 1
    # exact Delta: every input but topk_length / attn_sink is required, q kv dO aligned
    assert lib.LIB.smla_bwd_delta_exact(ctypes.byref(d), p, p, p, p, p, None, None, None, None) == 1
    assert lib.LIB.smla_bwd_delta_exact(ctypes.byref(d), p, p, None, p, p, None, None, p, None) == 1
    assert lib.LIB.smla_bwd_delta_exact(ctypes.byref(d), p, p, q, p, p, None, None, p, None) == 4
    bad = _dims(lib, d_qk=128)
    assert lib.LIB.smla_bwd_delta_exact(ctypes.byref(bad), p, p, p, p, p, None, None, p, None) == 3
    # backward from O: o is required and 16-byte aligned; then the workspace check of smla_bwd
    from_o = lib.LIB.smla_bwd_from_o
    assert from_o(ctypes.byref(d), p, p, p, None, p, p, p, None, None, p, p, None, p, 0, None) == 1
    assert from_o(ctypes.byref(d), p, p, p, q, p, p, p, None, None, p, p, None, p, 0, None) == 4
    assert from_o(ctypes.byref(d), p, p, p, p, p, None, p, None, None, p, p, None, p, 0, None) == 1
    assert from_o(ctypes.byref(d), p, p, p, p, p, p, p, None, None, p, p, None, p, 0, None) == 5
    assert from_o(ctypes.byref(bad), p, p, p, p, p, p, p, None, None, p, p, None, p, 0, None) == 3


def test_empty_problem_is_a_no_op(lib):
    d = _dims(lib, T=0)
    assert lib.LIB.smla_fwd(ctypes.byref(d), None, None, None, None, None, None, None, None) == 0
    assert lib.LIB.smla_bwd_workspace_size(ctypes.byref(d)) == 0
    assert lib.LIB.smla_bwd_delta_exact(ctypes.byref(d), None, None, None, None, None, None, None,
                                        None, None) == 0


def _ws_expected(C, S_kv, H, d_qk, W):
    """The documented workspace layout of smla_bwd for chunks of C tokens,
    each region 256-byte aligned."""
    a = lambda x: (x + 255) // 256 * 256
    Wp = (W + 63) // 64 * 64
    pd = C * H * Wp * 2
    off = a(pd)                          # P
    off = a(off + pd)                    # scale * dS
    nsub = min(256, max(1, (1 << 24) // S_kv), C)
    off = a(off + nsub * S_kv * 4)       # sub-chunk counts
    off = a(off + S_kv * 4)              # row counts
    off = a(off + (S_kv + 1) * 4)        # row offsets
    off = a(off + C * W * 4)             # row lists
    off = a(off + C * Wp * d_qk * 2)     # partials (16 bits per value)
    mp = C * W // 64 + min(S_kv, C * W)
    off = a(off + (S_kv + 1) * 4)        # part offsets
    off = a(off + mp * 4)                # part rows
    off = a(off + mp * d_qk * 4)         # part sums
    return a(off + C * _bwd_splits(C, W) * H * d_qk * 4)   # dQ shares of split blocks


def _bwd_splits(C, W):
    """Block ranges per token in the backward: none from 128 tokens per chunk
    on; below, up to about 256 workgroups, at most one range per block."""
    nb = (W + 63) // 64
    s = 1 if C >= 128 else min(nb, 256 // C)
    if s < 2:
        return 0
    bps = -(-nb // s)
    return -(-nb // bps)


DEFAULT_WS = 8 << 30


def _default_chunk(T, S_kv, H, d_qk, W):
    """Tokens per chunk for the default workspace: all T when that fits the
    8 GiB default, else equal chunks of at most the largest size that fits."""
    if _ws_expected(T, S_kv, H, d_qk, W) <= DEFAULT_WS:
        return T
    c = max(c for c in range(1, T + 1) if _ws_expected(c, S_kv, H, d_qk, W) <= DEFAULT_WS)
    n = -(-T // c)
    return -(-T // n)


def test_workspace_size_and_check(lib):
    d = _dims(lib, T=3, H=5, W=70)
    assert lib.LIB.smla_bwd_workspace_size(ctypes.byref(d)) == _ws_expected(3, 8, 5, 576, 70)
    d2 = _dims(lib, T=300, S_kv=1000, H=128, d_qk=512, W=640)
    assert lib.LIB.smla_bwd_workspace_size(ctypes.byref(d2)) == _ws_expected(300, 1000, 128, 512, 640)
    p = ctypes.c_void_p(0x1000)
    st = lib.LIB.smla_bwd(ctypes.byref(d), p, p, p, p, p, p, None, None, p, p, None, p,
                          ctypes.c_size_t(10), None)
    assert st == 5
    # a sink without a d_sink output
    st = lib.LIB.smla_bwd(ctypes.byref(d), p, p, p, p, p, p, None, p, p, p, None, p,
                          ctypes.c_size_t(1 << 20), None)
    assert st == 1


def test_workspace_is_chunked_past_the_default():
    """The T = 16384 pro shape: all tokens at once would take ~30 GB, so the
    default workspace holds equal token chunks within 8 GiB; a headline-size
    problem is one chunk."""
    from sparse_top_attention_topk_amd import _lib
    pro = (16384, 16384, 128, 512, 1152)
    full = _ws_expected(16384, 16384, 128, 512, 1152)
    assert full > DEFAULT_WS
    got = _lib.smla_bwd_workspace_size(16384, 16384, 128, 512, 512, 1152)
    C = _default_chunk(*pro)
    assert C < 16384 and got == _ws_expected(C, 16384, 128, 512, 1152) <= DEFAULT_WS
    head = _lib.smla_bwd_workspace_size(4096, 4096, 128, 576, 512, 640)
    assert head == _ws_expected(4096, 4096, 128, 576, 640) < DEFAULT_WS


def test_large_kv_sets_are_accepted(lib):
    """More KV rows than one workgroup's LDS counters cover (the inversion
    splits the rows into ranges): sizes are accepted and the workspace grows
    with S_kv only through per-row arrays."""
    d = _dims(lib, T=10, S_kv=100000, H=8, W=64)
    assert lib.LIB.smla_bwd_workspace_size(ctypes.byref(d)) == _ws_expected(10, 100000, 8, 576, 64)
    assert lib.LIB.smla_fwd(ctypes.byref(d), None, None, None, None, None, None, None, None) == 1


def test_profiled_rejects_missing_events(lib):
    d = _dims(lib)
    p = ctypes.c_void_p(0x1000)
    args = [ctypes.byref(d), p, p, p, p, p, p, None, None, p, p, None, p,
            ctypes.c_size_t(1 << 30), None]
    assert lib.LIB.smla_bwd_profiled(*args, None, 7) == 1
    evs = (ctypes.c_void_p * 7)(*([ctypes.c_void_p(0x10)] * 7))
    assert lib.LIB.smla_bwd_profiled(*args, evs, 6) == 2
    evs[3] = None
    assert lib.LIB.smla_bwd_profiled(*args, evs, 7) == 1


def test_noalloc_rejects_before_touching_the_gpu(lib):
    """smla_bwd_noalloc checks sizes first: unsupported dims, and a problem
    whose one-token chunk needs more than the fixed scratch (here a row of
    2^23 slots), are refused before any device call."""
    p = ctypes.c_void_p(0x1000)
    bad = _dims(lib, d_qk=128)
    args = (p, p, p, p, p, p, None, None, p, p, None, None)
    assert lib.LIB.smla_bwd_noalloc(ctypes.byref(bad), *args) == 3
    wide = _dims(lib, W=1 << 23, H=128)
    assert lib.LIB.smla_bwd_noalloc(ctypes.byref(wide), *args) == 7
    assert b"fixed scratch" in lib.LIB.smla_status_string(7)


@pytest.mark.parametrize("shape", [
    (1027, 1027, 64, 576, 192), (300, 300, 64, 576, 192), (128, 256, 128, 576, 1024),
    (320, 320, 96, 512, 160), (4096, 4096, 128, 576, 640), (64, 16384, 128, 576, 1152),
])
def test_chunk_choice_always_fits_its_workspace(shape):
    """For workspaces from one token's need up to all tokens', the chunk the
    backward picks has a layout no larger than the workspace given (below
    128 tokens a smaller chunk can need more, for the dQ shares of split
    blocks), the chunk is at most T, and all tokens' workspace gives T."""
    from sparse_top_attention_topk_amd import _lib
    T, S, H, dqk, W = shape
    one = _ws_expected(1, S, H, dqk, W)
    full = _ws_expected(T, S, H, dqk, W)
    assert _lib.smla_bwd_chunk_tokens(T, S, H, dqk, 512, W, one - 1) == 0
    assert _lib.smla_bwd_chunk_tokens(T, S, H, dqk, 512, W, full) == T
    for c in sorted(set([1, 2, 7, 63, 100, 200, 255, 256, 257, 300, T // 3, T - 1]) & set(range(1, T + 1))):
        for nbytes in (_ws_expected(c, S, H, dqk, W), _ws_expected(c, S, H, dqk, W) + 12345):
            got = _lib.smla_bwd_chunk_tokens(T, S, H, dqk, 512, W, nbytes)
            assert 1 <= got <= T and _ws_expected(got, S, H, dqk, W) <= nbytes, (c, nbytes, got)


def test_forward_split_count():
    """The split forward splits only when the tokens give fewer than 128
    workgroups (of up to 128 heads), then runs tiles of 64 heads and splits
    until about one round of 256 workgroups is filled, never more than one
    split per block nor 64 splits (the merge keeps one per lane)."""
    from sparse_top_attention_topk_amd import _lib
    for T, H, W, want in [(4096, 128, 640, 0), (128, 128, 1152, 0), (1, 128, 1152, 18), (64, 128, 1152, 2),
                          (16, 128, 1152, 8), (1, 8, 64, 0), (1, 128, 1 << 16, 64), (5, 24, 2176, 34)]:
        nb = -(-W // 64)
        ws = _lib.smla_fwd_splitkv_workspace_size(T, 16384, H, 576, 512, W)
        if want == 0:
            assert ws == 0, (T, H, W)
            continue
        bps = -(-nb // want)
        ns = -(-nb // bps)
        a = lambda x: (x + 255) // 256 * 256
        rows = T * ns * H
        assert ws == a(rows * 512 * 4) + a(rows * 16), (T, H, W, ws)
