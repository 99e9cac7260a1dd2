"""Benchmark: sparse MLA forward + backward on one MI355X.

One step = smla_fwd (smla_fwd_splitkv when few tokens make the forward split
its blocks) + smla_bwd_preprocess + smla_bwd over one batch of the
synthetic workload (inputs already resident in HBM).  ``value`` comes from the
wall clock around the timed steps (plain calls); the per-stage times in
``detail`` from a few more steps with HIP events at the stage boundaries.  Default workload:
DeepSeek-V4-like H=128, T = S_kv = 4096 causal, d_qk = 576 (512 latent + 64
rope), d_v = 512, window 128 + top-k 512 slots per token, -1 padded,
non-compact, fp32 sink.

FLOP convention of the pages ([flash-attn #2882] Performance): forward
2 * H * K * (d_qk + d_v) per token with K the valid gathered slots, backward
2.5x the forward.  Gathered bytes (the pages' TB/s model): gathered KV rows
(K * d_qk * 2 bytes per token) + Q read + O write.

Roofline (``roofline`` for the longest stage, ``detail.stage_roofline`` for
all): the method's own work per launch in the units of the hot-path table
(FLOP of the products a stage computes; bytes of the method's inputs and
outputs it touches, gathered KV rows counted per valid slot) against the
MI355X peaks, with the binding roof the one whose ideal time is longer.  The
library's intermediate buffers are not the method's bytes; the measured HBM
traffic of the stage (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated,
from profiles/) is reported next to them with its ratio, and the MFMA busy
share from the counter profile.

``detail.configs``: the other DeepSeek-V4-like workloads (H = 64, d = 512;
T = 16384 pro) timed the same way with fewer steps (``--no-detail`` skips).

Prints ONE JSON line.  ``--gpus N`` with N > 1 is refused: the library runs on
one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-MLA fwd+bwd TFLOPS & gather TB/s, H=128 T=4096 topk=512, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0       # dense bf16 MFMA, MI355X
PEAK_HBM_GBS = 8000.0           # HBM3E, MI355X


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    # the GPU's clocks settle over the first ~5 steps (kernel traces show
    # the first calls of each kernel 5-30 % slower)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv4_flash_h128")
    ap.add_argument("--cpu-tokens", type=int, default=2560,
                    help="tokens of the workload the CPU oracle is timed on")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-detail", action="store_true",
                    help="skip timing the other DeepSeek-V4-like configurations")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    return ap.parse_args()


def calibrate_copy():
    """A plain copy of known size (1 GiB read + 1 GiB written per launch), to
    scale the FETCH_SIZE / WRITE_SIZE counters of the same profiler runs."""
    dev = torch.device("cuda:0")
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}), flush=True)


def run_workload(p, steps, warmup, n_event_steps=5, exact_delta=True):
    """Time ``steps`` plain steps of problem p (inputs resident in HBM) and a
    few more with HIP events at the stage boundaries.  Returns a dict of
    times in ms."""
    from sparse_top_attention_topk_amd import _lib

    dev = torch.device("cuda:0")
    q, kv, dO = p.q.to(dev), p.kv.to(dev), p.dO.to(dev)
    idx = p.topk_idxs.to(dev)
    length = None if p.topk_length is None else p.topk_length.to(dev)
    sink = None if p.attn_sink is None else p.attn_sink.to(dev)
    o = torch.empty((p.T, p.H, p.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((p.T, p.H), dtype=torch.float32, device=dev)
    delta = torch.empty((p.T, p.H), dtype=torch.float32, device=dev)
    dq = torch.empty_like(q)
    dkv = torch.empty((p.S_kv, p.d_qk), dtype=torch.float32, device=dev)
    d_sink = torch.empty((p.H,), dtype=torch.float32, device=dev) if sink is not None else None
    ws_bytes = _lib.smla_bwd_workspace_size(p.T, p.S_kv, p.H, p.d_qk, p.d_v, p.W, p.scale)
    ws = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device=dev)
    # few tokens: the forward splits each token's blocks (none at the headline)
    fws_bytes = _lib.smla_fwd_splitkv_workspace_size(p.T, p.S_kv, p.H, p.d_qk, p.d_v, p.W, p.scale)
    fws = torch.empty((max(fws_bytes, 16),), dtype=torch.uint8, device=dev) if fws_bytes else None
    stream = torch.cuda.current_stream(dev)   # the library launches on this stream

    # events: [fwd start, fwd end = preprocess start, preprocess end = bwd stage 0, bwd stages...]
    nb = len(_lib.BWD_STAGES) + 1

    def new_events():
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 + nb)]
        for e in evs:          # materialise the HIP event handles
            e.record(stream)
        return evs

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if fws is None:
            _lib.smla_fwd(q, kv, idx, length, sink, p.scale, o=o, lse=lse, stream=stream)
        else:
            _lib.smla_fwd_splitkv(q, kv, idx, length, sink, p.scale, o=o, lse=lse, workspace=fws, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        _lib.smla_bwd_preprocess(o, dO, delta=delta, stream=stream)
        _lib.smla_bwd(q, kv, dO, lse, delta, idx, length, sink, p.scale, dq=dq, dkv=dkv,
                      d_sink=d_sink, workspace=ws, stream=stream,
                      stage_events=None if ev is None else ev[2:])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # the timed steps: plain calls (no events between the kernels)
    t0 = time.perf_counter()
    for k in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-stage times: the same steps again with events at the stage boundaries
    evs = [new_events() for _ in range(max(1, min(steps, n_event_steps)))]
    torch.cuda.synchronize()
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()

    out = {"ms_per_step": wall * 1e3 / steps, "ws_bytes": ws_bytes, "fwd_ws_bytes": fws_bytes}
    names = ["fwd", "preprocess"] + list(_lib.BWD_STAGES)
    out["stage_ms"] = {nm: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))
                       for i, nm in enumerate(names)}
    out["step_ms_events"] = float(np.mean([e[0].elapsed_time(e[-1]) for e in evs]))

    if exact_delta:
        # the high-accuracy Delta (smla_bwd_delta_exact, in place of the
        # preprocess): timed on its own after the steps, not part of `value`
        delta_x = torch.empty_like(delta)
        _lib.smla_bwd_delta_exact(q, kv, dO, lse, idx, length, sink, p.scale, delta=delta_x, stream=stream)
        ex0, ex1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ex0.record(stream)
        for _ in range(3):
            _lib.smla_bwd_delta_exact(q, kv, dO, lse, idx, length, sink, p.scale, delta=delta_x,
                                      stream=stream)
        ex1.record(stream)
        torch.cuda.synchronize()
        out["delta_exact_ms"] = ex0.elapsed_time(ex1) / 3
    del q, kv, dO, idx, o, lse, delta, dq, dkv, ws
    torch.cuda.empty_cache()
    return out


def flops_and_bytes(p):
    n_valid = p.valid_count()
    fwd_flop = 2.0 * p.H * (p.d_qk + p.d_v) * n_valid
    # the pages' timing tables count K = slots per token (W for every token),
    # valid or not: a second figure in that convention, for comparison only
    fwd_flop_nominal = 2.0 * p.H * (p.d_qk + p.d_v) * p.T * p.W
    gathered = n_valid * p.d_qk * 2 + p.T * p.H * (p.d_qk + p.d_v) * 2
    return n_valid, fwd_flop, 2.5 * fwd_flop, fwd_flop_nominal, gathered


def config_line(p, t):
    """Times and rates of one workload (fwd, bwd incl. preprocess, step)."""
    n_valid, fwd_flop, bwd_flop, nominal, gathered = flops_and_bytes(p)
    fwd_ms = t["stage_ms"]["fwd"]
    bwd_ms = t["step_ms_events"] - fwd_ms
    return {
        "T": p.T, "H": p.H, "d_qk": p.d_qk, "W": p.W, "valid_slots": n_valid,
        "fwd_us": round(fwd_ms * 1e3, 1), "bwd_us": round(bwd_ms * 1e3, 1),
        "step_us": round(t["ms_per_step"] * 1e3, 1),
        "step_tflops": round((fwd_flop + bwd_flop) / (t["ms_per_step"] * 1e-3) / 1e12, 1),
        "fwd_tflops": round(fwd_flop / (fwd_ms * 1e-3) / 1e12, 1),
        "bwd_tflops": round(bwd_flop / (bwd_ms * 1e-3) / 1e12, 1),
        "fwd_gathered_tbs": round(gathered / (fwd_ms * 1e-3) / 1e12, 3),
        "workspace_gb": round(t["ws_bytes"] / 1e9, 3),
    }


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested; the library runs on one GPU only "
              "(no collectives, no sharding).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from sparse_top_attention_topk_amd import workloads as wl

    p = wl.make_problem(args.workload)
    n_valid, fwd_flop, bwd_flop, fwd_flop_nominal, gathered = flops_and_bytes(p)
    t = run_workload(p, args.steps, args.warmup)
    stage_ms, step_ms, ms_per_step = t["stage_ms"], t["step_ms_events"], t["ms_per_step"]
    total_flop = fwd_flop + bwd_flop
    value = total_flop / (ms_per_step * 1e-3) / 1e12
    work = stage_work(p, n_valid)
    dominant = max((k for k in stage_ms if k in work), key=lambda k: stage_ms[k])
    roofline = roofline_for(dominant, stage_ms[dominant] * 1e-3, work[dominant], p.name)
    fwd_s = stage_ms["fwd"] * 1e-3

    # the other DeepSeek-V4-like configurations, timed the same way (fewer steps)
    configs = {}
    if not args.no_detail:
        for name in ("dsv4_flash_h64", "dsv4_pro"):
            if name == args.workload:
                continue
            q = wl.make_problem(name)
            configs[name] = config_line(q, run_workload(q, 3, 1, n_event_steps=2, exact_delta=False))
            del q

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(p, args.cpu_tokens)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": p.name,
            "T": p.T, "S_kv": p.S_kv, "H": p.H, "d_qk": p.d_qk, "d_v": p.d_v, "W": p.W,
            "window": p.meta.get("window"), "topk": p.meta.get("topk"),
            "layout": "compact" if p.topk_length is not None else "non-compact",
            "sink": p.attn_sink is not None, "valid_slots": n_valid,
        },
        "detail": {
            "stage_us": {k: round(v * 1e3, 1) for k, v in stage_ms.items()},
            "fwd_us": round(stage_ms["fwd"] * 1e3, 1),
            "bwd_us": round((step_ms - stage_ms["fwd"]) * 1e3, 1),
            "step_us_events": round(step_ms * 1e3, 1),
            "fwd_tflops": round(fwd_flop / fwd_s / 1e12, 1),
            "bwd_tflops": round(bwd_flop / ((step_ms - stage_ms["fwd"]) * 1e-3) / 1e12, 1),
            "fwd_gathered_tbs": round(gathered / fwd_s / 1e12, 3),
            "fwd_gathered_frac_hbm": round(gathered / fwd_s / 1e9 / PEAK_HBM_GBS, 4),
            "fwd_mfma_frac": round(fwd_flop / fwd_s / 1e12 / PEAK_BF16_TFLOPS, 4),
            "fwd_bwd_mfma_frac": round(value / PEAK_BF16_TFLOPS, 4),
            "fwd_flop": fwd_flop, "bwd_flop": bwd_flop, "gathered_bytes_fwd": gathered,
            "workspace_gb": round(t["ws_bytes"] / 1e9, 3),
            "tflops_nominal_k": {
                "fwd": round(fwd_flop_nominal / fwd_s / 1e12, 1),
                "bwd": round(2.5 * fwd_flop_nominal / ((step_ms - stage_ms["fwd"]) * 1e-3) / 1e12, 1),
                "step": round(3.5 * fwd_flop_nominal / (ms_per_step * 1e-3) / 1e12, 1),
            },
            "stage_roofline": {k: roofline_for(k, stage_ms[k] * 1e-3, work[k], p.name, brief=True)
                               for k in stage_ms if k in work},
            "delta_exact_us": round(t["delta_exact_ms"] * 1e3, 1),
            "step_us_exact_delta_mode": round((step_ms - stage_ms["preprocess"] + t["delta_exact_ms"]) * 1e3, 1),
            "configs": configs,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


# kernel-name fragment of each timed stage (for the counter profile)
STAGE_KERNEL = {"fwd": ("fwd_kernel",), "preprocess": ("preprocess_kernel",),
                "index_inversion": ("rows_",), "sdp_dq": ("bwd_sdq_kernel",),
                "dq_merge": ("dq_reduce_kernel",), "dkv": ("bwd_dkv_kernel",),
                "dkv_reduce": ("dkv_part_kernel", "dkv_combine_kernel"),
                "dsink": ("dsink_kernel",), "delta_exact": ("delta_exact_kernel",)}


def stage_work(p, n):
    """The method's algorithmic work per launch of each stage, in the units of
    the hot-path table: (FLOP, bytes).  n = valid (token, slot) pairs.  A
    valid slot is 2 H (d_qk + d_v) FLOP of S and PV (forward), of S and dP
    (recompute) and of dK and dV, and 2 H d_qk of dQ; gathered KV rows count
    2 d_qk bytes per valid slot (the pages' model).  Per token: q, O, dO, dQ
    are 2 H d bytes each.  The library's own intermediate buffers (P and dS,
    the per-slot dKV partials) are not the method's bytes: they show up in the
    measured traffic, which is reported next to these."""
    T, H, dqk, dv, S, W = p.T, p.H, p.d_qk, p.d_v, p.S_kv, p.W
    qb, ob = T * H * dqk * 2, T * H * dv * 2
    gath = n * dqk * 2
    return {
        "fwd": (2.0 * H * (dqk + dv) * n, gath + qb + ob + T * W * 4 + T * H * 4),
        "preprocess": (0.0, 2 * ob + T * H * 4),
        "index_inversion": (0.0, T * W * 4),
        "sdp_dq": (2.0 * H * (dqk + dv) * n + 2.0 * H * dqk * n, gath + 2 * qb + ob),
        "dkv": (2.0 * H * (dqk + dv) * n, qb + ob),
        "dkv_reduce": (0.0, S * dqk * 4),
        "dsink": (0.0, 2 * T * H * 4),
    }


_CODE_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)


def _strip_comments(text):
    """C/C++ source without comments, trailing blanks and empty lines (string
    and character literals kept as written)."""
    text = _CODE_TOKENS.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def source_hash():
    """sha256 over the kernel sources' code: comments and layout do not count,
    so that an edit of the documentation keeps a profile taken on the same code
    valid, while any change to the code voids it."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_top_attention_topk_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if not f.endswith((".hip", ".h", ".cpp")):
            continue
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + _strip_comments(fh.read()).encode())
    return h.hexdigest()


def _profile(fname, workload):
    """A committed counter profile (JSON) if it was taken on this workload with
    the current kernel sources, else None."""
    try:
        with open(os.path.join(ROOT, "profiles", fname)) as f:
            rec = json.load(f)
    except OSError:
        return None
    if rec.get("source_sha256") != source_hash() or rec.get("workload") != workload:
        return None
    return rec


def _per_stage(rec, stage, key, combine=sum):
    frags = STAGE_KERNEL[stage]
    vals = [k[key] for name, k in rec["kernels"].items() if any(f in name for f in frags) and key in k]
    return combine(vals) if vals else None


def measured_traffic(stage, workload):
    """HBM bytes per launch of the stage's kernel(s) from the committed counter
    profile (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when the
    kernel sources changed since it was taken or it covers another workload."""
    rec = _profile("hbm_traffic_dsv4_flash_h128.json", workload)
    if rec is None:
        return None
    v = _per_stage(rec, stage, "bytes_per_launch")
    return None if v is None else int(v)


def measured_mfma_util(stage, workload):
    """MFMA busy share of the stage's main kernel from the committed counter
    profile: sum over SIMDs of SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x
    1024 SIMDs), the rocprofv3 MfmaUtil definition; None if unavailable."""
    rec = _profile("mfma_util_dsv4_flash_h128.json", workload)
    if rec is None:
        return None
    return _per_stage(rec, stage, "mfma_util", combine=max)


def roofline_for(stage, seconds, work, workload, brief=False):
    """Roofline of one stage in the method's units: the binding roof is the
    one with the longer ideal time (FLOP at the bf16 MFMA peak, or bytes at
    the HBM peak); achieved = the method's work / the stage's event-timed
    duration."""
    flop, nbytes = work
    t_mfma = flop / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        achieved, peak, unit, bound = flop / seconds / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = nbytes / seconds / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    traffic = measured_traffic(stage, workload)
    out = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
           "frac": round(achieved / peak, 4), "avg_launch_us": round(seconds * 1e6, 1)}
    if brief:
        return out
    out.update({
        "kernel": stage, "traffic": traffic,
        "traffic_over_algorithmic_bytes": None if traffic is None else round(traffic / nbytes, 3),
        "mfma_util_counters": measured_mfma_util(stage, workload),
        "algorithmic_flop": flop, "algorithmic_bytes": int(nbytes),
    })
    return out


def cpu_baseline(p, n_tokens):
    """The fp64 oracle, as it stands, on the last n_tokens tokens of the same
    workload (full-width rows), forward + backward, on this host's cores."""
    import oracle
    toks = np.arange(max(0, p.T - n_tokens), p.T)
    tk = torch.from_numpy(toks)
    x = dict(q=p.q[tk].double().numpy(), kv=p.kv.double().numpy(), dO=p.dO[tk].double().numpy(),
             idx=p.topk_idxs[tk].numpy(),
             length=None if p.topk_length is None else p.topk_length[tk].numpy(),
             sink=None if p.attn_sink is None else p.attn_sink.double().numpy())
    idx = x["idx"]
    ok = (idx >= 0) & (idx < p.S_kv)
    if x["length"] is not None:
        ok &= np.arange(p.W)[None, :] < np.clip(x["length"], 0, p.W)[:, None]
    n_valid = int(ok.sum())
    flop = 3.5 * 2.0 * p.H * (p.d_qk + p.d_v) * n_valid
    t0 = time.perf_counter()
    oracle.oracle_fwd(x["q"], x["kv"], idx, x["length"], x["sink"], p.scale, p.d_v)
    oracle.oracle_bwd(x["q"], x["kv"], x["dO"], idx, x["length"], x["sink"], p.scale, p.d_v)
    dt = time.perf_counter() - t0
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:
        pass
    return {
        "value": round(flop / dt / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": threads or os.cpu_count(),
        "kind": "oracle",
        "sample": f"fwd+bwd of the last {len(toks)} tokens ({n_valid} valid slots) of {p.name}, "
                  f"fp64 NumPy, {dt:.1f} s",
    }


if __name__ == "__main__":
    main()
