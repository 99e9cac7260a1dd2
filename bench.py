"""Benchmark: sparse MLA forward + backward on one MI355X.

One step = smla_fwd + smla_bwd_preprocess + smla_bwd over one batch of the
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

Prints ONE JSON line.  ``--gpus N`` with N > 1 is refused: the library runs on
one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
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
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dsv4_flash_h128")
    ap.add_argument("--cpu-tokens", type=int, default=2560,
                    help="tokens of the workload the CPU oracle is timed on")
    ap.add_argument("--no-cpu", action="store_true")
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


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested; the library runs on one GPU only "
              "(no collectives, no sharding).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from sparse_top_attention_topk_amd import _lib, workloads as wl

    dev = torch.device("cuda:0")
    p = wl.make_problem(args.workload)
    n_valid = p.valid_count()
    fwd_flop = 2.0 * p.H * (p.d_qk + p.d_v) * n_valid
    bwd_flop = 2.5 * fwd_flop
    # the pages' timing tables count K = slots per token (W for every token),
    # valid or not: a second figure in that convention, for comparison only
    fwd_flop_nominal = 2.0 * p.H * (p.d_qk + p.d_v) * p.T * p.W
    gathered = n_valid * p.d_qk * 2 + p.T * p.H * (p.d_qk + p.d_v) * 2

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
        _lib.smla_fwd(q, kv, idx, length, sink, p.scale, o=o, lse=lse, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        _lib.smla_bwd_preprocess(o, dO, delta=delta, stream=stream)
        _lib.smla_bwd(q, kv, dO, lse, delta, idx, length, sink, p.scale, dq=dq, dkv=dkv,
                      d_sink=d_sink, workspace=ws, stream=stream,
                      stage_events=None if ev is None else ev[2:])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the timed steps: plain calls (no events between the kernels)
    t0 = time.perf_counter()
    for k in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-stage times: the same steps again with events at the stage boundaries
    evs = [new_events() for _ in range(min(args.steps, 5))]
    torch.cuda.synchronize()
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()

    # the high-accuracy Delta (smla_bwd_delta_exact, in place of the
    # preprocess): timed on its own after the steps, not part of `value`
    delta_x = torch.empty_like(delta)
    _lib.smla_bwd_delta_exact(q, kv, dO, lse, idx, length, sink, p.scale, delta=delta_x, stream=stream)
    ex0, ex1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ex0.record(stream)
    for _ in range(3):
        _lib.smla_bwd_delta_exact(q, kv, dO, lse, idx, length, sink, p.scale, delta=delta_x, stream=stream)
    ex1.record(stream)
    torch.cuda.synchronize()
    delta_exact_ms = ex0.elapsed_time(ex1) / 3

    names = ["fwd", "preprocess"] + list(_lib.BWD_STAGES)
    stage_ms = {nm: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))
                for i, nm in enumerate(names)}
    step_ms = float(np.mean([e[0].elapsed_time(e[-1]) for e in evs]))
    ms_per_step = wall * 1e3 / args.steps
    total_flop = fwd_flop + bwd_flop
    value = total_flop / (ms_per_step * 1e-3) / 1e12
    work = stage_work(p, n_valid)
    dominant = max(stage_ms, key=lambda k: stage_ms[k])
    roofline = roofline_for(dominant, stage_ms[dominant] * 1e-3, work[dominant], p.name)
    fwd_s = stage_ms["fwd"] * 1e-3

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
            "tflops_nominal_k": {
                "fwd": round(fwd_flop_nominal / fwd_s / 1e12, 1),
                "bwd": round(2.5 * fwd_flop_nominal / ((step_ms - stage_ms["fwd"]) * 1e-3) / 1e12, 1),
                "step": round(3.5 * fwd_flop_nominal / (ms_per_step * 1e-3) / 1e12, 1),
            },
            "delta_exact_us": round(delta_exact_ms * 1e3, 1),
            "step_us_exact_delta_mode": round((step_ms - stage_ms["preprocess"] + delta_exact_ms) * 1e3, 1),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


# kernel-name fragment of each timed stage (for the counter profile)
STAGE_KERNEL = {"fwd": ("fwd_kernel",), "preprocess": ("preprocess_kernel",),
                "index_inversion": ("rows_",), "sdp": ("bwd_sdp_kernel",),
                "dq": ("bwd_dq_kernel",), "dkv": ("bwd_dkv_kernel",),
                "dkv_reduce": ("dkv_part_kernel", "dkv_combine_kernel"),
                "dsink": ("dsink_kernel",), "delta_exact": ("delta_exact_kernel",)}


def stage_work(p, n):
    """Algorithmic work per launch of each stage: (FLOP, bytes).  n = valid
    (token, slot) pairs.  Gathered KV rows count 2 * d_qk bytes per valid slot
    (the pages' model); partials are 2 bytes per value per valid slot."""
    T, H, dqk, dv, S, W = p.T, p.H, p.d_qk, p.d_v, p.S_kv, p.W
    return {
        "fwd": (2.0 * H * (dqk + dv) * n, n * dqk * 2 + T * H * (dqk + dv) * 2),
        "preprocess": (0.0, 2 * T * H * dv * 2 + T * H * 4),
        "index_inversion": (0.0, 2 * T * W * 4 + n * 4),
        "sdp": (2.0 * H * (dqk + dv) * n, n * dqk * 2 + T * H * (dqk + dv) * 2 + 2 * H * n * 2),
        "dq": (2.0 * H * dqk * n, n * dqk * 2 + H * n * 2 + T * H * dqk * 2),
        "dkv": (2.0 * H * (dqk + dv) * n, 2 * H * n * 2 + T * H * (dqk + dv) * 2 + n * dqk * 2),
        "dkv_reduce": (0.0, n * dqk * 2 + n * 4 + S * dqk * 4),
        "dsink": (0.0, 2 * T * H * 4),
    }


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_top_attention_topk_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()


def measured_traffic(stage, workload):
    """HBM bytes per launch of the stage's kernel(s) from the committed counter
    profile (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when the
    kernel sources changed since it was taken or it covers another workload."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_dsv4_flash_h128.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except OSError:
        return None
    if rec.get("source_sha256") != source_hash() or rec.get("workload") != workload:
        return None
    frags = STAGE_KERNEL[stage]
    vals = [k["bytes_per_launch"] for name, k in rec["kernels"].items()
            if any(f in name for f in frags)]
    return int(sum(vals)) if vals else None


def roofline_for(stage, seconds, work, workload):
    flop, nbytes = work
    t_mfma = flop / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        achieved, peak, unit, bound = flop / seconds / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = nbytes / seconds / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    return {
        "kernel": stage, "bound": bound, "achieved": round(achieved, 1), "peak": peak,
        "unit": unit, "frac": round(achieved / peak, 4), "traffic": measured_traffic(stage, workload),
        "avg_launch_us": round(seconds * 1e6, 1), "algorithmic_flop": flop,
        "algorithmic_bytes": int(nbytes),
    }


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
