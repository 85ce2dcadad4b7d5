"""Benchmark of the pi0 action-expert denoise loop on one MI355X.

One "step" is one pi0x_denoise call: the whole num_steps-Euler loop over one
batch of synthetic inputs already resident in device memory, replayed from its
captured hipGraph.  The default workload is the bf16 pi0 expert at batch 64
(prefix 816, horizon 50 x 32, 10 Euler steps); the batch-1 latency workload
is measured in the same run and reported under "b1", and the prefix pass that
produces the K/V cache (the Gemma-2B-shaped PaliGemma language model over an
816-token prefix at batch 1) under "prefill".

Output: one JSON line with the throughput (action chunks/s), the roofline
figure of the dominant kernel (per-launch algorithmic bytes or flops over its
average duration, from HIP events around that kernel's launches in an eager
pass of the same loop), and the fp64 CPU oracle timed on a bounded sample on
this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "action chunks/s, 10-step π0 expert denoise at B=1 & B=64; % of roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
MFMA_FP32_PEAK_TFS = 157.3   # MI355X fp32 matrix
BALANCE = 312.5              # flop per byte at which bf16 MFMA and HBM peaks meet


def algorithmic_counts(shape, batch: int, valid: np.ndarray, num_steps: int, esz: int):
    """Bytes and flops of one denoise call, counted as the method defines it:
    every expert and head weight once per Euler step, the visible prefix K/V
    once per step, the action state in and out; 51 suffix tokens per sample and
    only visible keys in attention.  Intermediates are not counted."""
    from vla_flow_matching_amd import synth
    s = shape
    params = synth.weight_count(s)
    kv_bytes = int(np.sum(valid)) * s.depth * 2 * s.num_kv_heads * s.head_dim * esz
    io = batch * s.horizon * s.action_dim * 4 * 2 + batch * s.state_dim * 4
    bytes_step = params * esz + kv_bytes
    W, M, qd, kd = s.width, s.mlp_dim, s.num_heads * s.head_dim, s.num_kv_heads * s.head_dim
    dense_params = s.depth * (W * (qd + 2 * kd) + qd * W + 3 * M * W)
    S = s.suffix_len
    dense = 2.0 * dense_params * S * batch
    per_pair = 4.0 * s.head_dim  # q.k and p*v multiply-adds per (query head, key)
    attn = 0.0
    for v in valid:
        attn += s.depth * s.num_heads * per_pair * (s.horizon * (int(v) + S) + (int(v) + 1))
    head = 2.0 * batch * (s.state_dim * W + s.horizon * (s.action_dim * W + 2 * W * W + W * W + W * s.action_dim))
    return {"bytes": bytes_step * num_steps + io, "flops": (dense + attn + head) * num_steps,
            "bytes_per_step": bytes_step, "flops_per_step": dense + attn + head}


def kernel_unit_counts(shape, batch: int, esz: int, valid: np.ndarray):
    """Algorithmic bytes and flops of one launch of each kernel class."""
    s = shape
    W, M, qd, dh = s.width, s.mlp_dim, s.num_heads * s.head_dim, s.head_dim
    R = batch * s.suffix_len
    nqkv = qd + 2 * dh
    vis = float(np.sum(valid)) / max(batch, 1)
    return {
        "gate_up": {"bytes": (2 * M * W + R * W + R * M) * esz, "flops": 2.0 * R * 2 * M * W},
        "down": {"bytes": (W * M + R * M) * esz + R * W * 4 * 2, "flops": 2.0 * R * W * M},
        "qkv_rope": {"bytes": (nqkv * W + R * W + R * nqkv) * esz, "flops": 2.0 * R * nqkv * W},
        "o_proj": {"bytes": (W * qd + R * qd) * esz + R * W * 4 * 2, "flops": 2.0 * R * W * qd},
        "attention": {"bytes": (batch * vis * 2 * dh + R * (qd + 2 * dh) + R * qd) * esz,
                      "flops": batch * s.num_heads * 4.0 * dh * (s.horizon * (vis + s.suffix_len) + vis + 1)},
    }


def prefill_counts(shape, batch: int, valid: np.ndarray, L: int, esz: int):
    """Algorithmic bytes and flops of one prefix pass, counted for what the
    cache needs: every layer in full except the last, which only needs its
    q/k/v projection (its attention output and MLP feed the discarded prefix
    output); real tokens only, real keys only; weights once, embeddings in and
    the cache out.  Norm weights are not counted."""
    s = shape
    W, M, qd, kd, dh = s.width, s.mlp_dim, s.num_heads * s.head_dim, s.num_kv_heads * s.head_dim, s.head_dim
    qkv = W * (qd + 2 * kd)
    full = qkv + qd * W + 3 * M * W
    params = (s.depth - 1) * full + qkv
    rows = float(np.sum(valid))
    dense = 2.0 * params * rows
    attn = (s.depth - 1) * s.num_heads * 4.0 * dh * float(np.sum(np.asarray(valid, np.float64) ** 2))
    nbytes = params * esz + batch * L * W * esz + s.depth * 2 * batch * L * kd * esz
    unit_rows = batch * L  # rows one launch computes (padding included)
    units = {"gate_up": {"flops": 2.0 * unit_rows * 2 * M * W, "bytes": (2 * M * W + unit_rows * (W + M)) * esz},
             "down": {"flops": 2.0 * unit_rows * W * M, "bytes": (W * M + unit_rows * M) * esz + unit_rows * W * 8},
             "qkv_rope": {"flops": 2.0 * unit_rows * (qd + 2 * kd) * W,
                          "bytes": ((qd + 2 * kd) * W + unit_rows * (W + qd + 3 * kd)) * esz},
             "o_proj": {"flops": 2.0 * unit_rows * W * qd, "bytes": (W * qd + unit_rows * qd) * esz + unit_rows * W * 8}}
    return {"bytes": nbytes, "flops": dense + attn, "units": units}


def run_prefill(name: str, steps: int, warmup: int, timing_calls: int = 2):
    import torch
    from vla_flow_matching_amd import binding, synth

    w = synth.PREFILL_WORKLOADS[name]
    s = w.shape
    esz = 2 if w.dtype == "bf16" else 4
    blob = synth.make_prefill_weights(s, seed=w.seed, dtype=w.dtype)
    inputs = synth.make_prefill_inputs(w)
    cfg = binding.make_config(s, w.dtype, max_batch=w.batch, max_prefix_len=w.prefix_len)
    pm = binding.PrefixModel(cfg, blob)
    del blob
    d = binding.prefill_device_inputs(inputs, w.dtype)
    kv = torch.empty((s.depth, 2, w.batch, w.prefix_len, s.head_dim), dtype=d["embeddings"].dtype, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        pm.prefill(d["embeddings"], d["valid_len"], out=kv)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        call()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    pm.set_timing(True)
    for _ in range(timing_calls):
        call()
    timing = pm.read_timing()
    pm.set_timing(False)
    pm.close()
    valid = inputs["valid_len"]
    c = prefill_counts(s, w.batch, valid, w.prefix_len, esz)
    kern = {k: {"avg_us": 1e3 * tot / n, "launches_per_call": n // timing_calls} for k, (tot, n) in timing.items() if n}
    dom = max((k for k in kern if k in c["units"]), key=lambda k: kern[k]["avg_us"] * kern[k]["launches_per_call"])
    u = c["units"][dom]
    peak = MFMA_BF16_PEAK_TFS if esz == 2 else MFMA_FP32_PEAK_TFS
    ach = u["flops"] / (kern[dom]["avg_us"] * 1e-6) / 1e12
    sec = ms * 1e-3
    return {"workload": w.name, "batch": w.batch, "prefix_len": w.prefix_len, "real_tokens": int(np.sum(valid)),
            "ms_per_call": ms, "prefixes_per_s": w.batch / sec,
            "whole_pass": {"achieved_TFLOPs": c["flops"] / sec / 1e12, "mfma_frac": c["flops"] / sec / 1e12 / peak,
                           "flops_per_call": c["flops"], "bytes_per_call": c["bytes"],
                           "achieved_GBps": c["bytes"] / sec / 1e9},
            "roofline": {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                         "frac": ach / peak, "traffic": None,
                         "per_launch": {"flops": u["flops"], "bytes": u["bytes"], "avg_us": kern[dom]["avg_us"]}},
            "kernels": kern}


def code_text(src: bytes) -> bytes:
    """C/C++ source with comments and whitespace runs removed (the sources
    hold no string literal with a comment marker in it)."""
    import re
    src = re.sub(rb"/\*.*?\*/", b" ", src, flags=re.S)
    src = re.sub(rb"//[^\n]*", b" ", src)
    return re.sub(rb"\s+", b" ", src).strip()


def csrc_digest() -> str:
    """sha256 over the code (comments and layout stripped) of the HIP sources
    and the C header, to tell whether kernel code changed since HBM byte
    counters were taken."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "vla_flow_matching_amd", "csrc")
    # the kernels' sources and the header (not the C++ driver that only calls the ABI)
    for p in sorted(f for f in os.listdir(csrc) if f != "denoise_driver.cpp") + ["../../include/pi0x.h"]:
        with open(os.path.join(csrc, p), "rb") as f:
            h.update(p.encode() + b"\0" + code_text(f.read()))
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of a kernel class from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE passes (already scaled by the copy-kernel
    calibration), or None when absent or taken on different kernel code."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    e = table.get(workload, {}).get(kernel)
    if not e or e.get("csrc_sha256") != csrc_digest():
        return None
    return float(e["bytes_per_launch"])


def _profile_entry(filename: str, workload: str):
    """A workload's entry of a committed counter summary in profiles/, or None
    when absent or taken on different kernel code."""
    try:
        with open(os.path.join(ROOT, "profiles", filename)) as f:
            e = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not e or e.get("csrc_sha256") != csrc_digest():
        return None
    return e


def measured_mfma_busy(workload: str, kernel: str):
    """Share of the kernel's SIMD-cycles with the matrix pipe busy, from the
    committed SQ_VALU_MFMA_BUSY_CYCLES / SQ_BUSY_CYCLES pass, or None."""
    e = _profile_entry("mfma_busy.json", workload)
    return None if e is None else e.get("mfma_busy", {}).get(kernel)


def measured_call_bytes(workload: str):
    """HBM bytes of one call (all kernels, scaled FETCH_SIZE + WRITE_SIZE), or None."""
    e = _profile_entry("hbm_traffic.json", workload)
    return None if e is None or "per_call_bytes" not in e else float(e["per_call_bytes"])


def run_workload(name: str, steps: int, warmup: int, timing_calls: int = 2, latency_calls: int = 100):
    import torch
    from vla_flow_matching_amd import binding, synth

    w = synth.WORKLOADS[name]
    s = w.shape
    esz = 2 if w.dtype == "bf16" else 4
    blob = synth.make_weights(s, seed=w.seed, dtype=w.dtype)
    inputs = synth.make_inputs(w)
    cfg = binding.make_config(s, w.dtype, max_batch=w.batch, max_prefix_len=w.prefix_len, max_steps=w.num_steps)
    ex = binding.Expert(cfg, blob)
    del blob
    d = binding.device_inputs(inputs, w.dtype)
    out = torch.empty_like(d["noise"])
    stream = torch.cuda.current_stream()

    def call():
        ex.denoise(d["prefix_kv"], d["valid_len"], d["state"], d["noise"], w.num_steps, out=out)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        call()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    assert np.all(np.isfinite(out.cpu().numpy())), "non-finite actions"

    # per-launch latency distribution: each call bracketed by its own events
    lat = []
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(latency_calls)]
    for a, b in evs:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    lat = sorted(a.elapsed_time(b) for a, b in evs)
    pct = lambda q: float(np.percentile(lat, q)) if lat else None
    dist = {"median_ms": pct(50), "p10_ms": pct(10), "p90_ms": pct(90), "launches": len(lat)}

    # per-kernel durations: the same loop launched eagerly with HIP events
    ex.set_timing(True)
    for _ in range(timing_calls):
        call()
    timing = ex.read_timing()
    ex.set_timing(False)
    ex.close()

    valid = inputs["valid_len"]
    counts = algorithmic_counts(s, w.batch, valid, w.num_steps, esz)
    units = kernel_unit_counts(s, w.batch, esz, valid)
    kern = {}
    for k, (tot, n) in timing.items():
        if n:
            kern[k] = {"avg_us": 1e3 * tot / n, "launches_per_call": n // timing_calls,
                       "share": tot / max(sum(t for t, _ in timing.values()), 1e-12)}
    dom = max((k for k in kern if k in units), key=lambda k: kern[k]["avg_us"] * kern[k]["launches_per_call"])
    u = units[dom]
    avg_s = kern[dom]["avg_us"] * 1e-6
    intensity = u["flops"] / u["bytes"]
    if intensity < BALANCE:
        roof = {"bound": "hbm", "achieved": u["bytes"] / avg_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        peak = MFMA_BF16_PEAK_TFS if esz == 2 else MFMA_FP32_PEAK_TFS
        roof = {"bound": "mfma", "achieved": u["flops"] / avg_s / 1e12, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(name, dom)
    # counter-derived rates: the measured HBM bytes over the same launch time,
    # and the matrix pipes' busy share from the MFMA counters
    roof["traffic_GBps"] = roof["traffic"] / avg_s / 1e9 if roof["traffic"] else None
    roof["mfma_busy"] = measured_mfma_busy(name, dom)
    roof["kernel"] = dom
    roof["per_launch"] = {"bytes": u["bytes"], "flops": u["flops"], "avg_us": kern[dom]["avg_us"]}
    sec = ms * 1e-3
    whole = {"achieved_GBps": counts["bytes"] / sec / 1e9, "hbm_frac": counts["bytes"] / sec / 1e9 / HBM_PEAK_GBS,
             "achieved_TFLOPs": counts["flops"] / sec / 1e12,
             "mfma_frac": counts["flops"] / sec / 1e12 / (MFMA_BF16_PEAK_TFS if esz == 2 else MFMA_FP32_PEAK_TFS),
             "bytes_per_call": counts["bytes"], "flops_per_call": counts["flops"]}
    cb = measured_call_bytes(name)
    whole["counter_bytes_per_call"] = cb
    whole["counter_GBps"] = cb / sec / 1e9 if cb else None
    return {"workload": w, "ms": ms, "value": w.batch / sec, "roofline": roof, "kernels": kern, "whole_loop": whole,
            "latency": dist, "inputs": inputs}


def copy_bandwidth(mib: int = 1024, reps: int = 10) -> dict:
    """Achievable HBM bandwidth on this GPU: a device-to-device copy of `mib`
    MiB (read + write counted), the reference for the roofline's bytes."""
    import torch
    n = mib << 18  # float32 elements
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    sec = t0.elapsed_time(t1) * 1e-3 / reps
    del src, dst
    return {"GBps": 2.0 * n * 4 / sec / 1e9, "bytes_per_copy": 2 * n * 4,
            "kind": "device-to-device copy (torch copy_), read + write bytes"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_tiny_one_thread() -> dict:
    """The fp64 oracle on one thread for the tiny configuration (width 256,
    depth 2, batch 1, prefix 64, 2 steps): one whole chunk."""
    from oracle import oracle
    from vla_flow_matching_amd import synth
    w = synth.WORKLOADS["tiny_fp32_b1"]
    blob = synth.make_weights(w.shape, seed=w.seed, dtype=w.dtype)
    inputs = synth.make_inputs(w)
    prev = oracle.set_threads(0)
    oracle.set_threads(1)
    o = oracle.Oracle(w.shape, blob)
    t0 = time.perf_counter()
    o.denoise_batch(inputs, w.num_steps)
    sec = time.perf_counter() - t0
    oracle.set_threads(prev)
    return {"workload": w.name, "chunks_per_s": 1.0 / sec, "threads": 1}


def cpu_baseline(w, inputs, budget_s: float = 12.0):
    """fp64 oracle on this host's cores: sequential velocity evaluations of
    sample 0's chunk until the budget is spent (at most one whole chunk)."""
    from oracle import oracle
    from vla_flow_matching_amd import synth
    cores = len(os.sched_getaffinity(0))
    threads = oracle.set_threads(cores)
    blob = synth.make_weights(w.shape, seed=w.seed, dtype=w.dtype)
    o = oracle.Oracle(w.shape, blob)
    del blob
    kv = inputs["prefix_kv"][:, :, 0]
    L, v = w.prefix_len, int(inputs["valid_len"][0])
    x = inputs["noise"][0].astype(np.float64)
    dt = -1.0 / w.num_steps
    n, t0 = 0, time.perf_counter()
    while n < w.num_steps and (n == 0 or time.perf_counter() - t0 < budget_s):
        vel = o.velocity(inputs["state"][0], x, oracle.step_time(n, w.num_steps), kv, L, v)
        x = x + dt * vel
        n += 1
    per_eval = (time.perf_counter() - t0) / n
    return {"value": 1.0 / (per_eval * w.num_steps), "unit": "chunks/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of the {w.num_steps} Euler velocity evaluations of sample 0 (L={L}, valid {v}), "
                      f"fp64, {per_eval:.2f} s each; chunks/s = 1 / ({w.num_steps} x time per evaluation)",
            "cpu_model": cpu_model(), "tiny_one_thread": cpu_tiny_one_thread()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="pi0_bf16_b64")
    ap.add_argument("--b1-workload", default="pi0_bf16_b1", help="secondary latency workload ('' to skip)")
    ap.add_argument("--ragged-workload", default="pi0_bf16_b16_ragged",
                    help="ragged-prefix workload reported under 'ragged' ('' to skip)")
    ap.add_argument("--prefill-workload", default="paligemma_bf16_b1",
                    help="prefix-pass workload reported under 'prefill' ('' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-bandwidth", dest="copy_bandwidth", action="store_false",
                    help="skip the device-copy bandwidth reference")
    ap.add_argument("--latency-calls", type=int, default=100,
                    help="calls timed one by one for the latency median / p10 / p90 (0 to skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB (a known-size reference "
                         "kernel for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the denoise loop shards by "
              f"sample with no exchange, so N GPUs run N independent copies)", file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.set_device(0)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 18  # float32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    main_res = run_workload(args.workload, args.steps, args.warmup, latency_calls=args.latency_calls)
    w = main_res["workload"]
    line = {
        "metric": METRIC, "value": main_res["value"], "unit": "chunks/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": main_res["ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "prefix_len": w.prefix_len, "num_steps": w.num_steps,
                   "horizon": w.shape.horizon, "action_dim": w.shape.action_dim, "layers": w.shape.depth, "width": w.shape.width},
        "roofline": main_res["roofline"],
        "whole_loop": main_res["whole_loop"],
        "kernels": main_res["kernels"],
        "latency": main_res["latency"],
    }
    if args.b1_workload:
        r = run_workload(args.b1_workload, max(args.steps, 20), args.warmup, latency_calls=args.latency_calls)
        line["b1"] = {"workload": r["workload"].name, "chunks_per_s": r["value"], "latency_ms": r["ms"],
                      "latency": r["latency"], "roofline": r["roofline"], "whole_loop": r["whole_loop"],
                      "kernels": r["kernels"]}
    if args.ragged_workload:
        r = run_workload(args.ragged_workload, max(args.steps, 20), args.warmup, latency_calls=0)
        rw = r["workload"]
        line["ragged"] = {"workload": rw.name, "batch": rw.batch, "prefix_len": rw.prefix_len,
                          "valid_len": [int(v) for v in r["inputs"]["valid_len"]], "num_steps": rw.num_steps,
                          "chunks_per_s": r["value"], "ms_per_call": r["ms"], "roofline": r["roofline"],
                          "whole_loop": r["whole_loop"], "kernels": r["kernels"]}
    if args.prefill_workload:
        line["prefill"] = run_prefill(args.prefill_workload, max(args.steps // 2, 5), args.warmup)
    if args.copy_bandwidth:
        cb = copy_bandwidth()
        line["hbm_copy"] = cb
        line["whole_loop"]["hbm_frac_of_copy"] = line["whole_loop"]["achieved_GBps"] / cb["GBps"]
        for sub in ("b1", "ragged"):
            if sub in line:
                line[sub]["whole_loop"]["hbm_frac_of_copy"] = line[sub]["whole_loop"]["achieved_GBps"] / cb["GBps"]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, main_res["inputs"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
