#!/usr/bin/env python3
"""Benchmark of the masked sparse attention forward on one MI355X.

One step = one call of the whole hot path (spec parse and plan lookup on the
host, the fused kernel on the GPU) over one batch of synthetic input already
resident in HBM.  Default workload: the 32768-token sliding-window layer
(B=1, H=32, T=32768, d=128, bf16, causal window 4096).

Prints ONE JSON line.  Fields beyond the common contract:
  roofline     -- the kernel against its bound (bf16 MFMA peak here), from
                  HIP events around the timed launches on the launch stream;
                  `traffic` comes from a committed rocprofv3 counter summary
                  and is null if the kernel source changed since it was taken;
  cpu_baseline -- the fp64 oracle timed on this host's cores over a bounded
                  sample of rows of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "allowed attention cells/s and effective TFLOP/s at 1 MI355X; % of bf16 MFMA peak"
BF16_PEAK_TFLOPS = 2500.0
F32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
VENDOR_SCLK_MHZ = 2400.0  # the clock the vendor's peak figures are quoted at
CSRC = os.path.join(ROOT, "block_sparse_masked_spec_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

WORKLOADS = {
    "mistral32k_window4096": dict(B=1, H=32, T=32768, d=128, dtype="bf16",
                                  specs=["causal;window=4096"]),
    "code_layer512_w128_s64": dict(B=8, H=8, T=512, d=64, dtype="bf16",
                                   specs=["causal;window=128;stride=64;phase=0"]),
    "code_layer512_w128_s0": dict(B=8, H=8, T=512, d=64, dtype="bf16", specs=["causal;window=128"]),
    "code_layer512_w256_s64": dict(B=8, H=8, T=512, d=64, dtype="bf16",
                                   specs=["causal;window=256;stride=64;phase=0"]),
    "code_layer512_w256_s0": dict(B=8, H=8, T=512, d=64, dtype="bf16", specs=["causal;window=256"]),
    "code_layer512_full_causal": dict(B=8, H=8, T=512, d=64, dtype="bf16", specs=["causal"]),
    "longformer16k_r256_s16_g128": dict(B=1, H=16, T=16384, d=64, dtype="bf16",
                                        specs=["bidir;radius=256;stride=16;phase=0;global=0:128"]),
    "gemma_interleave_8k": dict(B=2, H=16, T=8192, d=128, dtype="bf16",
                                specs=["causal;window=1024"] * 5 + ["causal"]),
    "gemma_local_8k_w1024": dict(B=2, H=16, T=8192, d=128, dtype="bf16", specs=["causal;window=1024"]),
    "gemma_full_8k_causal": dict(B=2, H=16, T=8192, d=128, dtype="bf16", specs=["causal"]),
    "dilated16k_w512_g2": dict(B=1, H=16, T=16384, d=128, dtype="bf16",
                               specs=["causal;window=512;dilation=2"]),
    "bigbird4k_b8_h12_d64": dict(B=8, H=12, T=4096, d=64, dtype="bf16",
                                 specs=["blocks;block=64;radius=1;random=3;seed=0;global=0:128"]),
    "mistral32k_window4096_bwd": dict(kind="backward", B=1, H=32, T=32768, d=128, dtype="bf16",
                                      specs=["causal;window=4096"]),
    "longformer16k_r256_s16_g128_bwd": dict(kind="backward", B=1, H=16, T=16384, d=64, dtype="bf16",
                                            specs=["bidir;radius=256;stride=16;phase=0;global=0:128"]),
    "bigbird4k_b8_h12_d64_bwd": dict(kind="backward", B=8, H=12, T=4096, d=64, dtype="bf16",
                                     specs=["blocks;block=64;radius=1;random=3;seed=0;global=0:128"]),
    "mistral_decode_b64_w4096": dict(kind="decode", B=64, H=32, Hkv=8, d=128, dtype="bf16",
                                     n_new=1, C=4096, pos_range=(4096, 32768),
                                     specs=["causal;window=4096"]),
    "tiny_fp32_t16": dict(B=1, H=1, T=16, d=16, dtype="f32",
                          specs=["causal;window=2;stride=4;phase=3"]),
}
DEFAULT_WORKLOAD = "mistral32k_window4096"
ROTATE_BYTES = 512 << 20  # input copies touched per pass: above twice the 256 MB MALL
# At most this many copies: a workload under ROTATE_BYTES / MAX_COPIES (the
# 16-token case, 4 KiB) is bound by launch latency, not by where its bytes
# sit, and its 131,072 copies would only add half a million clone kernels
# to every profile of the run.
MAX_COPIES = 64


def kernel_source(wl) -> str:
    """The device source file of the kernels a workload times."""
    kind = wl.get("kind", "forward")
    if kind == "decode":
        return "decode.hip"
    if kind == "backward":
        return "bwd_kernel.hip"
    return "fwd_bf16.hip" if kernel_name(wl["dtype"], wl["d"]) == "sa_fwd_bf16_kernel" else "fwd_kernel.hip"


def kernel_sha(wl) -> str:
    """Hash of a workload's kernel source and the local headers it includes,
    transitively: counter readings taken for other code do not carry over."""
    h = hashlib.sha256()
    seen, todo = set(), [os.path.join(CSRC, kernel_source(wl))]
    while todo:
        f = os.path.normpath(todo.pop(0))
        if f in seen:
            continue
        seen.add(f)
        text = open(f, "rb").read()
        h.update(os.path.basename(f).encode() + b"\0" + text)
        for inc in re.findall(rb'^#include "([^"]+)"', text, re.M):
            todo.append(os.path.join(os.path.dirname(f), inc.decode()))
    return h.hexdigest()[:16]


def kernel_name(dtype: str, d: int) -> str:
    """The kernel that runs the forward for this dtype and head size."""
    return "sa_fwd_bf16_kernel" if dtype == "bf16" and d in (64, 128) else "sa_fwd_kernel"


def bwd_kernel_names(dtype: str, d: int) -> str:
    if dtype == "bf16" and d in (64, 128):
        return "sa_bwd_dq_dma_kernel + sa_bwd_dkv_dma_kernel"
    return "sa_bwd_dq_kernel + sa_bwd_dkv_kernel"


def median_step_ms(step, n, stream):
    """Median time of n steps, each timed alone with its own events on the
    stream (run after the timed region; the contract's figure is the mean)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    return float(statistics.median(e0.elapsed_time(e1) for e0, e1 in evs))


def load_counter(workload: str, field: str = "hbm_bytes_per_launch"):
    """A figure from the committed counter summary (HBM bytes per launch, or
    the MFMA-busy fraction), or None once the kernel source has changed."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    entry = data.get(workload)
    if not entry or entry.get("kernel_sha") != kernel_sha(WORKLOADS[workload]):
        return None
    return entry.get(field)


def load_traffic(workload: str):
    return load_counter(workload)


def _amdsmi_handle(amdsmi):
    """The amdsmi handle of torch's device 0 (matched by PCI address when
    several GPUs are listed)."""
    import torch
    handles = amdsmi.amdsmi_get_processor_handles()
    if len(handles) == 1:
        return handles[0]
    p = torch.cuda.get_device_properties(0)
    bdf = "%04x:%02x:%02x.0" % (getattr(p, "pci_domain_id", 0), p.pci_bus_id, p.pci_device_id)
    for h in handles:
        if amdsmi.amdsmi_get_gpu_device_bdf(h).lower() == bdf:
            return h
    raise RuntimeError(f"no amdsmi device at {bdf}")


def sclk_under_load(step, seconds: float):
    """The GFX clock while the step runs: after the timed region, the step is
    run back to back for `seconds` while a thread reads amdsmi's current GFX
    clock every 2 ms.  The reading trails the load by a few hundred ms (it
    still shows the idle clock at first), so only samples from the last 60%
    of the window count.  Returns the median and range in MHz, or the error."""
    import threading

    import torch
    if seconds <= 0:
        return None
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = _amdsmi_handle(amdsmi)
        read = lambda: float(amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX)["clk"])
        read()
    except Exception as e:  # no permission, no library: report why
        return {"mhz": None, "error": f"{type(e).__name__}: {e}"[:200]}
    samples, stop = [], threading.Event()

    settle = 0.4 * seconds

    def sampler():
        t_start = time.perf_counter()
        while not stop.is_set():
            try:
                v = read()
                if time.perf_counter() - t_start >= settle:
                    samples.append(v)
            except Exception:
                pass
            time.sleep(0.002)

    th = threading.Thread(target=sampler, daemon=True)
    torch.cuda.synchronize()
    th.start()
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        step(i)
        i += 1
        if i % 4 == 0:
            torch.cuda.synchronize()  # keep the queue short: samples see the kernels run
    torch.cuda.synchronize()
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    if not samples:
        return {"mhz": None, "error": "no samples"}
    return {"mhz": float(statistics.median(samples)), "min": min(samples), "max": max(samples),
            "samples": len(samples), "steps": i,
            "source": f"amdsmi current GFX clock, sampled every 2 ms over the last {seconds - settle:.1f} s "
                      f"of {seconds:.1f} s of back-to-back steps after the timed region"}


def at_clock(roofline: dict, sclk: dict):
    """Add the fraction of the peak at the recorded clock (the vendor peak is
    quoted at 2400 MHz) for an MFMA-bound line."""
    mhz = sclk.get("mhz") if sclk else None
    if roofline.get("bound") == "mfma" and mhz:
        peak = roofline["peak"] * mhz / VENDOR_SCLK_MHZ
        roofline["peak_at_sclk"] = peak
        roofline["frac_at_sclk"] = roofline["achieved"] / peak


def cpu_baseline(wl, specs, q, k, v, budget_s: float):
    """Time the oracle on a bounded, evenly spread sample of rows."""
    import random

    import oracle
    B, H, T = wl["B"], wl["H"], wl["T"]
    rng = random.Random(0)
    all_rows = [(rng.randrange(B), rng.randrange(H), rng.randrange(T)) for _ in range(1 << 20)]
    spec = specs[0]
    # calibrate on growing row counts until one run takes >= 1 s, then size
    # the sample to the budget
    n_cal = 256
    while True:
        t0 = time.perf_counter()
        oracle.forward_rows(spec, q, k, v, rows=all_rows[:n_cal])
        dt0 = time.perf_counter() - t0
        if dt0 >= 1.0 or n_cal >= len(all_rows):
            break
        n_cal = min(len(all_rows), n_cal * 4)
    n_rows = int(min(len(all_rows), max(256, n_cal * budget_s / max(dt0, 1e-6))))
    rows = all_rows[:n_rows]
    t0 = time.perf_counter()
    _, _, nset = oracle.forward_rows(spec, q, k, v, rows=rows)
    dt = time.perf_counter() - t0
    cells = int(nset.sum())
    return {
        "value": cells / dt,
        "unit": "allowed cells/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": f"{n_rows} random (b,h,i) rows of {spec} (T={T}), {cells} allowed cells, "
                  f"{dt:.1f} s fp64 on the host",
        "seconds": dt,
    }


def copy_calibration(args, result):
    """With --copy-calibration-mib N, end the run with one device-to-device
    copy of N MiB, so that a counter run can scale FETCH_SIZE / WRITE_SIZE
    by what they read for a copy of known size."""
    import torch

    if args.copy_calibration_mib <= 0:
        return
    n = args.copy_calibration_mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    result["copy_calibration_bytes"] = {"read": n * 4, "write": n * 4}
    del src, dst


def backward_bench(args, wl):
    """Backward pass: one step = one sparse_attn_bwd call (dQ, dK, dV) for a
    forward computed once beforehand.  Algorithmic flops 8 d E: dV, dP, dQ and
    dK each take 2 d per allowed cell (recomputing S is not counted)."""
    import torch

    from block_sparse_masked_spec_amd import binding as sa
    from block_sparse_masked_spec_amd import inputs

    B, H, T, d, spec = wl["B"], wl["H"], wl["T"], wl["d"], wl["specs"][0]
    q, k, v = inputs.qkv(B, H, T, d, "bf16", args.seed)
    g = inputs.qkv(B, H, T, d, "bf16", args.seed + 1)[0]
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), g.cuda()
    od = torch.empty_like(qd)
    lse = torch.empty(B, H, T, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(qd), torch.empty_like(qd)
    stream = torch.cuda.current_stream()
    sa.sparse_attn_fwd_lse(qd, kd, vd, od, lse, B, H, T, d, spec, stream)
    E_total = sa.sparse_attn_count(spec, T) * B * H
    flops = 8.0 * d * E_total
    # Q, K, V, O, dO read once, dQ, dK, dV written once (bf16), LSE read.
    alg_bytes = 8.0 * B * H * T * d * 2 + 4.0 * B * H * T

    def step():
        sa.sparse_attn_bwd(qd, kd, vd, od, gd, lse, dq, dk, dv, B, H, T, d, spec, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    ms_median = median_step_ms(step, args.steps, stream)
    secs = ms / 1e3
    tf = flops / secs / 1e12
    result = {
        "metric": METRIC,
        "value": E_total / secs,
        "unit": "allowed cells/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": ms_median,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1) Q/K/V/dO, no dataset)",
        "config": {"workload": args.workload, "B": B, "H": H, "T": T, "d": d, "mask_specs": [spec],
                   "allowed_cells_per_step": E_total, "pass": "backward (dQ, dK, dV)",
                   "parallelism": "single GPU"},
        "effective_tflops": tf,
        "wall_s_timed": wall,
        "kernel_sha": kernel_sha(wl),
        "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / BF16_PEAK_TFLOPS, "traffic": load_traffic(args.workload),
                     "kernel": bwd_kernel_names(wl["dtype"], d), "ms_per_launch": ms,
                     "mfma_busy": load_counter(args.workload, "mfma_busy"),
                     "algorithmic_flops_per_step": flops, "algorithmic_bytes_per_step": alg_bytes},
        "cpu_baseline": None,
    }
    result["sclk"] = sclk_under_load(lambda i: step(), args.sclk_seconds)
    at_clock(result["roofline"], result["sclk"])
    copy_calibration(args, result)
    if args.cpu_budget > 0:
        result["cpu_baseline"] = cpu_baseline_backward(spec, q, k, v, g, args.cpu_budget)
        result["cpu_baseline"]["gpu_over_cpu"] = result["value"] / result["cpu_baseline"]["value"]
    print(json.dumps(result), flush=True)
    return 0


def cpu_baseline_backward(spec, q, k, v, g, budget_s: float):
    """The oracle's backward (dQ, dK, dV in fp64) timed on a bounded sample:
    the first L positions of up to `threads` heads (the same rule on the
    shorter sequence; the oracle runs one head per thread), with L grown
    until one run takes about a second and then scaled to the budget."""
    import oracle
    B, H, T, d = q.shape
    nh = min(B * H, max(1, oracle.threads()))
    flat = lambda x: x.reshape(B * H, T, d)[:nh].unsqueeze(0)
    qs, ks, vs, gs = flat(q), flat(k), flat(v), flat(g)
    L = min(T, 256)
    while True:
        t0 = time.perf_counter()
        oracle.backward(spec, qs[:, :, :L], ks[:, :, :L], vs[:, :, :L], gs[:, :, :L])
        dt = time.perf_counter() - t0
        if dt >= 1.0 or L >= T:
            break
        L = min(T, L * 2)
    if L < T and dt < budget_s:
        # cells grow about linearly in L once L exceeds the band
        L = min(T, int(L * budget_s / max(dt, 1e-6)))
        t0 = time.perf_counter()
        oracle.backward(spec, qs[:, :, :L], ks[:, :, :L], vs[:, :, :L], gs[:, :, :L])
        dt = time.perf_counter() - t0
    cells = oracle.count(spec, L) * nh
    return {"value": cells / dt, "unit": "allowed cells/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"backward of the first {L} positions of {nh} heads of {spec} "
                      f"({cells} allowed cells), {dt:.1f} s fp64 on the host",
            "seconds": dt}


def cpu_baseline_decode(spec, q, kc, vc, pos, Hkv, budget_s: float):
    """The oracle timed on decode rows: for each sequence, the new token's row
    of the forward over the C live cache positions in position order (K and
    V repeated for the query heads that share a KV head), up to the budget
    or all B sequences."""
    import oracle
    import torch
    B, H, n_new, d = q.shape
    C = kc.shape[2]
    G = H // Hkv
    t0 = time.perf_counter()
    cells, done = 0, 0
    for b in range(B):
        order = torch.tensor([(pos[b] - C + 1 + x) % C for x in range(C)])
        kb = kc[b][:, order].repeat_interleave(G, dim=0).unsqueeze(0)
        vb = vc[b][:, order].repeat_interleave(G, dim=0).unsqueeze(0)
        qb = torch.zeros(1, H, C, d, dtype=q.dtype)
        qb[0, :, C - n_new:] = q[b]
        rows = [(0, h, C - n_new + t) for h in range(H) for t in range(n_new)]
        _, _, nset = oracle.forward_rows(spec, qb, kb, vb, rows=rows)
        cells += int(nset.sum())
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": cells / dt, "unit": "allowed cells/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{done} of {B} sequences, all {H} heads x {n_new} new tokens over {C} cached "
                      f"positions ({cells} allowed cells), {dt:.1f} s fp64 on the host including "
                      "the per-sequence gather of the ring rows",
            "seconds": dt}


def decode_bench(args, wl):
    """Windowed decode: one step = one call decoding n_new tokens of each of B
    sequences against ring-buffer caches of C rows (HBM-bound)."""
    import numpy as np
    import torch

    from block_sparse_masked_spec_amd import binding as sa
    from block_sparse_masked_spec_amd import inputs

    B, H, Hkv, d, n_new, C = wl["B"], wl["H"], wl["Hkv"], wl["d"], wl["n_new"], wl["C"]
    spec = wl["specs"][0]
    rng = np.random.default_rng(args.seed)
    pos = [int(x) for x in rng.integers(*wl["pos_range"], size=B)]
    _, kc, vc = inputs.qkv(B, Hkv, C, d, "bf16", args.seed)
    q = inputs.qkv(B, H, n_new, d, "bf16", args.seed + 1)[0]
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    od = torch.empty_like(qd)
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    rows = sa.sparse_attn_decode_cache_rows(spec, n_new)
    # allowed keys per new token: the window (all cache rows hold live positions here)
    allowed = sum(min(rows - n_new + 1 if rows else p + 1, p + 1) for p in pos) * H * n_new
    stream = torch.cuda.current_stream()

    def step():
        sa.sparse_attn_decode(qd, kd, vd, od, posd, B, H, Hkv, n_new, C, d, spec, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    ms_median = median_step_ms(step, args.steps, stream)
    secs = ms / 1e3
    # Algorithmic bytes: every allowed K and V row once, Q read, O written.
    kv_rows = min(C, rows) if rows else C
    alg_bytes = (2.0 * B * Hkv * kv_rows * d + 2.0 * B * H * n_new * d) * 2
    flops = 4.0 * d * allowed
    traffic = load_traffic(args.workload)
    result = {
        "metric": METRIC,
        "value": allowed / secs,
        "unit": "allowed cells/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": ms_median,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1) Q/K/V, no dataset)",
        "config": {"workload": args.workload, "B": B, "H": H, "Hkv": Hkv, "d": d, "n_new": n_new,
                   "cache_rows": C, "mask_specs": [spec], "allowed_cells_per_step": allowed,
                   "parallelism": "single GPU"},
        "effective_tflops": flops / secs / 1e12,
        "wall_s_timed": wall,
        "kernel_sha": kernel_sha(wl),
        "roofline": {"bound": "hbm", "achieved": alg_bytes / secs / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": alg_bytes / secs / 1e9 / HBM_PEAK_GBS,
                     "traffic": traffic, "kernel": "sa_decode_kernel", "ms_per_launch": ms,
                     "algorithmic_bytes_per_step": alg_bytes},
        "cpu_baseline": None,
    }
    result["sclk"] = sclk_under_load(lambda i: step(), args.sclk_seconds)
    copy_calibration(args, result)
    if args.cpu_budget > 0:
        result["cpu_baseline"] = cpu_baseline_decode(spec, q, kc, vc, pos, Hkv, args.cpu_budget)
        result["cpu_baseline"]["gpu_over_cpu"] = result["value"] / result["cpu_baseline"]["value"]
    print(json.dumps(result), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--sclk-seconds", type=float, default=1.5,
                    help="after timing, run the step back to back this long while sampling the "
                         "GFX clock (0 = skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a "
                         "known-size kernel for scaling HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported and nothing "
              "was run (the forward shards over heads and query blocks with no communication, "
              "so N GPUs each run this same kernel on H/N heads).", file=sys.stderr)
        return 2

    import torch

    from block_sparse_masked_spec_amd import binding as sa
    from block_sparse_masked_spec_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    sa.load()
    wl = WORKLOADS[args.workload]
    if wl.get("kind") == "decode":
        return decode_bench(args, wl)
    if wl.get("kind") == "backward":
        return backward_bench(args, wl)
    B, H, T, d, dtype, specs = wl["B"], wl["H"], wl["T"], wl["d"], wl["dtype"], wl["specs"]
    fwd = sa.sparse_attn_fwd if dtype == "bf16" else sa.sparse_attn_fwd_f32

    # Inputs: one fresh seeded set per call of the step (the interleave
    # workload runs several independent calls), resident on the GPU.  Small
    # workloads rotate over enough copies that one pass touches more than
    # twice the 256 MB last-level cache, so each step reads HBM, not cache
    # (up to MAX_COPIES).
    host_sets, dev_sets = [], []
    for c, spec in enumerate(specs):
        q, k, v = inputs.qkv(B, H, T, d, dtype, args.seed + c)
        host_sets.append((q, k, v))
        dev_sets.append((q.cuda(), k.cuda(), v.cuda(), torch.empty_like(q, device="cuda")))
    set_bytes = 4 * q.numel() * q.element_size() * len(specs)
    n_copies = min(MAX_COPIES, max(1, -(-ROTATE_BYTES // set_bytes)))
    copies = [dev_sets] + [[tuple(t.clone() for t in ds) for ds in dev_sets] for _ in range(n_copies - 1)]
    allowed = [sa.sparse_attn_count(s, T) for s in specs]
    E_total = sum(allowed) * B * H  # allowed (b,h,i,j) pairs per step
    flops = 4.0 * d * E_total
    alg_bytes = 4.0 * B * H * T * d * (2 if dtype == "bf16" else 4) * len(specs)
    info = [sa.sparse_attn_plan_info_bh(s, B, H, T, d, sa.SA_DTYPE_BF16 if dtype == "bf16" else sa.SA_DTYPE_F32)
            for s in specs]
    executed = sum(i["executed_cells"] for i in info) * B * H
    # Plans that split heavy query blocks add a merge kernel to each call.
    kernels = kernel_name(dtype, d) + (" + sa_fwd_merge_kernel" if any(i["split_parts"] for i in info) else "")

    stream = torch.cuda.current_stream()

    def step(i):
        for (qd, kd, vd, od), spec in zip(copies[i % n_copies], specs):
            fwd(qd, kd, vd, od, B, H, T, d, spec, stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = gpu_ms / args.steps
    launches = args.steps * len(specs)
    ms_per_launch = gpu_ms / launches
    # After the timed region: the same number of steps timed one by one, for
    # the median step time (each bracketed by its own events on the stream).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i, (e0, e1) in enumerate(evs):
        e0.record(stream)
        step(args.warmup + args.steps + i)
        e1.record(stream)
    torch.cuda.synchronize()
    ms_median = float(statistics.median(e0.elapsed_time(e1) for e0, e1 in evs))
    secs = ms_per_step / 1e3
    eff_tflops = flops / secs / 1e12
    peak = BF16_PEAK_TFLOPS if dtype == "bf16" else F32_PEAK_TFLOPS

    if len(specs) == 1 and flops / alg_bytes < (peak * 1e12) / (HBM_PEAK_GBS * 1e9) / 4:
        bound, unit, achieved, pk = "hbm", "GB/s", alg_bytes / secs / 1e9, HBM_PEAK_GBS
    else:
        bound, unit, achieved, pk = "mfma", "TFLOP/s", eff_tflops, peak
    traffic = load_traffic(args.workload)
    roofline = {
        "bound": bound, "achieved": achieved, "peak": pk, "unit": unit,
        "frac": achieved / pk, "traffic": traffic,
        "kernel": kernels, "ms_per_launch": ms_per_launch,
        "mfma_busy": load_counter(args.workload, "mfma_busy"),
        "algorithmic_flops_per_step": flops, "algorithmic_bytes_per_step": alg_bytes,
        "executed_over_allowed": executed / (E_total if E_total else 1),
    }

    result = {
        "metric": METRIC,
        "value": E_total / secs,
        "unit": "allowed cells/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_median": ms_median,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded iid N(0,1) Q/K/V, no dataset)",
        "config": {
            "workload": args.workload, "B": B, "H": H, "T": T, "d": d,
            "mask_specs": specs, "allowed_cells_per_step": E_total,
            "input_copies": n_copies, "parallelism": "single GPU",
        },
        "us_per_step": ms_per_step * 1e3,
        "effective_tflops": eff_tflops,
        "frac_bf16_peak": eff_tflops / BF16_PEAK_TFLOPS,
        "wall_s_timed": wall,
        "kernel_sha": kernel_sha(wl),
        "roofline": roofline,
        "cpu_baseline": None,
    }
    result["sclk"] = sclk_under_load(lambda i: step(i), args.sclk_seconds)
    at_clock(roofline, result["sclk"])
    copy_calibration(args, result)
    if args.cpu_budget > 0:
        q, k, v = host_sets[0]
        result["cpu_baseline"] = cpu_baseline(wl, specs, q, k, v, args.cpu_budget)
        result["cpu_baseline"]["gpu_over_cpu"] = result["value"] / result["cpu_baseline"]["value"]
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
