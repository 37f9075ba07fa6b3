"""Parallax decode benchmark on one MI355X.

A step is one pass of the whole hot path over one batch: the probe
rho = W_R x, the decode split-K pass and the merge of the splits, for every
sequence.
The default workload is the mid-context GQA decode (B=16, Hq=16, Hkv=8, d=128,
ctx=4096, d_model=2048, bf16 cache). Inputs are resident in HBM before timing;
several independently seeded input sets are rotated so that every step reads
its K/V cold (their total exceeds the last-level cache).

Output: one JSON line (metric, value = decode tokens/s, ms_per_step, roofline
of the dominant kernel, CPU oracle baseline, ...), with a compact record per
other workload under "configs" (step and per-kernel times, algorithmic bytes,
fraction of peak, launch plan) and a compact batch x context record under
"sweep" (--sweep runs the whole grid, one line per point).

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload 2]
                    [--sets 3] [--no-cpu-baseline] [--no-configs] [--no-sweep-record]
                    [--sweep] [--fusion-sweep]
                    [--copy-calibration]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Parallax decode tokens/s and HBM GB/s (% of peak) over batch×context sweep"
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak, GB/s
PROFILES = os.path.join(ROOT, "profiles")
# Each decode kernel's sources: its own file and the shared device header.
CSRC = os.path.join(ROOT, "parallax_covariance_corrected_amd", "csrc")
DECODE_SRCS = {"decode_mfma": ("decode_mfma.hip", "common.h"),
               "decode_generic": ("decode_generic.hip", "common.h")}


def kernel_source_hash(kernel: str = "decode_mfma") -> str:
    h = hashlib.sha256()
    for f in DECODE_SRCS[kernel]:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload_name: str, kernel: str = "decode_mfma"):
    """HBM bytes per decode launch from the committed rocprofv3 PMC summary, or
    None when there is none or the kernel source changed since it was taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload_name}_traffic.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\s*(\{.*?\})\s*```", open(path).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(kernel):
        return None
    return rec.get("traffic_bytes_per_launch")


def upload_set(s, device="cuda"):
    import torch
    from parallax_covariance_corrected_amd.workloads import padded_cache
    return dict(x=s.x.to(device), W_R=s.W_R.to(device), q=s.q.to(device),
                seq_lens=s.seq_lens.to(device),
                K=padded_cache(s.K, s.max_ctx, 0.0, device=device),
                V=padded_cache(s.V, s.max_ctx, 0.0, device=device),
                rho=torch.empty((s.wl.B, s.wl.Hq, s.wl.d), dtype=torch.float32, device=device),
                out=torch.empty((s.wl.B, s.wl.Hq, s.wl.d), dtype=s.q.dtype, device=device))


def step(pb, wl, d):
    """One decode step: probe and decode in one library call (the plan places
    the probe inside the decode kernel or in a launch of its own)."""
    pb.probe_decode(d["W_R"], d["x"], d["q"], d["K"], d["V"], d["seq_lens"], out=d["out"])


def fill_rho(pb, wl, d):
    """rho of a set in its own buffer, for the decode-only measurements."""
    pb.probe(d["W_R"], d["x"], wl.Hq, wl.d, out=d["rho"])


_SLEEP_CYCLES_PER_US = None


def _sleep_cycles_per_us() -> float:
    """Rate of torch's spin kernel (cycles of its clock per microsecond)."""
    global _SLEEP_CYCLES_PER_US
    import torch
    if _SLEEP_CYCLES_PER_US is None:
        n = 2_000_000
        torch.cuda._sleep(n)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(n)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_US = n / max(e0.elapsed_time(e1) * 1e3, 1.0)
    return _SLEEP_CYCLES_PER_US


def per_launch_us(pb, fn, reps: int, kinds):
    """Average duration in microseconds of each kernel kind in `kinds` over reps
    calls of fn(i), from per-launch HIP events stamped on the launch stream.

    A per-launch event brackets its kernel only while the stream has work
    queued ahead of it; when the host enqueues more slowly than the GPU runs,
    the start stamp can precede the kernel by the host's own launch latency.
    So the stream is first held by a spin kernel of bounded length (long enough
    for the host to enqueue all reps calls behind it), and the launches then
    run back to back as in the timed steps. Returns ({kind: us}, queued), where
    queued says whether the host had enqueued every call before the spin ended."""
    import torch
    rate = _sleep_cycles_per_us()
    gate = torch.cuda.Event()
    with pb.options(profile=1):
        # one untimed pass creates the library's pooled events, then the host
        # cost of one call with its launches stamped
        for i in range(reps):
            fn(i)
        torch.cuda.synchronize()
        pb.profile_reset()
        t0 = time.perf_counter()
        for i in range(min(reps, 20)):
            fn(i)
        host_us = (time.perf_counter() - t0) * 1e6 / min(reps, 20)
        torch.cuda.synchronize()
        hold_us = min(1.5 * host_us * reps + 2000.0, 500_000.0)
        pb.profile_reset()
        torch.cuda._sleep(int(hold_us * rate))
        gate.record()
        for i in range(reps):
            fn(i)
        queued = not gate.query()
        torch.cuda.synchronize()
        out = {}
        for name, k in kinds:
            ms, n = pb.profile_read(k)
            out[name] = ms / n * 1e3 if n else 0.0
    return out, queued


def timed_steps(fn, reps: int, warm: int = 5) -> float:
    """Average microseconds of fn(i) over reps calls, events on the current stream."""
    import torch
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def probe_fusion(pb, wl, dev_sets, reps: int):
    """Whole-step time with the probe in a launch of its own and inside the
    decode kernel (where the plan can place it there), same inputs."""
    code = pb.BF16 if wl.dtype == "bf16" else pb.F32
    auto = pb.probe_decode_plan(wl.B, wl.Hq, wl.Hkv, wl.d, wl.d_model, wl.capacity, code)
    rec = {"auto_plan": "fused" if auto else "separate"}
    for name, f in (("separate", 1), ("fused", 2)):
        with pb.options(fuse=f):
            if f == 2 and not pb.probe_decode_plan(wl.B, wl.Hq, wl.Hkv, wl.d, wl.d_model,
                                                   wl.capacity, code):
                rec[f"{name}_step_us"] = None
                continue
            rec[f"{name}_step_us"] = round(
                timed_steps(lambda i: step(pb, wl, dev_sets[i % len(dev_sets)]), reps), 3)
    return rec


def cpu_baseline(s, budget_s: float = 12.0):
    """The fp64 oracle on the host over a bounded sample of (sequence, head)
    pairs of the same workload; tokens/s scaled to whole sequences."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    wl = s.wl
    t0 = time.perf_counter()
    rho = oracle.probe(s.W_R, s.x, wl.Hq, wl.d)
    t_probe = time.perf_counter() - t0
    q = s.q.float().numpy().astype(np.float64)
    lens = s.seq_lens.tolist()
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.Hq)]
    done = 0
    t0 = time.perf_counter()
    for (b, h) in pairs:
        oracle.decode_heads(q, rho, s.K, s.V, lens, wl.Hkv, [(b, h)])
        done += 1
        if time.perf_counter() - t0 > budget_s and done >= 4:
            break
    t_dec = time.perf_counter() - t0
    # seconds for one full step = probe + all B*Hq heads at the measured per-head rate
    step_s = t_probe + t_dec * (wl.B * wl.Hq) / done
    return {"value": wl.B / step_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle probe for all {wl.B} sequences + decode of {done} of "
                      f"{wl.B * wl.Hq} (sequence, head) pairs in {t_dec:.1f} s, "
                      f"scaled to the full step"}


def matched_ratios(pb, wl, dev_sets, reps: int):
    """Decode-only time of Parallax against plain softmax attention run by the
    same kernel without the correction branch: at the same KV bytes
    (I/O-matched: same heads) and at the same arithmetic (compute-matched:
    twice the query heads over the same cache). Speed-up = softmax time /
    Parallax time, so values above 1 mean Parallax is faster."""
    import torch
    q2 = [d["q"].repeat_interleave(2, dim=1).contiguous() for d in dev_sets]
    out2 = torch.empty_like(q2[0])

    def timed(fn):
        return timed_steps(fn, reps)

    def par(i):
        d = dev_sets[i % len(dev_sets)]
        pb.decode(d["q"], d["rho"], d["K"], d["V"], d["seq_lens"], out=d["out"])

    def soft(i):
        d = dev_sets[i % len(dev_sets)]
        pb.softmax_decode(d["q"], d["K"], d["V"], d["seq_lens"], out=d["out"])

    def soft2(i):
        d = dev_sets[i % len(dev_sets)]
        pb.softmax_decode(q2[i % len(dev_sets)], d["K"], d["V"], d["seq_lens"], out=out2)

    t_par, t_soft, t_soft2 = timed(par), timed(soft), timed(soft2)
    return {"parallax_decode_us": round(t_par, 3), "softmax_decode_us": round(t_soft, 3),
            "softmax_2x_heads_decode_us": round(t_soft2, 3),
            "io_matched_speedup": round(t_soft / t_par, 4),
            "compute_matched_speedup": round(t_soft2 / t_par, 4)}


def read_ceiling(pb, reps: int = 30):
    """Rate of the library's read reference (the decode's K load shape) over
    three rotated 256 MiB buffers: a read-only ceiling measured on this GPU."""
    import torch
    n = 256 << 20
    bufs = [torch.full((n,), i + 1, dtype=torch.uint8, device="cuda") for i in range(3)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    us = per_launch_us(pb, lambda i: pb.read_bandwidth(bufs[i % 3], sink), reps,
                       (("read", pb.KERNEL_READ),))[0]["read"]
    del bufs
    torch.cuda.empty_cache()
    return n / (us * 1e-6) / 1e9


def step_percentiles(pb, wl, dev_sets, reps: int):
    """p10 / p50 / p90 of single-step times (each step bracketed by its own
    events), cold (rotated input sets) and warm (one set repeated)."""
    import torch

    def times(pick):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for i, (a, b) in enumerate(ev):
            a.record()
            step(pb, wl, pick(i))
            b.record()
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        return [round(t[int(q * (reps - 1))], 2) for q in (0.1, 0.5, 0.9)]

    cold = times(lambda i: dev_sets[i % len(dev_sets)])
    for _ in range(5):
        step(pb, wl, dev_sets[0])
    warm = times(lambda i: dev_sets[0])
    return {"cold_p10_p50_p90_us": cold, "warm_p10_p50_p90_us": warm}


def correction_ratio(pb, d):
    """||C rho|| / ||out||: the share of the correction in the output, from the
    Parallax and softmax-only outputs of the same kernels on the same inputs."""
    import torch
    par = pb.decode(d["q"], d["rho"], d["K"], d["V"], d["seq_lens"], out_dtype=torch.float32)
    soft = pb.softmax_decode(d["q"], d["K"], d["V"], d["seq_lens"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    return round(float((par - soft).norm() / par.norm()), 4)


def run_config(args, wl_id: int, reps: int):
    """One of the other workloads, measured like the main line but compactly:
    whole steps (parallax_probe_decode) timed back to back, then the same steps
    with per-launch events for the probe, decode and merge kernels. x, W_R, q
    and the lengths are the seeded host draws; K/V are drawn on the device
    (same distribution), with enough rotated sets that at least 1 GiB of other
    K/V streams between two uses of one set (every step reads cold)."""
    import math
    import torch
    from parallax_covariance_corrected_amd import binding as pb
    from parallax_covariance_corrected_amd.workloads import (WORKLOADS, algorithmic_bytes,
                                                             device_cache, make_inputs)
    wl = WORKLOADS[wl_id]
    print(f"# bench: config {wl.name}", file=sys.stderr, flush=True)
    es = 2 if wl.dtype == "bf16" else 4
    first = make_inputs(wl, 0, with_kv=False)
    kv_set = 2 * first.total_tokens() * wl.Hkv * wl.d * es
    nsets = max(2, min(12, 1 + math.ceil((1 << 30) / max(kv_set, 1))))
    sets, tokens = [], []
    for seed in range(nsets):
        h = first if seed == 0 else make_inputs(wl, seed, with_kv=False)
        K, V = device_cache(wl, 1000 + seed)
        sets.append(dict(W_R=h.W_R.cuda(), x=h.x.cuda(), q=h.q.cuda(), seq_lens=h.seq_lens.cuda(),
                         K=K, V=V, out=torch.empty((wl.B, wl.Hq, wl.d), dtype=h.q.dtype,
                                                   device="cuda")))
        tokens.append(h.total_tokens())
    torch.cuda.synchronize()
    code = pb.BF16 if wl.dtype == "bf16" else pb.F32
    chunk, splits, kernel = pb.decode_plan(wl.B, wl.Hq, wl.Hkv, wl.d, wl.capacity, code)
    fused = pb.probe_decode_plan(wl.B, wl.Hq, wl.Hkv, wl.d, wl.d_model, wl.capacity, code)
    step_us = timed_steps(lambda i: step(pb, wl, sets[i % nsets]), reps, warm=max(args.warmup, 3))
    per, queued = per_launch_us(pb, lambda i: step(pb, wl, sets[i % nsets]), reps,
                                (("probe", pb.KERNEL_PROBE), ("decode", pb.KERNEL_DECODE),
                                 ("merge", pb.KERNEL_MERGE)))
    ab = [algorithmic_bytes(wl, t) for t in tokens]
    dec_bytes = sum(a["decode_read"] for a in ab) / len(ab)
    step_bytes = sum(a["total"] for a in ab) / len(ab) + wl.Hq * wl.d * wl.d_model * es

    def frac(us):
        return round(dec_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4) if us > 0 else None
    rec = {"workload": wl.name, "tokens_per_s": round(wl.B / (step_us * 1e-6), 1),
           "step_us": round(step_us, 3), "decode_kernel_us": round(per["decode"], 3),
           "merge_us": round(per["merge"], 3), "probe_us": round(per["probe"], 3),
           "decode_bytes_per_launch": int(dec_bytes),
           "frac_decode_kernel": frac(per["decode"]),
           "frac_decode_call": frac(per["decode"] + per["merge"]),
           "pct_peak_step": round(100 * step_bytes / (step_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
           "mean_tokens_per_set": round(sum(tokens) / len(tokens), 1),
           "kv_sets_rotated": nsets, "reps": reps, "launches_queued_ahead": queued,
           "plan": {"chunk": chunk, "splits": splits, "kernel": kernel,
                    "probe": "fused" if fused else "separate"}}
    del sets
    torch.cuda.empty_cache()
    return rec


def run_workload(args, wl_id: int, emit: bool = True):
    import torch
    from parallax_covariance_corrected_amd import binding as pb
    from parallax_covariance_corrected_amd.workloads import WORKLOADS, make_inputs, algorithmic_bytes

    wl = WORKLOADS[wl_id]
    if args.hq:
        wl = wl.scaled(Hq=args.hq, name=re.sub(r"Hq\d+", f"Hq{args.hq}", wl.name))
    print(f"# bench: generating {args.sets} input sets for {wl.name}", file=sys.stderr, flush=True)
    sets_host = [make_inputs(wl, seed) for seed in range(args.sets)]
    dev_sets = [upload_set(s) for s in sets_host]
    for d in dev_sets:
        fill_rho(pb, wl, d)
    torch.cuda.synchronize()
    tokens = [s.total_tokens() for s in sets_host]
    code = pb.BF16 if wl.dtype == "bf16" else pb.F32
    chunk, splits, kernel = pb.decode_plan(wl.B, wl.Hq, wl.Hkv, wl.d, wl.capacity, code)
    fused = pb.probe_decode_plan(wl.B, wl.Hq, wl.Hkv, wl.d, wl.d_model, wl.capacity, code)

    for i in range(args.warmup):
        step(pb, wl, dev_sets[i % len(dev_sets)])
    torch.cuda.synchronize()
    print(f"# bench: warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # Timed region: K steps, nothing else on the stream.
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        step(pb, wl, dev_sets[i % len(dev_sets)])
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    print(f"# bench: timed {args.steps} steps in {total_ms:.3f} ms", file=sys.stderr, flush=True)

    # Same K steps again with per-launch HIP events (stamped by each kernel's
    # dispatch on the launch stream) for the dominant kernel's duration.
    per, queued = per_launch_us(pb, lambda i: step(pb, wl, dev_sets[i % len(dev_sets)]),
                                args.steps, (("probe", pb.KERNEL_PROBE),
                                             ("decode", pb.KERNEL_DECODE),
                                             ("merge", pb.KERNEL_MERGE)))

    ms_step = total_ms / args.steps
    # algorithmic bytes, averaged over the rotated sets
    es = 2 if wl.dtype == "bf16" else 4
    ab = [algorithmic_bytes(wl, t) for t in tokens]
    step_bytes = sum(a["total"] for a in ab) / len(ab) + wl.Hq * wl.d * wl.d_model * es
    dec_bytes = sum(a["decode_read"] for a in ab) / len(ab)
    dec_avg_ms = per["decode"] * 1e-3
    mrg_avg_ms = per["merge"] * 1e-3
    achieved = dec_bytes / (dec_avg_ms * 1e-3) / 1e9
    traffic = measured_traffic(wl.name, "decode_mfma" if kernel >= 2 else "decode_generic")
    rec = {
        "metric": METRIC,
        "value": round(wl.B / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "d": wl.d,
                   "ctx": wl.ctx, "max_ctx": wl.capacity, "d_model": wl.d_model,
                   "kv_dtype": wl.dtype, "input_sets_rotated": args.sets,
                   "plan": {"chunk": chunk, "splits": splits, "kernel": kernel,
                            "probe": "fused" if fused else "separate"}},
        "hbm_gbps_step": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "pct_peak_step": round(100 * step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic,
                     "kernel": ("decode_mfma_kernel" if kernel >= 2 else "decode_generic_kernel")
                               + (" (probe fused in)" if fused else " (split-K pass)"),
                     "bytes_per_launch": int(dec_bytes),
                     "avg_launch_us": round(dec_avg_ms * 1e3, 3),
                     "merge_avg_us": round(mrg_avg_ms * 1e3, 3),
                     # the decode call (split-K pass + merge launch) over the same bytes
                     "frac_decode_call": round(dec_bytes / ((dec_avg_ms + mrg_avg_ms) * 1e-3)
                                               / 1e9 / PEAK_HBM_GBS, 4),
                     "probe_avg_us": round(per["probe"], 3),
                     "launches_queued_ahead": queued},
        "cpu_baseline": None,
    }
    rec["step_time_distribution"] = step_percentiles(pb, wl, dev_sets, args.steps)
    rec["probe_fusion"] = probe_fusion(pb, wl, dev_sets, min(args.steps, 100))
    if wl.dtype == "bf16":
        rec["matched"] = matched_ratios(pb, wl, dev_sets, args.steps)
        rec["correction_to_output"] = correction_ratio(pb, dev_sets[0])
        ceiling = read_ceiling(pb)
        rec["roofline"]["read_ceiling_gbps"] = round(ceiling, 1)
        rec["roofline"]["frac_of_read_ceiling"] = round(achieved / ceiling, 4)
    if args.cpu_baseline:
        print("# bench: timing the CPU oracle baseline", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(sets_host[0])
    if args.configs:
        del dev_sets
        torch.cuda.empty_cache()
        rec["configs"] = {str(i): run_config(args, i, max(args.steps, 20))
                          for i in sorted(WORKLOADS) if i != wl_id}
    if args.configs and args.sweep_record:
        rec["sweep"] = compact_sweep(pb)
    if emit:
        print(json.dumps(rec), flush=True)
    return rec


def sweep_point(pb, B: int, ctx: int, warm: int = 20, reps: int = 100) -> dict:
    """One batch x context point at Hq=16, Hkv=8, d=128, d_model=2048, bf16, on
    rotated K/V sets (at least two, three below 768 MB, so that every call
    reads its K/V cold): the decode call (split-K pass + merge) timed over reps
    calls after warm warm-up calls, each call bracketed by its own events
    (median, p10, p90), the same calls back to back (mean per call), the decode
    kernel's own duration (per-launch events), the probe alone, the whole step
    through parallax_probe_decode, and the share of the correction in the
    output, ||C rho|| / ||out||. GB/s counts K/V, q, rho, out and seq_lens;
    `pct_peak` is over the decode call's median, `kernel_pct_peak` over the
    decode kernel's own duration."""
    import torch
    dev, d_model = "cuda", 2048
    kv = 2 * B * ctx * 8 * 128 * 2
    nsets = max(2, min(3, (768 << 20) // kv + 1))
    g = torch.Generator(device=dev).manual_seed(B * 100003 + ctx)
    sets = []
    for _ in range(nsets):
        K = torch.randn((B, 8, ctx, 128), generator=g, device=dev, dtype=torch.bfloat16)
        V = torch.randn((B, 8, ctx, 128), generator=g, device=dev, dtype=torch.bfloat16)
        sets.append((K, V))
    x = torch.randn((B, d_model), generator=g, device=dev).to(torch.bfloat16)
    W_R = (torch.randn((16 * 128, d_model), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    q = torch.randn((B, 16, 128), generator=g, device=dev).to(torch.bfloat16)
    rho = pb.probe(W_R, x, 16, 128)
    lens = torch.full((B,), ctx, dtype=torch.int32, device=dev)
    out = torch.empty((B, 16, 128), dtype=torch.bfloat16, device=dev)

    def call(i):
        K, V = sets[i % nsets]
        pb.decode(q, rho, K, V, lens, out=out)

    for i in range(warm):
        call(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for i, (a, b) in enumerate(ev):
        a.record()
        call(i)
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    p10, med, p90 = (t[int(f * (reps - 1))] for f in (0.1, 0.5, 0.9))
    # the same calls back to back (mean per call), then with per-launch
    # events: the decode kernel alone
    b2b = timed_steps(call, reps, warm=5)
    kus = per_launch_us(pb, call, reps, (("decode", pb.KERNEL_DECODE),))[0]["decode"]
    pus = per_launch_us(pb, lambda i: pb.probe(W_R, x, 16, 128, out=rho), reps,
                        (("probe", pb.KERNEL_PROBE),))[0]["probe"]

    def step(i):
        K, V = sets[i % nsets]
        pb.probe_decode(W_R, x, q, K, V, lens, out=out)

    step_us = timed_steps(step, reps, warm=5)
    par = pb.decode(q, rho, *sets[0], lens, out_dtype=torch.float32)
    soft = pb.softmax_decode(q, *sets[0], lens, out_dtype=torch.float32)
    torch.cuda.synchronize()
    corr = float((par - soft).norm() / par.norm())
    byts = kv + B * 16 * 128 * (2 + 4 + 2) + B * 4
    chunk, splits, kern = pb.decode_plan(B, 16, 8, 128, ctx)
    del sets, q, rho, lens, out, x, W_R, par, soft
    torch.cuda.empty_cache()

    def pct(us):
        return round(100 * byts / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 2)
    return {"B": B, "ctx": ctx, "plan": [chunk, splits, kern],
            "us_per_step": round(med, 2), "p10_us": round(p10, 2),
            "p90_us": round(p90, 2),
            "tokens_per_s": round(B / (med * 1e-6), 1),
            "gbps": round(byts / (med * 1e-6) / 1e9, 1),
            "pct_peak": pct(med),
            "call_us_back_to_back": round(b2b, 2), "call_pct_peak_back_to_back": pct(b2b),
            "kernel_us": round(kus, 2), "kernel_pct_peak": pct(kus),
            "probe_us": round(pus, 2), "probe_decode_step_us": round(step_us, 2),
            "correction_to_output": round(corr, 4)}


def run_sweep(args):
    """Batch x context sweep (B 1..2048, ctx 128..32768, powers of two): one JSON
    line per point (sweep_point)."""
    from parallax_covariance_corrected_amd import binding as pb
    from parallax_covariance_corrected_amd.workloads import sweep_points

    max_bytes = args.sweep_max_gib << 30
    for (B, ctx) in sweep_points(max_bytes // 2 if args.sweep_max_gib else 64 << 30):
        print(json.dumps({"sweep": True, **sweep_point(pb, B, ctx)}), flush=True)


# Points of the compact sweep record in the default line: batch 1 .. 512 by
# factors of 8 against a short, a mid and a long context (K+V up to 16 GiB).
COMPACT_SWEEP = [(B, c) for B in (1, 8, 64, 512) for c in (256, 4096, 32768)
                 if 2 * B * c * 8 * 128 * 2 <= 16 << 30]


def compact_sweep(pb) -> dict:
    """A subset of the batch x context sweep for the default line: per point
    the decode kernel's and the decode call's fraction of peak, the one-call
    step and its tokens/s (50 calls per measurement)."""
    pts = []
    for (B, c) in COMPACT_SWEEP:
        print(f"# bench: sweep point B={B} ctx={c}", file=sys.stderr, flush=True)
        r = sweep_point(pb, B, c, warm=10, reps=50)
        pts.append({"B": B, "ctx": c, "plan": r["plan"], "kernel_us": r["kernel_us"],
                    "kernel_pct_peak": r["kernel_pct_peak"],
                    "call_us_back_to_back": r["call_us_back_to_back"],
                    "call_pct_peak_back_to_back": r["call_pct_peak_back_to_back"],
                    "step_us": r["probe_decode_step_us"],
                    "step_tokens_per_s": round(B / (r["probe_decode_step_us"] * 1e-6), 1)})
    return {"model": "Hq 16, Hkv 8, d 128, d_model 2048, bf16, every sequence full",
            "points": pts}


def run_fusion_sweep(args):
    """Whole-step time of parallax_probe_decode with the probe in its own launch
    and inside the decode kernel, over batch x d_model x context (bf16, Hq=16,
    Hkv=8, d=128; and the fp32 tiny shape family), three rotated input sets
    drawn on the device. One line per point on stdout (markdown table)."""
    import torch
    from parallax_covariance_corrected_amd import binding as pb
    g = torch.Generator(device="cuda").manual_seed(0)
    pts = [("bf16", B, 16, 8, 128, dm, ctx) for B in (1, 4, 16, 64)
           for dm in (64, 128, 256, 512, 1024, 2048) for ctx in (128, 1024, 4096)]
    pts += [("f32", B, 2, 2, 64, dm, ctx) for B in (1, 4) for dm in (128, 512) for ctx in (128, 1024)]
    print("| dtype | B | Hq/Hkv | d | d_model | ctx | plan kernel, splits | W_R bytes per item "
          "| items | separate us | fused us | fused/separate | auto |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    for (dt, B, Hq, Hkv, d, dm, ctx) in pts:
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        code = pb.BF16 if dt == "bf16" else pb.F32

        def rnd(*shape, std=1.0):
            return (torch.randn(*shape, generator=g, device="cuda") * std).to(tdt)
        sets = [dict(W_R=rnd(Hq * d, dm, std=0.02), x=rnd(B, dm), q=rnd(B, Hq, d),
                     K=rnd(B, Hkv, ctx, d), V=rnd(B, Hkv, ctx, d),
                     seq_lens=torch.full((B,), ctx, dtype=torch.int32, device="cuda"),
                     out=torch.empty((B, Hq, d), dtype=tdt, device="cuda")) for _ in range(3)]

        def run(i):
            e = sets[i % 3]
            pb.probe_decode(e["W_R"], e["x"], e["q"], e["K"], e["V"], e["seq_lens"], out=e["out"])
        _, splits, kern = pb.decode_plan(B, Hq, Hkv, d, ctx, code)
        G = Hq // Hkv
        gh = max(g for g in range(1, 9) if G % g == 0)
        item = gh * d * dm * (2 if dt == "bf16" else 4)
        items = B * Hkv * (G // gh) * splits
        with pb.options(fuse=1):
            t_sep = timed_steps(run, args.steps)
        with pb.options(fuse=2):
            can = pb.probe_decode_plan(B, Hq, Hkv, d, dm, ctx, code)
            t_fus = timed_steps(run, args.steps) if can else float("nan")
        auto = pb.probe_decode_plan(B, Hq, Hkv, d, dm, ctx, code)
        print(f"| {dt} | {B} | {Hq}/{Hkv} | {d} | {dm} | {ctx} | {kern}, {splits} | {item} | {items} "
              f"| {t_sep:.2f} | {t_fus:.2f} | {t_fus / t_sep:.3f} | {'fused' if auto else 'separate'} |",
              flush=True)
        del sets


def run_prefill(args):
    """Causal many-query forward (parallax_prefill) on the mid-context heads
    (Hq=16, Hkv=8, d=128, bf16) at B sequences of T new tokens, no prefix.
    Algorithmic work: 8d flops per visible (query head, key) pair (q.k, k.rho,
    e v and e p v), Hq * B * T (T + 1) / 2 pairs; bound by the bf16 matrix
    cores (2.5 PFLOP/s dense)."""
    import torch
    from parallax_covariance_corrected_amd import binding as pb
    B, T, Hq, Hkv, d = args.prefill_B, args.prefill_T, 16, 8, 128
    g = torch.Generator(device="cuda").manual_seed(0)
    q = torch.randn((B, T, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    rho = torch.randn((B, T, Hq, d), generator=g, device="cuda") * 0.9
    K = torch.randn((B, Hkv, T, d), generator=g, device="cuda").to(torch.bfloat16)
    V = torch.randn((B, Hkv, T, d), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device="cuda")
    print(f"# bench: prefill B={B} T={T} Hq={Hq} Hkv={Hkv} d={d}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        pb.prefill(q, rho, K, V, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        pb.prefill(q, rho, K, V, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    kern_us = per_launch_us(pb, lambda i: pb.prefill(q, rho, K, V, out=out), args.steps,
                            (("prefill", pb.KERNEL_PREFILL),))[0]["prefill"]
    pairs = Hq * B * T * (T + 1) // 2
    flops = 8 * d * pairs
    achieved = flops / (kern_us * 1e-6) / 1e12

    # Matched ratios: the softmax-only forward on the same inputs (same bytes,
    # half the algorithmic flops) and with twice the query heads (same flops).
    def kernel_us(fn):
        return per_launch_us(pb, lambda i: fn(), args.steps,
                             (("prefill", pb.KERNEL_PREFILL),))[0]["prefill"]
    soft_us = kernel_us(lambda: pb.prefill(q, None, K, V, out=out))
    q2 = torch.randn((B, T, 2 * Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    out2 = torch.empty((B, T, 2 * Hq, d), dtype=torch.bfloat16, device="cuda")
    soft2_us = kernel_us(lambda: pb.prefill(q2, None, K, V, out=out2))
    del q2, out2
    cpu = prefill_cpu_baseline(q, rho, K, V, budget_s=args.cpu_budget) if args.cpu_baseline else None
    line = {
        "metric": "Parallax prefill tokens/s (causal, many-query forward)",
        "value": round(B * T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"prefill_B{B}_T{T}_Hq{Hq}_Hkv{Hkv}_d{d}", "B": B, "T": T, "Hq": Hq,
                   "Hkv": Hkv, "d": d, "prefix": 0},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(achieved / 2500.0, 4), "traffic": None,
                     "kernel": "prefill_mfma_kernel", "algorithmic_flops_per_launch": flops,
                     "avg_launch_us": round(kern_us, 3),
                     "mfma_flops_issued_per_launch_note":
                         "14d per (row, key) incl. bf16 hi/lo splits, whole 64-key blocks"},
        "cpu_baseline": cpu,
        "matched": {"parallax_prefill_us": round(kern_us, 3), "softmax_prefill_us": round(soft_us, 3),
                    "softmax_2x_heads_prefill_us": round(soft2_us, 3),
                    "io_matched_speedup": round(soft_us / kern_us, 4),
                    "compute_matched_speedup": round(soft2_us / kern_us, 4)},
    }
    print(json.dumps(line), flush=True)


def prefill_cpu_baseline(q, rho, K, V, budget_s: float = 12.0):
    """The fp64 oracle on a bounded sample of (token, head) rows, scaled to the
    whole forward. Tokens are drawn uniformly, so the mean cost per row is an
    unbiased estimate (a row's cost grows with its token index)."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    B, T, Hq, d = q.shape
    qh = q.float().cpu().numpy().astype(np.float64)
    rh = rho.cpu().numpy().astype(np.float64)
    Kp = [K[b].float().cpu().numpy().astype(np.float64) for b in range(B)]
    Vp = [V[b].float().cpu().numpy().astype(np.float64) for b in range(B)]
    Hkv = K.shape[1]
    pre = np.zeros(B, dtype=np.int64)
    r = np.random.default_rng(0)
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        rows = [(int(r.integers(0, B)), int(r.integers(0, T)), int(r.integers(0, Hq))) for _ in range(8)]
        oracle.prefill_rows(qh, rh, Kp, Vp, pre, Hkv, rows)
        done += len(rows)
    el = time.perf_counter() - t0
    full_s = el / done * (B * T * Hq)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(B * T / full_s, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle on {done} uniformly drawn (token, head) rows of {B * T * Hq} "
                      f"in {el:.1f} s, scaled to the whole forward"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--sets", type=int, default=3)
    ap.add_argument("--hq", type=int, default=0,
                    help="query heads of the workload (a multiple of its KV heads): another "
                         "GQA group size at the same cache")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--no-configs", dest="configs", action="store_false",
                    help="skip the compact records of the other four workloads")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--no-sweep-record", dest="sweep_record", action="store_false",
                    help="skip the compact batch x context record of the default line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 256 MiB device-to-device 3 times (a kernel of known "
                         "traffic, to scale hardware byte counters)")
    ap.add_argument("--sweep-max-gib", type=int, default=0)
    ap.add_argument("--fusion-sweep", action="store_true",
                    help="time the probe inside the decode kernel against a separate probe "
                         "launch over batch x d_model x context")
    ap.add_argument("--prefill", action="store_true",
                    help="measure the causal many-query forward instead of decode")
    ap.add_argument("--prefill-T", type=int, default=4096)
    ap.add_argument("--prefill-B", type=int, default=1)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the Parallax decode path here is built and "
              "measured on a single MI355X (multi-GPU sharding is a design note, not a run).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.sweep:
        run_sweep(args)
        return
    if args.fusion_sweep:
        run_fusion_sweep(args)
        return
    if args.prefill:
        run_prefill(args)
        return
    run_workload(args, args.workload)


if __name__ == "__main__":
    main()
