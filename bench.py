#!/usr/bin/env python3
"""Benchmark: useful (unpadded, unmasked) attention TFLOPS of jagged attention fwd+bwd on 1 MI355X.

A step is one pass of the whole hot path over one batch: the forward pass (work-list driven
forward kernel and, when the plan split items, the combine kernel) and the backward pass
(dQ kernel, which also forms Delta = rowsum(dO * O), dK/dV kernel, partial reduces), all through
the C ABI. The plan (offset validation and the longest-first work lists) is built once per batch
of offsets before the timed region; its host time is reported as ``plan_ms`` (first plan of the
process) and ``plan_ms_steady`` (a plan for a reordered batch built while a step runs, as a
training loop would build the next batch's plan).

``value`` is useful FLOPs per step over the wall time of the K timed steps (bracketed by device
synchronisations); ``median_step_ms`` is the median of the per-step HIP-event times. The timed
steps carry the library's per-launch timing events (the per-kernel times come from them);
``no_kernel_events`` repeats the K steps without them.

Useful FLOPs per visible (query, key) pair and head: 4 D forward + 10 D backward. Inputs are the
seeded synthetic workload from ``jfa_inputs``, resident in HBM before timing starts.

Prints ONE JSON line. ``--gpus`` above 1 is refused: this build runs on one GPU.
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

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA (the scaled MX products run at this rate)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
METRIC = "useful (unpadded) attention TFLOPS fwd+bwd and % of bf16 MFMA peak, 1×MI355X"
DEFAULT_WORKLOAD = "longtail"  # the long-tail production-like workload (B = 512, 333,877 tokens)
# FLOPs each kernel must execute per visible pair and head (its own matrix products):
#   forward: S = QK^T, O = PV; dK/dV: S, dP = dO V^T, dV = P^T dO, dK = dS^T Q; dQ: S, dP, dQ = dS K
#   fused short-query backward: S, dP, dV, dK and dQ once each
KERNEL_FLOPS_PER_PAIR_D = {"forward": 4, "dkdv": 8, "dq": 6, "bwd_fused": 10}


def kernel_bytes(kernel: str, Tq: int, Tkv: int, H: int, D: int, out_bytes: int, softmax: bool,
                 mx: bool = False) -> int:
    """Algorithmic HBM bytes of one launch: every tensor the kernel must read or write, once.

    bf16 inputs (2 bytes per element; MXFP8 forward: 1 byte plus one scale byte per 32 elements);
    outputs and gradients in the chosen dtype; lse and Delta fp32.
    forward: read Q, K, V; write O (and lse). dK/dV: read Q, dO, K, V (lse, Delta); write dK, dV.
    dQ: read Q, dO, K, V (lse, Delta); write dQ. Fused short-query backward: read Q, dO, K, V, O
    (for Delta) and lse; write dQ, dK, dV.
    """
    q, kv = Tq * H * D, Tkv * H * D
    stats = 2 * Tq * H * 4 if softmax else 0
    if kernel == "forward":
        ins = (q + 2 * kv) * 33 // 32 if mx else 2 * (q + 2 * kv)
        return ins + out_bytes * q + (Tq * H * 4 if softmax else 0)
    if kernel == "dkdv":
        return 2 * (2 * q + 2 * kv) + stats + out_bytes * 2 * kv
    if kernel == "bwd_fused":
        return 2 * (2 * q + 2 * kv) + out_bytes * q + Tq * H * 4 + out_bytes * (2 * kv + q)
    return 2 * (2 * q + 2 * kv) + stats + out_bytes * q


KERNEL_SOURCES = {"forward": ["fwd.hip", "device_common.h", "tile_lds.h", "jfa_internal.h"],
                  "dkdv": ["bwd.hip", "device_common.h", "tile_lds.h", "jfa_internal.h"],
                  "dq": ["bwd.hip", "device_common.h", "tile_lds.h", "jfa_internal.h"],
                  "bwd_fused": ["bwd.hip", "device_common.h", "tile_lds.h", "jfa_internal.h"]}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "jagged_sequence_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None.

    The summary under profiles/ records FETCH_SIZE and WRITE_SIZE per dispatch (KiB), the copy-kernel
    calibration factor and the hash of the kernel sources it was taken with; a changed kernel makes
    the figure stale and it is not reported.
    """
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_hash:\s*(\w+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != source_hash(kernel):
        return None
    return float(t.group(1))


def host_cpu():
    """(model name, cores this process may run on) of the host."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return model, n


def _parse_clock(tool: str, text: str):
    if tool == "amd-smi":  # sections "GFX_<n>:" followed by "CLK: <v> MHz"
        vals = [int(m.group(1)) for m in re.finditer(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", text)]
    else:
        vals = [int(v) for v in re.findall(r"sclk[^(]*\((\d+)\s*Mhz\)", text, re.I)]
    if not vals:
        return None
    return {"mhz_max": max(vals), "mhz_mean": round(sum(vals) / len(vals), 1), "source": tool}


def gpu_clock_under_load(step, seconds: float, median_ms: float):
    """Shader (GFX) clock in MHz as the SMI tool samples it while steps run.

    Steps keep the GPU busy for a second before the tool starts (its reading averages over a recent
    window, so a short busy period reads as idle) and until it has printed (at most ``seconds``):
    chunks of about 50 ms of steps, a new one queued whenever the oldest of two queued chunks has
    finished, so the queue never runs dry and never holds much more than the tool's remaining
    sampling time. These steps are outside the timed region. Not run under a profiler (the tool is
    a script whose interpreter the profiler's preload would follow)."""
    import subprocess

    import torch
    if any("ROCPROF" in k for k in os.environ) or "rocprof" in os.environ.get("LD_PRELOAD", ""):
        return None
    per_chunk = max(1, int(50.0 / max(median_ms, 1e-3)))

    def chunk():
        for _ in range(per_chunk):
            step()
        ev = torch.cuda.Event()
        ev.record()
        return ev

    for tool, cmd in (("amd-smi", ["amd-smi", "metric", "--clock"]), ("rocm-smi", ["rocm-smi", "--showclocks"])):
        queued = [chunk(), chunk()]
        t_busy = time.perf_counter() + 1.0
        while time.perf_counter() < t_busy:
            queued.pop(0).synchronize()
            queued.append(chunk())
        try:
            proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
        except OSError:
            torch.cuda.synchronize()
            continue
        t_end = time.perf_counter() + seconds
        while proc.poll() is None and time.perf_counter() < t_end:
            queued.pop(0).synchronize()
            queued.append(chunk())
        torch.cuda.synchronize()
        try:
            text = proc.communicate(timeout=60)[0]
        except subprocess.SubprocessError:
            proc.kill()
            continue
        res = _parse_clock(tool, text)
        if res:
            res["sampled_during_steps"] = True
            return res
    return None


def cpu_baseline(x, workload, seconds_target=15.0):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload's sequences."""
    import numpy as np

    from oracle import attention as A

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    model, nproc = host_cpu()
    cores = blas_threads or nproc
    import jfa_inputs as ji
    from jagged_sequence_amd.flops import useful_flops
    f = A.bf16_bits_to_f64
    lq = np.diff(x.q_off.astype(np.int64))
    lkv = np.diff(x.kv_off.astype(np.int64))
    causal = x.mask == "causal"
    bw_on = workload_backward(workload)
    bias = None if x.bias is None else x.bias.astype(np.float64)
    kw = dict(mask=x.mask, act=x.act, bias_kind=x.bias_kind, bias=bias, window=x.window, block=x.block)

    def sample(seqs):
        rows = np.concatenate([np.arange(x.q_off[b], x.q_off[b + 1]) for b in seqs])
        krows = np.concatenate([np.arange(x.kv_off[b], x.kv_off[b + 1]) for b in seqs])
        sq = np.concatenate([[0], np.cumsum(lq[seqs])])
        sk = np.concatenate([[0], np.cumsum(lkv[seqs])])
        return rows, krows, sq, sk

    def run(seqs):
        rows, krows, sq, sk = sample(seqs)
        k, v = f(x.k[krows]), f(x.v[krows])
        t0 = time.perf_counter()
        if ji.WORKLOADS[workload].mxfp8:  # the MXFP8 forward oracle
            from oracle import mx
            mx.forward(f(x.q[rows]), k, v, sq, sk, mask=x.mask, bias_kind=x.bias_kind, bias=bias,
                       window=x.window, block=x.block)
        elif x.shared_q:  # the seed rows are shared by every sequence
            A.forward_shared_q(f(x.q), k, v, sk, **kw)
            if bw_on:
                A.backward_shared_q(f(x.q), k, v, sk, f(x.do[rows]), **kw)
        else:
            q = f(x.q[rows])
            A.forward(q, k, v, sq, sk, **kw)
            if bw_on:
                A.backward(q, k, v, sq, sk, f(x.do[rows]), **kw)
        return time.perf_counter() - t0

    # the oracle's cost follows the dense score rows it forms, whatever the window or block
    n = np.minimum(lq, lkv)
    cost = ((n * (n + 1) // 2) if causal else lq * lkv).astype(np.float64) * (4 + (10 if bw_on else 0)) * x.D * x.H
    # The sample: the sequences in order, each timed on its own (the oracle handles sequences one
    # after another), until the timed total reaches the target; a sequence whose predicted time
    # (its cost at the fastest rate seen so far) would take the total past twice the target is
    # skipped.
    seqs, dt, best_rate, skipped = [], 0.0, 0.0, 0
    for b in range(len(lq)):
        if dt >= seconds_target:
            break
        if best_rate > 0 and dt + cost[b] / best_rate > 2 * seconds_target:
            skipped += 1
            continue
        t = run([b])
        dt += t
        seqs.append(b)
        best_rate = max(best_rate, cost[b] / max(t, 1e-9))
    _, _, sq, sk = sample(seqs)
    fw, bw = useful_flops(sq, sk, x.H, x.D, causal, workload_backward(workload), x.window, x.block)
    return {"value": (fw + bw) / dt / 1e12, "unit": "TFLOPS", "cores": int(cores), "kind": "oracle",
            "nproc": nproc, "cpu_model": model, "blas_threads": blas_threads,
            "sample": f"{len(seqs)} of {len(lq)} sequences (in order; {skipped} longer ones skipped), all {x.H} heads, "
                      f"fwd{'+bwd' if workload_backward(workload) else ''}, {dt:.1f} s, numpy float64 "
                      f"(matrix products in BLAS with {cores} threads, elementwise steps on one)"}


def workload_backward(name: str) -> bool:
    import jfa_inputs as ji
    return ji.WORKLOADS[name].backward


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true", help="skip the SMI clock sample after the timed region")
    ap.add_argument("--out-dtype", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--dbias", action="store_true",
                    help="also compute the bias gradient in every backward pass (a learned bias needs it)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 3 device-to-device copies of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the benchmark runs on one GPU only "
              f"(the attention shards by heads or sequences with no exchange; see the design notes)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import jfa_inputs as ji
    from jagged_sequence_amd import binding as J
    from jagged_sequence_amd.flops import useful_flops, visible_pairs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n}), flush=True)
        return 0
    w = ji.WORKLOADS[args.workload]
    x = ji.workload_inputs(args.workload)
    causal = w.mask == "causal"
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = dev(x.q), dev(x.k), dev(x.v)
    do = dev(x.do) if w.backward else None
    qo, ko = torch.from_numpy(x.q_off).cuda(), torch.from_numpy(x.kv_off).cuda()
    bias = torch.from_numpy(x.bias).cuda() if x.bias is not None else None
    torch.cuda.synchronize()

    plan_kw = dict(mask=w.mask, act=w.act, bias=w.bias, window=w.window, block=w.block, out_dtype=args.out_dtype,
                   grad_dtype=args.out_dtype, shared_q=x.shared_q, mxfp8=w.mxfp8)
    t0 = time.perf_counter()
    plan = J.Plan(x.q_off, x.kv_off, w.H, w.D, **plan_kw)
    plan_ms = (time.perf_counter() - t0) * 1e3
    fwd_ws, bwd_ws = plan.workspace_bytes()
    ws_f = torch.empty(max(fwd_ws, 1), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(max(bwd_ws, 1), dtype=torch.uint8, device="cuda")
    odt = torch.float32 if args.out_dtype == "f32" else torch.bfloat16
    Tq = int(x.q_off[-1])
    out = torch.empty((Tq, w.H, w.D), dtype=odt, device="cuda")
    lse = torch.empty((w.H, Tq), dtype=torch.float32, device="cuda") if w.act == "softmax" else None
    dq = torch.empty((x.q.shape[0], w.H, w.D), dtype=odt, device="cuda")  # shared queries: one set of rows
    dk = torch.empty((x.k.shape[0], w.H, w.D), dtype=odt, device="cuda")
    dv = torch.empty_like(dk)
    want_db = args.dbias and bias is not None and w.backward
    db = torch.empty(bias.shape, dtype=torch.float32, device="cuda") if want_db else None
    stream = torch.cuda.current_stream()

    def step():
        plan.forward(q, k, v, qo, ko, bias, out=out, lse=lse, workspace=ws_f, stream=stream)
        if w.backward:
            plan.backward(q, k, v, qo, ko, bias, out, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws_b, stream=stream,
                          dbias=db)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Planning in steady state: offsets change with every batch, so the next batch's plan is built
    # while the GPU runs the current step. Here a batch with the same lengths in another order (new
    # offsets) is planned while a step runs; the host time of that call is reported.
    perm = np.random.default_rng(1).permutation(w.B)
    lq_b, lkv_b = np.diff(x.q_off)[perm], np.diff(x.kv_off)[perm]
    qo2, ko2 = ji.offsets(lq_b), ji.offsets(lkv_b)
    steady = []
    for _ in range(3):
        step()
        t1 = time.perf_counter()
        p2 = J.Plan(qo2, ko2, w.H, w.D, **plan_kw)
        steady.append((time.perf_counter() - t1) * 1e3)
        del p2
    torch.cuda.synchronize()

    # The library creates its timing events on first use: K untimed steps with timing on fill its
    # event pool, and enabling timing again clears their records, so the timed steps reuse events.
    plan.timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    plan.timing_enable(True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]  # step boundaries
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    median_ms = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])
    kernels = {}
    for name in J.KERNELS:
        ms, n = plan.timing_read(name)
        if n:
            kernels[name] = {"avg_ms": ms / n, "launches_per_step": n / args.steps, "total_ms": ms}
    plan.timing_enable(False)

    # The same number of steps without the per-launch timing events (outside the timed region), as a
    # caller that does not time kernels runs them.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    no_events_ms = e0.elapsed_time(e1) / args.steps

    # Cold-cache rung of the metric ladder (outside the timed region): the same step after 512 MiB
    # have been written over the caches (twice the 256 MB last-level cache), so that every input
    # comes from HBM.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = []
    plan.timing_enable(True)
    for _ in range(min(args.steps, 10)):
        flush.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush
    cold_kernels = {}
    for name in J.KERNELS:
        ms, n = plan.timing_read(name)
        if n:
            cold_kernels[name] = round(ms / n, 5)
    plan.timing_enable(False)
    cold.sort()
    cold_ms = cold[len(cold) // 2] if len(cold) % 2 else 0.5 * (cold[len(cold) // 2 - 1] + cold[len(cold) // 2])
    clock = None if args.no_clock else gpu_clock_under_load(step, 20.0, median_ms)
    torch.cuda.synchronize()

    fw, bw = useful_flops(x.q_off, x.kv_off, w.H, w.D, causal, w.backward, w.window, w.block)
    ms_per_step = elapsed / args.steps * 1e3
    props = torch.cuda.get_device_properties(0)
    with open(J.LIB_PATH, "rb") as fh:
        lib_hash = hashlib.sha256(fh.read()).hexdigest()[:16]
    value = (fw + bw) / (elapsed / args.steps) / 1e12
    pairs = visible_pairs(x.q_off, x.kv_off, causal, w.window, w.block) * w.H

    # roofline of the dominant kernel (largest share of the timed region): its algorithmic FLOPs and
    # bytes per launch decide the bound (MFMA above the ridge point, HBM below it)
    dom = max((kk for kk in kernels if kk in KERNEL_FLOPS_PER_PAIR_D), key=lambda kk: kernels[kk]["total_ms"])
    per_launch_flops = KERNEL_FLOPS_PER_PAIR_D[dom] * w.D * pairs / kernels[dom]["launches_per_step"]
    out_b = 4 if args.out_dtype == "f32" else 2
    per_launch_bytes = kernel_bytes(dom, int(x.q_off[-1]), int(x.kv_off[-1]), w.H, w.D, out_b, w.act == "softmax",
                                    mx=w.mxfp8)
    secs = kernels[dom]["avg_ms"] * 1e-3
    traffic = counter_traffic(dom, args.workload)
    # a contraction is priced at the peak of its own operand type: the MXFP8 forward's products are
    # scaled fp8 MFMAs
    peak = PEAK_FP8_TFLOPS if (w.mxfp8 and dom == "forward") else PEAK_BF16_TFLOPS
    if per_launch_flops / per_launch_bytes >= peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = per_launch_flops / secs / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": dom,
                    "algorithmic_flops_per_launch": per_launch_flops, "algorithmic_bytes_per_launch": per_launch_bytes}
    else:
        achieved = per_launch_bytes / secs / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic, "kernel": dom,
                    "algorithmic_flops_per_launch": per_launch_flops, "algorithmic_bytes_per_launch": per_launch_bytes}

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8 (e4m3 + e8m0 block scales)" if w.mxfp8 else "bf16",
        "data": "synthetic (seeded jagged lengths and N(0,1) bf16 values; no dataset)",
        "config": {"workload": args.workload, "B": w.B, "H": w.H, "D": w.D, "mask": w.mask, "act": w.act,
                   "bias": w.bias, "window": w.window, "block": w.block, "tokens_q": int(x.q_off[-1]), "tokens_kv": int(x.kv_off[-1]),
                   "visible_pairs_x_heads": int(pairs), "out_dtype": args.out_dtype, "bias_gradient": bool(want_db),
                   "description": w.description},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "median_step_ms": round(median_ms, 4),
        "value_at_median_step": round((fw + bw) / (median_ms * 1e-3) / 1e12, 2),
        "no_kernel_events": {"ms_per_step": round(no_events_ms, 4),
                             "value": round((fw + bw) / (no_events_ms * 1e-3) / 1e12, 2),
                             "note": "the same steps without the library's per-launch timing events"},
        "cold_cache": {"median_step_ms": round(cold_ms, 4), "steps": len(cold), "kernels_avg_ms": cold_kernels,
                       "value_at_median_step": round((fw + bw) / (cold_ms * 1e-3) / 1e12, 2),
                       "flush": "512 MiB written before each step (caches cold), outside the timed region"},
        "plan_ms": round(plan_ms, 3),
        "plan_ms_steady": round(min(steady), 3),
        "gpu": {"name": props.name, "arch": getattr(props, "gcnArchName", None), "cus": props.multi_processor_count,
                "clock_during_run": clock},
        "library": {"path": os.path.relpath(J.LIB_PATH, ROOT), "sha256": lib_hash},
        "kernels": {kk: {"avg_ms": round(vv["avg_ms"], 5), "per_step": vv["launches_per_step"]}
                    for kk, vv in kernels.items()},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, args.workload)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
