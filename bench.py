"""Benchmark of the sink-aware GQA attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload full] [--pass fwd|bwd]

A step is one sink_attn_fwd call (K prologue + varlen schedule, then attention
with the fused Q prologue) over one synthetic batch already resident in HBM.
The default workload is the full-causal layer: one document of 32768 tokens,
32 query / 4 kv heads, head_dim 128, bf16, no RoPE, sinks N(0,1).

Throughput counts visible score entries only:
    N_vis = sum over documents of sum_{i < L} min(i + 1, W)   (W = inf when causal)
    FLOP  = 4 * head_dim * Hq * N_vis      (QK^T and PV, 2 * head_dim each)
and is reported in TFLOP/s for the whole step.  The printed JSON line also
carries the roofline of the dominant kernel (the attention stage, timed with
HIP events on the stream it is launched on) against the bf16 dense MFMA peak,
and the fp64 CPU oracle timed on a bounded sample of the same workload.  The
attention stage is one launch of the narrow-tile kernel or, with wide tiles,
the main launch plus the follow-up that reruns the (normally no) blocks whose
fixed softmax reference proved too low; the events cover both.

--workload sliding_bshd times the padded entry point (sink_attn_fwd_padded):
a BSHD batch of 8 rows of 4096 slots with trailing padding (real lengths those
of the sliding workload), the boundaries computed once from the attention mask
before the timed region (sink_attn_mask_to_seqlens, timed on its own); the
step's events cover all of its launches (K prologue, attention, padding-row
fill).  FLOP counts real visible entries only.

--dtype f16 runs the same step on fp16 q, k, v and out (the fp16 I/O
variant; fp16 and bf16 share the 2.5 PFLOP/s dense MFMA peak).

Timing.  value = FLOP / (wall time of the K timed steps / K), the steps
bracketed by torch.cuda.synchronize().  Each step also carries HIP events on
its stream, which give the median and minimum per-call time ("timing").  The
default run then times the other forward workloads (sliding, long,
mixed_sliding, mixed_causal) as extra keys of the same line ("workloads"),
each by the protocol: 3 warm-up calls, then max(10, ceil(200 ms / t)) calls
with HIP events, median and minimum of the whole call and of each stage.
These have no CPU leg.  The CPU leg's parity sample (out and lse against
the oracle) must meet the bf16 bounds (max-abs 2e-2, mean-abs 2e-3):
otherwise the line is still printed and bench.py exits with status 3.

--pass bwd times the backward instead: a step is one sink_attn_bwd call (key
and column tile preparation, the dK/dV and dQ kernels, the final sums) on the
out and lse of one forward, counted as 2.5 forward passes
(FLOP = 10 * head_dim * Hq * N_vis: recomputed scores, dP, dV, dK and dQ).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sink-attn fwd TFLOP/s (visible entries) + % bf16 MFMA peak, 32q/4kv d128, 1 GPU"
METRIC_BWD = ("sink-attn bwd TFLOP/s (visible entries, 10*d*Hq per entry) + % bf16 MFMA peak, "
              "32q/4kv d128, 1 GPU")
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
CSRC = os.path.join(ROOT, "attention_qk_rmsnorm_amd", "csrc")
# tile configuration -> (attention kernel, its source file)
ATTN_KERNELS = {1: ("attn_fwd_narrow_kernel", "attn_narrow.hip"),
                2: ("attn_fwd_wide_kernel", "attn_wide.hip"),
                3: ("attn_fwd_wide_kernel", "attn_wide.hip")}
TILE_NAMES = {1: "narrow", 2: "wide", 3: "wide_exact"}
TILE_CHOICES = {"auto": 0, "narrow": 1, "wide": 2, "wide_exact": 3}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_wide_traffic.json")
PARITY_MAX, PARITY_MEAN = 2e-2, 2e-3   # bf16 bounds against the fp64 oracle
OTHER_WORKLOADS = ("sliding", "long", "mixed_sliding", "mixed_causal")


def protocol_calls(t_ms: float) -> int:
    """Timed calls of the measurement protocol: max(10, ceil(200 ms / t))."""
    return max(10, math.ceil(200.0 / max(t_ms, 1e-3)))


def library_record(A) -> dict:
    """Which build of the library this process loaded (path and sha256)."""
    path = os.path.realpath(A.library_path())
    return {"path": os.path.relpath(path, ROOT) if path.startswith(ROOT) else path,
            "sha256": source_digest(path)[:16]}


def stats_ms(xs) -> dict:
    xs = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(xs)), "min": float(xs.min()), "mean": float(xs.mean())}


def time_forward_stages(call, stream, n: int):
    """n forward calls, each with HIP events around its two stages (K prologue
    and schedule; attention) on the launch stream.  Returns per-call lists of
    (prologue ms, attention ms)."""
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    for i in range(n):
        ev[i][0].record(stream)
        call.prologue()
        ev[i][1].record(stream)
        call.attention()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    return ([e[0].elapsed_time(e[1]) for e in ev], [e[1].elapsed_time(e[2]) for e in ev])


def other_workloads(A, dev, names) -> dict:
    """The other forward workloads by the timing protocol (no CPU leg)."""
    import torch
    import workloads
    res = {}
    stream = torch.cuda.current_stream(dev)
    ws = workloads.named_workloads()
    cache = {}
    for name in names:
        w = ws[name]
        key = (w.lengths, w.dtype)
        if key not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            cache[key] = {k: v.to(dev) for k, v in workloads.make_inputs(w, seed=0).items()}
        d = cache[key]
        call = A.Call(d["q"], d["k"], d["v"], d["cu_seqlens"], d["sinks"], d["qnorm_w"],
                      d["knorm_w"], w.window, w.use_rope, rms_eps=w.rms_eps,
                      rope_theta=w.rope_theta)
        for _ in range(3):
            call.fwd()
        torch.cuda.synchronize()
        pro, attn = time_forward_stages(call, stream, 3)
        n = protocol_calls(float(np.median(np.add(pro, attn))))
        pro, attn = time_forward_stages(call, stream, n)
        tot = np.add(pro, attn)
        flop = 4.0 * w.head_dim * w.num_q_heads * visible_entries(w.lengths, w.window)
        med = float(np.median(tot))
        res[name] = {
            "workload": w.description, "tokens": w.total_tokens, "docs": w.num_docs,
            "window": w.window, "rope": w.use_rope,
            "tile_config": TILE_NAMES[A.tile_config(call.desc, w.window)],
            "flop": flop, "calls": n,
            "call_ms": stats_ms(tot), "prologue_ms": stats_ms(pro), "attention_ms": stats_ms(attn),
            "tflops_median": flop / (med * 1e-3) / 1e12,
            "pct_bf16_peak_median": 100.0 * flop / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "attention_tflops_median": flop / (float(np.median(attn)) * 1e-3) / 1e12,
        }
        del call
    cache.clear()
    torch.cuda.empty_cache()
    return res


def parity_ok(base) -> bool:
    p = (base or {}).get("parity_on_sample")
    if not p:
        return True
    return (p["out_max_abs"] <= PARITY_MAX and p["out_mean_abs"] <= PARITY_MEAN
            and p["lse_max_abs"] <= PARITY_MAX and p["lse_mean_abs"] <= PARITY_MEAN)


def visible_entries(lengths, window: int) -> int:
    total = 0
    for L in lengths:
        L = int(L)
        if window <= 0 or window >= L:
            total += L * (L + 1) // 2
        else:
            total += window * (window + 1) // 2 + (L - window) * window
    return total


def source_digest(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_traffic(workload: str, kernel: str, source: str):
    """HBM bytes per attention launch from the committed rocprofv3 PMC summary,
    or None when it is missing, for another workload or kernel, or the kernel
    source has changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (t.get("workload") != workload or t.get("kernel") != kernel
            or t.get("source_sha256") != source_digest(os.path.join(CSRC, source))):
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(inp, w, out_gpu, lse_gpu, target_seconds: float):
    """The fp64 oracle as it stands, on an evenly spaced sample of query tokens
    (all heads of each), sized to about target_seconds of host time."""
    import oracle.oracle as O
    k = inp["k"].double().numpy()
    v = inp["v"].double().numpy()
    common = dict(cu_seqlens=inp["cu_seqlens"].numpy(), sinks=inp["sinks"].double().numpy(),
                  qnorm_w=inp["qnorm_w"].double().numpy(),
                  knorm_w=inp["knorm_w"].double().numpy(), window=w.window,
                  use_rope=w.use_rope, eps=w.rms_eps, theta=w.rope_theta)
    T = w.total_tokens
    cu = inp["cu_seqlens"].numpy()
    pos = np.concatenate([np.arange(L) for L in w.lengths])

    def vis_of(rows):
        p = pos[rows].astype(np.int64) + 1
        return int(np.minimum(p, w.window).sum() if w.window > 0 else p.sum())

    def run(n):
        rows = np.unique(np.linspace(0, T - 1, n).round().astype(np.int32))
        q = inp["q"][rows].double().numpy()
        t0 = time.perf_counter()
        out, lse = O.sink_attn_fwd(q, k, v, rows=rows, **common)
        return rows, out, lse, time.perf_counter() - t0

    rows, _, _, dt = run(16)                     # calibration run (not reported)
    rate = vis_of(rows) / max(dt, 1e-6)
    per_row = vis_of(np.arange(T, dtype=np.int32)) / T
    n = int(min(T, max(16, target_seconds * rate / per_row)))
    rows, out, lse, dt = run(n)
    n_vis = vis_of(rows)
    flop = 4.0 * w.head_dim * w.num_q_heads * n_vis
    got = out_gpu[rows].float().cpu().numpy()
    err = np.abs(got - out)
    lerr = np.abs(lse_gpu[:, rows].cpu().numpy() - lse)
    del cu
    return {
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": O.max_threads(),
        "kind": "oracle",
        "sample": (f"{len(rows)} query tokens evenly spaced over the {T}-token batch, all "
                   f"{w.num_q_heads} heads each ({n_vis} visible entries per head, "
                   f"{flop:.3e} FLOP), fp64, {dt:.1f} s"),
        "seconds": dt,
        "parity_on_sample": {"out_max_abs": float(err.max()), "out_mean_abs": float(err.mean()),
                             "lse_max_abs": float(lerr.max()),
                             "lse_mean_abs": float(lerr.mean()),
                             "bounds": {"max_abs": PARITY_MAX, "mean_abs": PARITY_MEAN}},
    }


def cpu_baseline_bwd(w, target_seconds: float):
    """The fp64 backward oracle as it stands on a prefix of the workload's first
    document, taken as a document of its own, sized to about target_seconds."""
    import oracle.oracle as O
    import workloads

    def run(L):
        sub = workloads.custom_workload([L], w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype,
                                        w.window, w.use_rope, w.sink_mean)
        inp = workloads.make_inputs(sub, seed=0)
        dout = workloads.make_grad_output(sub, seed=0)
        f = lambda t: t.double().numpy()  # noqa: E731
        t0 = time.perf_counter()
        O.sink_attn_bwd(f(inp["q"]), f(inp["k"]), f(inp["v"]), inp["cu_seqlens"].numpy(),
                        f(inp["sinks"]), f(inp["qnorm_w"]), f(inp["knorm_w"]), w.window,
                        w.use_rope, f(dout), eps=w.rms_eps, theta=w.rope_theta)
        return time.perf_counter() - t0

    L = min(256, w.lengths[0])
    dt = run(L)                                   # calibration run (not reported)
    rate = visible_entries([L], w.window) / max(dt, 1e-6)
    L = max(L, min(w.lengths[0], 8192))
    while L > 256 and visible_entries([L], w.window) / rate > target_seconds:
        L = int(L * 0.8)
    dt = run(L)
    n_vis = visible_entries([L], w.window)
    flop = 10.0 * w.head_dim * w.num_q_heads * n_vis
    return {
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": O.max_threads(),
        "kind": "oracle",
        "sample": (f"backward of the first {L} tokens of the workload's first document as a "
                   f"document of its own, all {w.num_q_heads} heads ({n_vis} visible entries "
                   f"per head, {flop:.3e} FLOP), fp64, {dt:.1f} s"),
        "seconds": dt,
    }


def unpadded_view(inp, w, out_gpu, lse_gpu):
    """The real rows of a padded workload as an unpadded batch (the oracle's
    own definition of the padded call: its real rows are the unpadded call on
    the gathered documents), with the matching rows of the GPU results."""
    import workloads
    rows = np.concatenate([np.arange(b * w.pad_to, b * w.pad_to + L)
                           for b, L in enumerate(w.lengths)]).astype(np.int64)
    sub = workloads.custom_workload(w.lengths, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                    w.dtype, w.window, w.use_rope, w.sink_mean,
                                    name=w.name + " (real rows)")
    got = dict(inp, q=inp["q"][rows], k=inp["k"][rows], v=inp["v"][rows])
    return got, sub, out_gpu[rows], lse_gpu[:, rows]


def run_fwd_padded(args, A, w, inp, d_inp, dev):
    import torch

    cu, cu_padded = A.mask_to_seqlens(d_inp["attention_mask"])
    if not (torch.equal(cu.cpu(), inp["cu_seqlens"])
            and torch.equal(cu_padded.cpu(), inp["cu_seqlens_padded"])):
        raise RuntimeError("mask_to_seqlens disagrees with the workload's boundaries")
    stream = torch.cuda.current_stream(dev)
    m_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    mask_ms = []
    for _ in range(3):
        m_ev[0].record(stream)
        A.mask_to_seqlens(d_inp["attention_mask"])   # checks the mask: synchronises
        m_ev[1].record(stream)
        torch.cuda.synchronize()
        mask_ms.append(m_ev[0].elapsed_time(m_ev[1]))
    call = A.Call(d_inp["q"], d_inp["k"], d_inp["v"], cu, d_inp["sinks"], d_inp["qnorm_w"],
                  d_inp["knorm_w"], w.window, w.use_rope, rms_eps=w.rms_eps,
                  rope_theta=w.rope_theta, cu_seqlens_padded=cu_padded)
    for _ in range(args.warmup):
        call.fwd()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        call.fwd()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    call_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    n_vis = visible_entries(w.lengths, w.window)
    flop = 4.0 * w.head_dim * w.num_q_heads * n_vis
    value = flop / (ms_step * 1e-3) / 1e12
    achieved = flop / (call_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.description}",
            "tokens": w.total_tokens, "rows": w.num_rows, "docs": w.num_docs,
            "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "window": w.window, "rope": w.use_rope, "visible_entries": n_vis,
            "flop_per_step": flop, "parallelism": "single GPU",
        },
        "pct_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "roofline": {
            "bound": "mfma",
            "kernel": "sink_attn_fwd_padded (all launches)",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": None,
            "avg_launch_ms": call_ms,
        },
        "kernels": {"mask_to_seqlens_ms": float(np.median(mask_ms))},
        "library": library_record(A),
    }
    if args.cpu_seconds > 0:
        call.fwd()
        torch.cuda.synchronize()
        got, sub, out_r, lse_r = unpadded_view(inp, w, call.out, call.lse)
        base = cpu_baseline(got, sub, out_r, lse_r, args.cpu_seconds)
        base["sample"] += " (the real rows of the padded batch)"
        result["cpu_baseline"] = base
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    if not parity_ok(result["cpu_baseline"]):
        print("bench.py: the GPU result misses the bf16 bounds on the oracle's sample",
              file=sys.stderr)
        sys.exit(3)


def run_bwd(args, A, w, d_inp, call, dev):
    import torch
    import workloads

    call.fwd()
    dout = workloads.make_grad_output(w, seed=0).to(dev)
    torch.cuda.synchronize()
    bc = A.BwdCall(d_inp["q"], d_inp["k"], d_inp["v"], d_inp["cu_seqlens"], d_inp["sinks"],
                   d_inp["qnorm_w"], d_inp["knorm_w"], w.window, w.use_rope, call.out, call.lse,
                   dout, rms_eps=w.rms_eps, rope_theta=w.rope_theta,
                   cu_seqlens_padded=d_inp.get("cu_seqlens_padded"),
                   tile_config=TILE_CHOICES[args.tile])
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        bc.run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        bc.run()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    call_l = [e[0].elapsed_time(e[1]) for e in ev]
    n_proto = protocol_calls(float(np.median(call_l)))
    if n_proto > args.steps and not args.quick:
        # more calls for the per-call statistics, after the timed region
        ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
               for _ in range(n_proto - args.steps)]
        for e in ev2:
            e[0].record(stream)
            bc.run()
            e[1].record(stream)
        torch.cuda.synchronize()
        call_l += [e[0].elapsed_time(e[1]) for e in ev2]
    call_ms = float(np.mean(call_l[:args.steps]))
    n_vis = visible_entries(w.lengths, w.window)
    flop = 10.0 * w.head_dim * w.num_q_heads * n_vis
    value = flop / (ms_step * 1e-3) / 1e12
    achieved = flop / (call_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC_BWD,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{w.name} backward: {w.description}",
            "tokens": w.total_tokens, "rows": w.num_rows, "docs": w.num_docs,
            "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "window": w.window, "rope": w.use_rope, "visible_entries": n_vis,
            "flop_per_step": flop, "parallelism": "single GPU",
        },
        "pct_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "roofline": {
            "bound": "mfma",
            "kernel": "sink_attn_bwd%s (all launches)" % ("_padded" if w.pad_to else ""),
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": None,
            "avg_launch_ms": call_ms,
        },
        "timing": {"calls": len(call_l), "protocol_calls": n_proto,
                   "call_ms": stats_ms(call_l),
                   "tflops_median": flop / (float(np.median(call_l)) * 1e-3) / 1e12},
        "library": library_record(A),
    }
    result["cpu_baseline"] = (cpu_baseline_bwd(w, args.cpu_seconds) if args.cpu_seconds > 0
                              else None)
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="full",
                    choices=["full", "sliding", "long", "mixed_sliding", "mixed_causal",
                             "sliding_bshd"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target host time of the oracle sample (0 skips the CPU baseline)")
    ap.add_argument("--dtype", default=None, choices=["bf16", "f16"],
                    help="storage dtype of q, k, v, out (default: the workload's, bf16); f16 "
                         "runs the fp16 I/O variant")
    ap.add_argument("--pass", dest="which", default="fwd", choices=["fwd", "bwd"],
                    help="time the forward (default) or the backward pass")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--tile", default="auto", choices=list(TILE_CHOICES),
                    help="attention tile configuration (default: the library's automatic "
                         "choice)")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other forward workloads the default run also times")
    ap.add_argument("--quick", action="store_true",
                    help="time exactly the K steps (no extra calls for the per-call "
                         "statistics, no other workloads): for runs under a profiler")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library runs on one GPU and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_qk_rmsnorm_amd as A
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))
        return

    if not os.path.exists(A.library_path()):
        from attention_qk_rmsnorm_amd.build import build
        build()
    A.load_library()

    w = workloads.named_workloads()[args.workload]
    if args.dtype:
        w = dataclasses.replace(w, dtype=args.dtype)
    inp = workloads.make_inputs(w, seed=0)
    d_inp = {k: v.to(dev) for k, v in inp.items()}
    torch.cuda.synchronize()
    call = A.Call(d_inp["q"], d_inp["k"], d_inp["v"], d_inp["cu_seqlens"], d_inp["sinks"],
                  d_inp["qnorm_w"], d_inp["knorm_w"], w.window, w.use_rope,
                  rms_eps=w.rms_eps, rope_theta=w.rope_theta,
                  cu_seqlens_padded=d_inp.get("cu_seqlens_padded"),
                  tile_config=TILE_CHOICES[args.tile])
    if args.which == "bwd":
        run_bwd(args, A, w, d_inp, call, dev)
        return
    if w.pad_to:
        run_fwd_padded(args, A, w, inp, d_inp, dev)
        return
    stream = torch.cuda.current_stream(dev)
    tile = A.tile_config(call.desc, w.window)
    kernel, kernel_src = ATTN_KERNELS[tile]

    for _ in range(args.warmup):
        call.fwd()
    torch.cuda.synchronize()

    # timed region: K whole steps, each bracketed by events around the two
    # stages on the launch stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        call.prologue()
        ev[i][1].record(stream)
        call.attention()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms_step = elapsed * 1e3 / args.steps
    pro_l = [e[0].elapsed_time(e[1]) for e in ev]
    attn_l = [e[1].elapsed_time(e[2]) for e in ev]
    pro_ms = float(np.mean(pro_l))
    attn_ms = float(np.mean(attn_l))
    call_l = np.add(pro_l, attn_l)
    n_proto = protocol_calls(float(np.median(call_l)))
    if n_proto > args.steps and not args.quick:
        # more calls for the per-call statistics, after the timed region
        p2, a2 = time_forward_stages(call, stream, n_proto - args.steps)
        pro_l, attn_l = pro_l + p2, attn_l + a2
        call_l = np.add(pro_l, attn_l)
    n_vis = visible_entries(w.lengths, w.window)
    flop = 4.0 * w.head_dim * w.num_q_heads * n_vis
    value = flop / (ms_step * 1e-3) / 1e12
    achieved = flop / (attn_ms * 1e-3) / 1e12
    T = w.total_tokens
    pro_bytes = T * w.num_kv_heads * w.head_dim * 2 * 4      # read K, V; write k_hat, V^T

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.description}",
            "tokens": T, "docs": w.num_docs, "q_heads": w.num_q_heads,
            "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "window": w.window,
            "rope": w.use_rope, "visible_entries": n_vis, "flop_per_step": flop,
            "tile_config": TILE_NAMES[tile],
            "parallelism": "single GPU",
        },
        "pct_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "roofline": {
            "bound": "mfma",
            "kernel": kernel,
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": load_traffic(w.name if w.dtype == "bf16" else f"{w.name}/{w.dtype}",
                                    kernel, kernel_src),
            "avg_launch_ms": attn_ms,
        },
        "kernels": {
            "prologue_ms": pro_ms,
            "prologue_GBps": pro_bytes / (pro_ms * 1e-3) / 1e9,
            "prologue_frac_hbm": pro_bytes / (pro_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "attention_ms": attn_ms,
        },
        # per-call HIP-event times of the K timed steps (the protocol asks for
        # max(10, ceil(200 ms / t)) calls: protocol_calls)
        "timing": {
            "calls": len(call_l), "protocol_calls": n_proto,
            "call_ms": stats_ms(call_l), "prologue_ms": stats_ms(pro_l),
            "attention_ms": stats_ms(attn_l),
            "tflops_median": flop / (float(np.median(call_l)) * 1e-3) / 1e12,
            "tflops_min_time": flop / (float(np.min(call_l)) * 1e-3) / 1e12,
        },
        "library": library_record(A),
    }
    if args.cpu_seconds > 0:
        call.fwd()
        torch.cuda.synchronize()
        result["cpu_baseline"] = cpu_baseline(inp, w, call.out, call.lse, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    if (not args.no_others and not args.quick and args.workload == "full"
            and args.dtype in (None, "bf16") and args.tile == "auto"):
        del call, d_inp
        torch.cuda.empty_cache()
        result["workloads"] = other_workloads(A, dev, OTHER_WORKLOADS)
    print(json.dumps(result), flush=True)
    if not parity_ok(result["cpu_baseline"]):
        print("bench.py: the GPU result misses the bf16 bounds on the oracle's sample "
              f"({result['cpu_baseline']['parity_on_sample']})", file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
