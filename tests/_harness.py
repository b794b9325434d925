"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded bits, and compare element by element.

Tolerances: bf16 inputs and outputs with fp32 accumulation must agree with the
fp64 oracle within max-abs 2e-2 and mean-abs 2e-3 (out and lse); fp16 (unit
roundoff 2^-11 against bf16's 2^-8, so the operand errors shrink eightfold)
within max-abs 4e-3 and mean-abs 3e-4 -- the max keeps room for half an fp16
ulp of an output of magnitude 4 to 8 (1.95e-3) on top of the attention error;
the fp32 debug path within max-abs 1e-5."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

BF16_MAX, BF16_MEAN = 2e-2, 2e-3
FP16_MAX, FP16_MEAN = 4e-3, 3e-4
F32_MAX = 1e-5


def dtype_name(t) -> str:
    return {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[t]


def fwd_bounds(dtype):
    """(max-abs, mean-abs) bound on out and lse for a storage dtype."""
    return {torch.bfloat16: (BF16_MAX, BF16_MEAN), torch.float16: (FP16_MAX, FP16_MEAN),
            torch.float32: (F32_MAX, F32_MAX)}[dtype]


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    import attention_qk_rmsnorm_amd as A
    if not os.path.exists(A.library_path()):
        from attention_qk_rmsnorm_amd.build import build
        build()
    A.load_library()
    return A


def to_device(inp: dict, device="cuda:0") -> dict:
    return {k: v.to(device) for k, v in inp.items()}


def gpu_forward(inp_dev: dict, window: int, use_rope: bool, **kw):
    import attention_qk_rmsnorm_amd as A
    out, lse = A.sink_attn_fwd(inp_dev["q"], inp_dev["k"], inp_dev["v"], inp_dev["cu_seqlens"],
                               inp_dev["sinks"], inp_dev["qnorm_w"], inp_dev["knorm_w"],
                               window, use_rope, **kw)
    torch.cuda.synchronize()
    return out, lse


def oracle_forward(inp: dict, window: int, use_rope: bool, rows=None, eps=1e-6, theta=1e6,
                   scale=None):
    import oracle.oracle as O
    q = inp["q"].double().numpy()
    if rows is not None:
        q = q[rows]
    return O.sink_attn_fwd(q, inp["k"].double().numpy(), inp["v"].double().numpy(),
                           inp["cu_seqlens"].numpy(), inp["sinks"].double().numpy(),
                           inp["qnorm_w"].double().numpy(), inp["knorm_w"].double().numpy(),
                           window, use_rope, eps=eps, theta=theta, scale=scale, rows=rows)


def errors(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got.astype(np.float64) - ref)
    if d.size == 0:
        return 0.0, 0.0
    return float(d.max()), float(d.mean())


def check_parity(inp: dict, window: int, use_rope: bool, rows=None, label="", bound_scale=1.0,
                 **kw):
    """Run both sides and assert the tolerance for the input dtype (times
    bound_scale).  Returns the (out, lse) max/mean errors for reporting."""
    dev = to_device(inp)
    out, lse = gpu_forward(dev, window, use_rope, **kw)
    ref_out, ref_lse = oracle_forward(inp, window, use_rope, rows=rows,
                                      scale=kw.get("softmax_scale"),
                                      eps=kw.get("rms_eps", 1e-6),
                                      theta=kw.get("rope_theta", 1e6))
    out_np = out.float().cpu().numpy().astype(np.float64)
    lse_np = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        out_np = out_np[rows]
        lse_np = lse_np[:, rows]
    assert np.all(np.isfinite(out_np)), f"{label}: non-finite output"
    eo = errors(out_np, ref_out)
    el = errors(lse_np, ref_lse)
    print(f"  {label}: out max/mean {eo[0]:.3e}/{eo[1]:.3e} lse max/mean {el[0]:.3e}/{el[1]:.3e}",
          flush=True)
    bmax, bmean = fwd_bounds(inp["q"].dtype)
    bmax, bmean = bmax * bound_scale, bmean * bound_scale
    if inp["q"].dtype == torch.float32:
        assert eo[0] <= bmax and el[0] <= bmax, f"{label}: out {eo} lse {el}"
    else:
        assert eo[0] <= bmax and eo[1] <= bmean, f"{label}: out max/mean {eo}"
        assert el[0] <= bmax and el[1] <= bmean, f"{label}: lse max/mean {el}"
    return eo, el


def custom_inputs(lengths, Hq=32, Hkv=4, d=128, dtype="bf16", sink_mean=0.0, seed=0):
    w = workloads.custom_workload(lengths, Hq, Hkv, d, dtype, sink_mean=sink_mean)
    return workloads.make_inputs(w, seed=seed)


# ---- backward ----------------------------------------------------------------
# Gradient tensors scale with the number of terms they collect (a key early in
# a long causal document gathers P * dout from every later token and head), so
# the bf16 bound is taken relative to each reference tensor's largest entry:
# max |got - ref| <= BWD_REL_MAX * max|ref| and
# mean |got - ref| <= BWD_REL_MEAN * mean|ref|.  fp16: a fifth of that (the
# operand roundoff is an eighth; the mean keeps room for fp16's own output
# rounding, 2^-12 .. 2^-11 relative).
BWD_REL_MAX, BWD_REL_MEAN = 2e-2, 1e-2
BWD_REL_FP16 = (4e-3, 2e-3)
GRAD_KEYS = ("dq", "dk", "dv", "dsinks", "dqnorm_w", "dknorm_w")


def gpu_backward(inp_dev: dict, window: int, use_rope: bool, dout=None, seed=0,
                 return_forward=False, **kw):
    """Forward then backward through the C ABI; dout from the seeded generator
    unless given."""
    import attention_qk_rmsnorm_amd as A
    if dout is None:
        T, Hq, d = inp_dev["q"].shape
        w = workloads.Workload("g", (T,), Hq, inp_dev["k"].shape[1], d,
                               dtype_name(inp_dev["q"].dtype))
        dout = workloads.make_grad_output(w, seed).to(inp_dev["q"].device)
    # bwd_tile_config goes to the backward only (the forward keeps its own choice)
    bwd_tile = kw.pop("bwd_tile_config", None)
    fkw = {k: v for k, v in kw.items() if k in ("rms_eps", "rope_theta", "softmax_scale")}
    if bwd_tile is not None:
        fkw["tile_config"] = bwd_tile
    out, lse = A.sink_attn_fwd(inp_dev["q"], inp_dev["k"], inp_dev["v"], inp_dev["cu_seqlens"],
                               inp_dev["sinks"], inp_dev["qnorm_w"], inp_dev["knorm_w"],
                               window, use_rope, **kw)
    g = A.sink_attn_bwd(inp_dev["q"], inp_dev["k"], inp_dev["v"], inp_dev["cu_seqlens"],
                        inp_dev["sinks"], inp_dev["qnorm_w"], inp_dev["knorm_w"], window,
                        use_rope, out, lse, dout, **fkw)
    torch.cuda.synchronize()
    if return_forward:
        return g, out, dout
    return g


def oracle_backward(inp: dict, window: int, use_rope: bool, dout, eps=1e-6, theta=1e6,
                    scale=None):
    import oracle.oracle as O
    f = lambda t: t.double().numpy()  # noqa: E731
    return O.sink_attn_bwd(f(inp["q"]), f(inp["k"]), f(inp["v"]), inp["cu_seqlens"].numpy(),
                           f(inp["sinks"]), f(inp["qnorm_w"]), f(inp["knorm_w"]), window,
                           use_rope, f(dout), eps=eps, theta=theta, scale=scale)


def check_bwd_parity(inp: dict, window: int, use_rope: bool, label="", seed=0, **kw):
    """Backward on the GPU and in the oracle on the same bits; assert the
    relative bound on every gradient tensor.  Returns the GPU gradients."""
    T, Hq, d = inp["q"].shape
    w = workloads.Workload("g", (T,), Hq, inp["k"].shape[1], d, dtype_name(inp["q"].dtype))
    dout = workloads.make_grad_output(w, seed)
    rel_max_bound, rel_mean_bound = (BWD_REL_FP16 if inp["q"].dtype == torch.float16
                                     else (BWD_REL_MAX, BWD_REL_MEAN))
    dev = to_device(inp)
    g = gpu_backward(dev, window, use_rope, dout=dout.to("cuda:0"), **kw)
    ref = oracle_backward(inp, window, use_rope, dout, eps=kw.get("rms_eps", 1e-6),
                          theta=kw.get("rope_theta", 1e6), scale=kw.get("softmax_scale"))
    msg = []
    bad = []
    for key in GRAD_KEYS:
        got = g[key].float().cpu().numpy().astype(np.float64)
        r = ref[key]
        assert np.all(np.isfinite(got)), f"{label}: non-finite {key}"
        if r.size == 0:
            continue
        emax, emean = errors(got, r)
        smax = float(np.abs(r).max())
        smean = float(np.abs(r).mean())
        rel_max = emax / smax if smax > 0 else emax
        rel_mean = emean / smean if smean > 0 else emean
        msg.append(f"{key} {rel_max:.2e}/{rel_mean:.2e}")
        if rel_max > rel_max_bound or rel_mean > rel_mean_bound:
            bad.append(f"{key}: max {emax:.3e} (scale {smax:.3e}) mean {emean:.3e} "
                       f"(scale {smean:.3e})")
    print(f"  {label}: rel max/mean " + ", ".join(msg), flush=True)
    assert not bad, f"{label}: " + "; ".join(bad)
    return g


# ---- the wide tiles' redo table ----------------------------------------------
# The forward workspace (16-bit paths) holds, in order and each 256-byte
# aligned: the k_hat and V^T tile images (Hkv * t_pad * 128 elements each,
# t_pad = T rounded up to 64), the narrow and the wide schedules (int32:
# 4 + 2 * items_ub + D + 1 each, items_ub = T / tokens_per_block + D with
# 128 / G and 256 / G tokens per block), then one int32 per wide workgroup:
# 1 if the main launch handed the block to the exact-max launch.  A test that
# reads it also checks the offset (every block marked when all are forced
# through the exact pass, none on moderate inputs).

def _round_up(x, m):
    return (x + m - 1) // m * m


def redo_table(call):
    """(marked, blocks): the redo flags the last wide-tile forward of `call`
    left in its workspace, and the number of workgroups that hold an item."""
    d = call.desc
    T, D, Hq, Hkv = d.total_tokens, d.num_docs, d.num_q_heads, d.num_kv_heads
    G = Hq // Hkv
    t_pad = _round_up(T, 64)
    items_ub = T // (128 // G) + D
    items_ub_wide = T // (256 // G) + D
    off = _round_up(Hkv * t_pad * 128 * 2, 256)
    off = _round_up(off + Hkv * t_pad * 128 * 2, 256)
    off = _round_up(off + 4 * (4 + 2 * items_ub + D + 1), 256)
    sched_wide_off = off
    off = _round_up(off + 4 * (4 + 2 * items_ub_wide + D + 1), 256)
    if Hkv <= 8 and 8 % Hkv == 0:
        per = 8 // Hkv
        grid = 8 * ((items_ub_wide + per - 1) // per)
    else:
        grid = items_ub_wide * Hkv
    ws = call.workspace
    redo = ws[off:off + 4 * grid].view(torch.int32).cpu().numpy()
    n_items = int(ws[sched_wide_off:sched_wide_off + 4].view(torch.int32).item())
    return redo, n_items * Hkv
