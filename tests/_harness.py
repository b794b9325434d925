"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded bits, and compare element by element.

Tolerances: bf16 inputs and outputs with fp32 accumulation must agree with the
fp64 oracle within max-abs 2e-2 and mean-abs 2e-3 (out and lse); the fp32
debug path within max-abs 1e-5."""
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
F32_MAX = 1e-5


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


def check_parity(inp: dict, window: int, use_rope: bool, rows=None, label="", **kw):
    """Run both sides and assert the tolerance for the input dtype.  Returns the
    (out, lse) max/mean errors for reporting."""
    dev = to_device(inp)
    out, lse = gpu_forward(dev, window, use_rope, **kw)
    ref_out, ref_lse = oracle_forward(inp, window, use_rope, rows=rows,
                                      scale=kw.get("softmax_scale"))
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
    if inp["q"].dtype == torch.float32:
        assert eo[0] <= F32_MAX and el[0] <= F32_MAX, f"{label}: out {eo} lse {el}"
    else:
        assert eo[0] <= BF16_MAX and eo[1] <= BF16_MEAN, f"{label}: out max/mean {eo}"
        assert el[0] <= BF16_MAX and el[1] <= BF16_MEAN, f"{label}: lse max/mean {el}"
    return eo, el


def custom_inputs(lengths, Hq=32, Hkv=4, d=128, dtype="bf16", sink_mean=0.0, seed=0):
    w = workloads.custom_workload(lengths, Hq, Hkv, d, dtype, sink_mean=sink_mean)
    return workloads.make_inputs(w, seed=seed)
