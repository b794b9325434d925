"""The backward at the sizes the backward bench times, checked against the fp64
oracle on every output element.

Workloads: every named one -- full (one causal document of 32,768 tokens, no
RoPE), long (two documents of 65,536 tokens, window 4,096, NeoX RoPE, sinks
N(2, 1)), sliding (8 documents of U[256, 4096] tokens, window 1,024, RoPE) and
the two mixed ones (512 documents of geometric lengths with mean 200, causal
without RoPE, or window 512 with RoPE) -- 32 query / 4 kv heads, d = 128,
bf16 (full and mixed causal also with fp16 storage, at the fp16 bounds),
through sink_attn_bwd with its automatic kernel choices (the launch
configuration the bench times).

dout is zero except on a seeded sample of query tokens, every head of each:
each document's first and last 64 tokens (8 for the mixed workloads' short
documents), the tokens around the window edge, and 128 random ones
(workloads.sample_rows).  A row whose dout is zero adds
exactly nothing to any gradient (its D = dout . out is 0, so dS = P (dP - D)
is 0 for every key it sees, and its dv terms are P * 0), so every gradient is
a sum over the sampled rows alone.  The oracle skips the zero rows, which
makes the whole backward of these sizes a matter of seconds, and every
element of dk, dv, dsinks and both norm-weight gradients -- each key of the
document gets terms from the last sampled rows -- and of dq on the sampled
rows is compared with it; dq of every other row must be exactly zero.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from _harness import (BWD_REL_FP16, BWD_REL_MAX, BWD_REL_MEAN, GRAD_KEYS, errors,
                      gpu_backward, oracle_backward, require_gpu, to_device)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


# (workload, rows sampled at each document end, storage type): the mixed
# workloads' 512 short documents take 8 rows at each end (64 would be half
# their tokens); two of the workloads again with fp16 storage
@pytest.mark.parametrize("name,edge,dtype", [
    ("full", 64, "bf16"), ("long", 64, "bf16"), ("sliding", 64, "bf16"),
    ("mixed_causal", 8, "bf16"), ("mixed_sliding", 8, "bf16"),
    ("full", 64, "f16"), ("mixed_causal", 8, "f16")])
def test_full_size_backward_on_sampled_rows(name, edge, dtype):
    require_gpu()
    w = dataclasses.replace(workloads.named_workloads()[name], dtype=dtype)
    _say(f"case bwd {name} {dtype} T={w.total_tokens} sampled dout rows")
    inp = workloads.make_inputs(w, seed=0)
    rows = workloads.sample_rows(w.lengths, w.window, 128, seed=5, edge=edge)
    live = torch.zeros(w.total_tokens, dtype=torch.bool)
    live[torch.from_numpy(rows).long()] = True
    dout = workloads.make_grad_output(w, seed=0)
    dout[~live] = 0
    g = gpu_backward(to_device(inp), w.window, w.use_rope, dout=dout.to("cuda:0"),
                     rms_eps=w.rms_eps, rope_theta=w.rope_theta)
    ref = oracle_backward(inp, w.window, w.use_rope, dout, eps=w.rms_eps, theta=w.rope_theta)
    dq = g["dq"].float().cpu()
    assert bool((dq[~live] == 0).all()), "dq of a row with zero dout is not zero"
    rel_max, rel_mean = (BWD_REL_FP16 if dtype == "f16" else (BWD_REL_MAX, BWD_REL_MEAN))
    msg, bad = [], []
    for key in GRAD_KEYS:
        got = g[key].float().cpu().numpy().astype(np.float64)
        r = ref[key]
        if key == "dq":
            got, r = got[rows], r[rows]
        assert np.all(np.isfinite(got)), f"{name}: non-finite {key}"
        emax, emean = errors(got, r)
        smax, smean = float(np.abs(r).max()), float(np.abs(r).mean())
        msg.append(f"{key} {emax / smax:.2e}/{emean / smean:.2e}")
        if emax > rel_max * smax or emean > rel_mean * smean:
            bad.append(f"{key}: max {emax:.3e} (scale {smax:.3e}) mean {emean:.3e} "
                       f"(scale {smean:.3e})")
    _say(f"  {name} {dtype} bwd, {len(rows)} sampled tokens: rel max/mean " + ", ".join(msg))
    assert not bad, f"{name}: " + "; ".join(bad)
