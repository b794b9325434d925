"""GPU parity of the fp16 I/O variant (flint.config attention_compute_dtype =
'fp16': q, k, v and out, and in the backward dout and the input gradients,
stored in fp16) against the fp64 oracle on the same fp16 bits.

The kernels are the bf16 ones instantiated with fp16 MFMA operands, so the
cases mirror the bf16 tests: ragged documents, windows, RoPE, group sizes,
sinks, both tile configurations, long documents, the backward, and the
full-size causal workload on sampled rows.  fp16's narrow range adds one
case: weights against the wide tiles' fixed reference overflow fp16 once a
score is 16 log2 units above it (bf16 allows 90), which sends the block to
the exact-max rerun; it must agree with the narrow tiles."""
import numpy as np
import pytest
import torch

import workloads
from _harness import (FP16_MAX, FP16_MEAN, check_bwd_parity, check_parity, custom_inputs,
                      gpu_forward, require_gpu, to_device)

pytestmark = pytest.mark.gpu

NARROW, WIDE, WIDE_EXACT = 1, 2, 3
RAGGED = [1, 2, 3, 17, 63, 64, 65, 127, 128, 129, 200, 0, 31, 300]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    return require_gpu()


def _say(msg):
    print(msg, flush=True)


def _f16(lengths, **kw):
    return custom_inputs(lengths, dtype="f16", **kw)


@pytest.mark.parametrize("tile", [NARROW, WIDE, WIDE_EXACT])
@pytest.mark.parametrize("window,use_rope", [(-1, False), (1, True), (65, False), (512, True)])
def test_forward_ragged(tile, window, use_rope):
    _say(f"case fp16 fwd tile={tile} W={window} rope={use_rope}")
    check_parity(_f16(RAGGED), window, use_rope, label=f"fp16 tile{tile} W={window}",
                 tile_config=tile)


@pytest.mark.parametrize("heads", [(32, 4), (8, 8), (32, 1), (16, 16)])
def test_forward_group_sizes(heads):
    _say(f"case fp16 fwd heads={heads}")
    inp = _f16([150, 33, 290], Hq=heads[0], Hkv=heads[1])
    for tile in (NARROW, WIDE):
        check_parity(inp, 100, True, label=f"fp16 {heads} tile{tile}", tile_config=tile)
        check_parity(inp, -1, False, label=f"fp16 {heads} tile{tile}", tile_config=tile)


def test_forward_long_document_and_sinks():
    _say("case fp16 fwd one doc 2500, sinks")
    inp = _f16([2500])
    for tile in (NARROW, WIDE):
        check_parity(inp, -1, False, label=f"fp16 causal tile{tile}", tile_config=tile)
        check_parity(inp, 700, True, label=f"fp16 W=700 tile{tile}", tile_config=tile)
    small = _f16([70, 130])
    check_parity(dict(small, sinks=torch.full((32,), float("-inf"))), 40, True, label="-inf")
    check_parity(_f16([70, 130], sink_mean=2.0), -1, False, label="N(2,1)")
    big = to_device(dict(small, sinks=torch.full((32,), 60.0)))
    for tile in (NARROW, WIDE):
        out, lse = gpu_forward(big, -1, False, tile_config=tile)
        assert out.float().abs().max().item() < 1e-6
        assert torch.allclose(lse, torch.full_like(lse, 60.0), atol=1e-3)


@pytest.mark.parametrize("weight", [1.6, 1.35])
@pytest.mark.parametrize("window", [-1, 300])
def test_weights_past_fp16_range_take_the_rerun(window, weight):
    # norm weights of w give scores a standard deviation of about w^2 nats: a
    # row's peak over hundreds of keys sits ~3 standard deviations above the
    # mean, and where the token's own score is low that peak is more than 16
    # log2 units (11 nats) above it -- past what an fp16 weight can hold -- so
    # the wide main launch hands that row's block to the exact-max launch (the
    # redo table read back from the workspace shows which).  At w = 1.6 every
    # block of these inputs has such a row; at w = 1.35 about a third do
    # (counted on the CPU from the same inputs), so marked and unmarked blocks
    # run side by side.  The result must match the fp64 oracle, the narrow
    # tiles (running max) and the all-exact configuration.  Bound against the
    # oracle: the operand roundings move each score by an amount proportional
    # to |q_hat| |k_hat|, which the weights raise w^2-fold over the
    # unit-weight inputs the fp16 bounds are set for, so both fp16 bounds are
    # scaled by w^2.
    import attention_qk_rmsnorm_amd as A
    from _harness import errors, oracle_forward, redo_table
    _say(f"case fp16 large scores W={window} weight={weight}")
    inp = _f16([700, 1400])
    inp = dict(inp, qnorm_w=torch.full((128,), weight), knorm_w=torch.full((128,), weight),
               sinks=torch.full((32,), float("-inf")))
    dev = to_device(inp)
    c = A.Call(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], dev["sinks"], dev["qnorm_w"],
               dev["knorm_w"], window, False, tile_config=WIDE)
    c.fwd()
    torch.cuda.synchronize()
    redo, blocks = redo_table(c)
    marked = int(redo.sum())
    _say(f"  {marked} of {blocks} wide blocks took the exact-max rerun")
    assert marked > 0 and (weight > 1.5 or marked < blocks)
    outs = {t: gpu_forward(dev, window, False, tile_config=t) for t in (NARROW, WIDE_EXACT)}
    outs[WIDE] = (c.out, c.lse)
    ref_out, ref_lse = oracle_forward(inp, window, False)
    bmax, bmean = weight ** 2 * FP16_MAX, weight ** 2 * FP16_MEAN
    for t in (NARROW, WIDE, WIDE_EXACT):
        o, l = outs[t]
        assert torch.isfinite(o.float()).all() and torch.isfinite(l).all()
        eo = errors(o.float().cpu().numpy(), ref_out)
        el = errors(l.cpu().numpy(), ref_lse)
        _say(f"  tile {t} vs oracle: out max/mean {eo[0]:.3e}/{eo[1]:.3e} "
             f"lse max/mean {el[0]:.3e}/{el[1]:.3e}")
        assert eo[0] <= bmax and eo[1] <= bmean, (t, eo)
        assert el[0] <= bmax and el[1] <= bmean, (t, el)
    for t in (WIDE, WIDE_EXACT):
        o, l = outs[t]
        d = (o.float() - outs[NARROW][0].float()).abs()
        assert d.max().item() <= FP16_MAX and d.mean().item() <= FP16_MEAN


@pytest.mark.parametrize("window,use_rope", [(-1, False), (1, True), (100, True), (512, True)])
def test_backward_ragged(window, use_rope):
    _say(f"case fp16 bwd ragged W={window} rope={use_rope}")
    check_bwd_parity(_f16(RAGGED), window, use_rope, label=f"fp16 W={window}")


@pytest.mark.parametrize("heads", [(32, 4), (8, 8), (32, 1)])
def test_backward_group_sizes(heads):
    _say(f"case fp16 bwd heads={heads}")
    inp = _f16([150, 33, 290], Hq=heads[0], Hkv=heads[1])
    check_bwd_parity(inp, 100, True, label=f"fp16 {heads} W=100")
    check_bwd_parity(inp, -1, False, label=f"fp16 {heads} causal")


def test_backward_long_document():
    _say("case fp16 bwd one doc 1500")
    inp = _f16([1500])
    check_bwd_parity(inp, -1, False, label="fp16 causal 1500")
    check_bwd_parity(inp, 700, True, label="fp16 W=700 1500")


def test_full_workload_sampled_rows():
    # the full-causal layer (one document of 32768 tokens) in fp16, in the
    # launch configuration the benchmark times (automatic tile choice)
    w = workloads.named_workloads()["full"]
    w = workloads.Workload(w.name, w.lengths, w.num_q_heads, w.num_kv_heads, w.head_dim, "f16",
                           w.window, w.use_rope, w.sink_mean)
    _say(f"case fp16 full T={w.total_tokens}")
    inp = workloads.make_inputs(w)
    rows = workloads.sample_rows(w.lengths, w.window, 192)
    eo, el = check_parity(inp, w.window, w.use_rope, rows=rows, label="fp16 full")
    assert np.isfinite(eo[0])
