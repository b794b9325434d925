"""GPU parity of both bf16 tile configurations, forced through the descriptor's
tile_config (the automatic choice sends the small cases of the other GPU tests
to the narrow tiles and the long workloads to the wide ones):

* narrow (1), wide (2) and wide with the exact-max pass for every block (3)
  against the fp64 oracle on ragged documents, windows, RoPE, group sizes,
  sinks and multi-tile documents;
* inputs whose scores span far more than the 90 log2 units the wide tiles'
  fixed reference allows, so some blocks rerun with the exact row max: the
  three configurations must agree (the logits are too large for the fp64
  oracle to be a fair bf16 target, but the configurations share the bf16
  operands and differ only in how the softmax reference is chosen)."""
import pytest
import torch

from _harness import BF16_MAX, BF16_MEAN, check_parity, custom_inputs, gpu_forward, \
    require_gpu, to_device

pytestmark = pytest.mark.gpu

NARROW, WIDE, WIDE_EXACT = 1, 2, 3
RAGGED = [1, 2, 3, 17, 63, 64, 65, 127, 128, 129, 200, 0, 31, 300]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    return require_gpu()


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("tile", [WIDE, WIDE_EXACT])
@pytest.mark.parametrize("window,use_rope", [(-1, False), (1, True), (65, False), (100, True),
                                             (512, True)])
def test_ragged_documents(tile, window, use_rope):
    _say(f"case tile={tile} ragged W={window} rope={use_rope}")
    check_parity(custom_inputs(RAGGED), window, use_rope, label=f"tile{tile} W={window}",
                 tile_config=tile)


@pytest.mark.parametrize("tile", [WIDE, WIDE_EXACT])
@pytest.mark.parametrize("heads", [(32, 4), (8, 8), (32, 1), (4, 2)])
def test_group_sizes(tile, heads):
    _say(f"case tile={tile} heads={heads}")
    inp = custom_inputs([150, 33, 290], Hq=heads[0], Hkv=heads[1])
    check_parity(inp, 100, True, label=f"tile{tile} {heads}", tile_config=tile)
    check_parity(inp, -1, False, label=f"tile{tile} {heads}", tile_config=tile)


@pytest.mark.parametrize("tile", [NARROW, WIDE])
def test_long_document(tile):
    _say(f"case tile={tile} one doc 2500")
    inp = custom_inputs([2500])
    check_parity(inp, -1, False, label=f"tile{tile} causal", tile_config=tile)
    check_parity(inp, 700, True, label=f"tile{tile} W=700", tile_config=tile)


@pytest.mark.parametrize("tile", [WIDE, WIDE_EXACT])
def test_sinks(tile):
    inp = custom_inputs([70, 130])
    _say(f"case tile={tile} sinks")
    check_parity(dict(inp, sinks=torch.full((32,), float("-inf"))), 40, True,
                 label="-inf", tile_config=tile)
    check_parity(custom_inputs([70, 130], sink_mean=2.0), -1, False, label="N(2,1)",
                 tile_config=tile)
    check_parity(dict(inp, sinks=torch.full((32,), 8.0)), -1, False, label="8",
                 tile_config=tile)
    big = dict(inp, sinks=torch.full((32,), 60.0))
    dev = to_device(big)
    out, lse = gpu_forward(dev, -1, False, tile_config=tile)
    assert out.float().abs().max().item() < 1e-6
    assert torch.allclose(lse, torch.full_like(lse, 60.0), atol=1e-3)


def test_stages_and_determinism_wide():
    _say("case wide stages + determinism")
    import attention_qk_rmsnorm_amd as A
    inp = to_device(custom_inputs([333, 1, 900]))
    ref = gpu_forward(inp, 64, True, tile_config=WIDE)
    again = gpu_forward(inp, 64, True, tile_config=WIDE)
    assert torch.equal(ref[0], again[0]) and torch.equal(ref[1], again[1])
    c = A.sink_attn_prologue(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], inp["sinks"],
                             inp["qnorm_w"], inp["knorm_w"], 64, True, tile_config=WIDE)
    c.attention()
    torch.cuda.synchronize()
    assert torch.equal(c.out, ref[0]) and torch.equal(c.lse, ref[1])


@pytest.mark.parametrize("window", [-1, 300])
def test_scores_far_above_the_fixed_reference(window):
    # norm weights of 2.5 stretch the scores to about +-70 nats (+-100 log2
    # units): many tokens' own score sits more than 90 log2 units below their
    # row max, so the wide tiles' main launch hands those blocks to the
    # exact-max launch
    _say(f"case large scores W={window}")
    inp = custom_inputs([700, 1400])
    inp = dict(inp, qnorm_w=torch.full((128,), 2.5), knorm_w=torch.full((128,), 2.5),
               sinks=torch.full((32,), float("-inf")))
    dev = to_device(inp)
    outs = {t: gpu_forward(dev, window, False, tile_config=t) for t in (NARROW, WIDE, WIDE_EXACT)}
    for t in (WIDE, WIDE_EXACT):
        o, l = outs[t]
        assert torch.isfinite(o.float()).all() and torch.isfinite(l).all()
        d = (o.float() - outs[NARROW][0].float()).abs()
        dl = (l - outs[NARROW][1]).abs()
        _say(f"  tile {t} vs narrow: out max/mean {d.max().item():.3e}/{d.mean().item():.3e} "
             f"lse max {dl.max().item():.3e}")
        assert d.max().item() <= BF16_MAX and d.mean().item() <= BF16_MEAN
        assert dl.max().item() <= 1e-3 * max(1.0, outs[NARROW][1].abs().max().item())
