"""GPU parity of the bf16 tile configurations, forced through the descriptor's
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
@pytest.mark.parametrize("window,use_rope", [(-1, False), (1, True), (2, False), (65, False),
                                             (100, True), (512, True)])
def test_ragged_documents(tile, window, use_rope):
    _say(f"case tile={tile} ragged W={window} rope={use_rope}")
    check_parity(custom_inputs(RAGGED), window, use_rope, label=f"tile{tile} W={window}",
                 tile_config=tile)


@pytest.mark.parametrize("tile", [WIDE, WIDE_EXACT])
@pytest.mark.parametrize("heads", [(32, 4), (8, 8), (32, 1), (4, 2), (16, 1), (2, 2)])
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


def _trigger_inputs(lengths, starts, w0, use_rope):
    """Moderate random inputs in which the second token of each document in
    `starts` takes the wide tiles' natural exact-max rerun.

    Token a (a document's first) has the key c*e0; token a + 1 has the query
    c*e0 in every head and the key -c*e0.  With norm weight w0 on channel 0,
    query a + 1 scores +w0^2 sqrt(128) against key a (times cos(1) under
    RoPE, which turns channel 0 into channel 64 by one radian per position)
    and -w0^2 sqrt(128) against its own key: 70.7 nats above its own score
    at w0 = 2.5 (75 nats at w0 = 3.5 with RoPE), more than the 90 log2 units
    (62 nats) the fixed reference max(sink, own score) allows, so its block
    marks itself for the rerun.  Every other token has channels 0 and 64 of
    its query and key zeroed: its scores against the two trigger keys are 0
    exactly and all its other scores are the usual moderate ones, so the
    rest of each rerun block is an ordinary row recomputed by the exact pass.
    Returns the inputs and the trigger rows."""
    inp = custom_inputs(lengths)
    q, k = inp["q"].clone(), inp["k"].clone()
    q[:, :, 0] = 0
    q[:, :, 64] = 0
    k[:, :, 0] = 0
    k[:, :, 64] = 0
    c = 4.0
    trig = []
    for a in starts:
        k[a] = 0
        k[a, :, 0] = c
        q[a + 1] = 0
        q[a + 1, :, 0] = c
        k[a + 1] = 0
        k[a + 1, :, 0] = -c
        trig.append(a + 1)
    qw, kw = inp["qnorm_w"].clone(), inp["knorm_w"].clone()
    qw[0] = w0
    kw[0] = w0
    return dict(inp, q=q, k=k, qnorm_w=qw, knorm_w=kw), trig


@pytest.mark.parametrize("window,use_rope", [(-1, False), (513, False), (300, True)])
def test_natural_rerun_against_oracle(window, use_rope):
    import attention_qk_rmsnorm_amd as A
    import numpy as np
    from _harness import errors, oracle_forward, redo_table
    lengths = [40, 300, 2, 130, 700]
    cu = np.cumsum([0] + lengths)
    w0 = 3.5 if use_rope else 2.5
    inp, trig = _trigger_inputs(lengths, [int(cu[1]), int(cu[3])], w0, use_rope)
    _say(f"case bf16 natural rerun W={window} rope={use_rope} triggers {trig}")
    dev = to_device(inp)
    c = A.Call(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], dev["sinks"], dev["qnorm_w"],
               dev["knorm_w"], window, use_rope, tile_config=WIDE)
    # the redo table's offset: the all-exact configuration marks every block
    c_all = A.Call(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], dev["sinks"],
                   dev["qnorm_w"], dev["knorm_w"], window, use_rope, tile_config=WIDE_EXACT)
    c_all.fwd()
    torch.cuda.synchronize()
    redo_all, blocks = redo_table(c_all)
    assert blocks > 0 and bool((redo_all == 1).all())
    c.fwd()
    torch.cuda.synchronize()
    redo, blocks = redo_table(c)
    marked = int(redo.sum())
    _say(f"  {marked} of {blocks} wide blocks took the exact-max rerun")
    # one block per trigger token and kv head, and no other
    assert marked == len(trig) * 4, redo
    ref_out, ref_lse = oracle_forward(inp, window, use_rope)
    out = c.out.float().cpu().numpy()
    lse = c.lse.cpu().numpy()
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    eo = errors(out, ref_out)
    _say(f"  out max/mean {eo[0]:.3e}/{eo[1]:.3e}")
    assert eo[0] <= BF16_MAX and eo[1] <= BF16_MEAN
    normal = np.setdiff1d(np.arange(sum(lengths)), trig)
    el = errors(lse[:, normal], ref_lse[:, normal])
    _say(f"  lse (ordinary rows) max/mean {el[0]:.3e}/{el[1]:.3e}")
    assert el[0] <= BF16_MAX and el[1] <= BF16_MEAN
    # a trigger row's lse is its dominant score (~70 nats), which carries the
    # bf16 rounding of its two operands: at most 2 * 2^-9 relative
    for t in trig:
        bound = BF16_MAX + 2.0 ** -8 * np.abs(ref_lse[:, t])
        dl = np.abs(lse[:, t] - ref_lse[:, t])
        _say(f"  trigger row {t}: lse {ref_lse[:, t].min():.1f}..{ref_lse[:, t].max():.1f}, "
             f"error max {dl.max():.3e}")
        assert np.all(dl <= bound)
    # the narrow tiles (running max) and the all-exact wide tiles
    for t in (NARROW, WIDE_EXACT):
        o, l = gpu_forward(dev, window, use_rope, tile_config=t)
        e2 = errors(o.float().cpu().numpy(), ref_out)
        assert e2[0] <= BF16_MAX and e2[1] <= BF16_MEAN, (t, e2)


def test_wide_deterministic_and_fully_written():
    # NaN guard bands around out and lse: the wide tiles write every row of
    # out and lse -- blocks that take the rerun included -- and nothing
    # outside them; repeated calls are bitwise equal
    _say("case wide determinism + poison")
    inp, _ = _trigger_inputs([333, 1, 90], [334], 2.5, False)
    dev = to_device(inp)
    T, row = 424, 32 * 128
    nan = float("nan")
    for tile in (WIDE, WIDE_EXACT):
        base = torch.full(((T + 64) * row,), nan, dtype=torch.bfloat16, device="cuda")
        out = base[32 * row:(32 + T) * row].view(T, 32, 128)
        flat = torch.full((32 * T + 128,), nan, dtype=torch.float32, device="cuda")
        lse = flat[64:64 + 32 * T].view(32, T)
        o1, l1 = gpu_forward(dev, 64, False, out=out, lse=lse, tile_config=tile)
        assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
        assert torch.isnan(base[:32 * row].float()).all()
        assert torch.isnan(base[(32 + T) * row:].float()).all()
        assert torch.isnan(flat[:64]).all() and torch.isnan(flat[64 + 32 * T:]).all()
        o2, l2 = gpu_forward(dev, 64, False, tile_config=tile)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_huge_values_take_the_rerun():
    # A trigger pair (see _trigger_inputs) alone in a 2-token document, with
    # norm weight 2 on channel 0: the second token's weight for the first key
    # is about 2^65 against the fixed reference max(sink, own score), below
    # the 2^90 denominator bound, and that key's value is scaled by 2^70, so
    # the fp32 O accumulator overflows (2^135) while the denominator is in
    # range.  The main launch must hand that block to the exact-max launch
    # (weights at most 1) instead of writing inf or NaN.  The document's rows
    # are compared with the oracle after dividing by 2^70 (exact for a power
    # of two), at the usual bounds; the trigger row's lse (its ~45-nat
    # dominant score) at the usual bound plus 2^-8 of its size, as in
    # test_natural_rerun_against_oracle.
    import attention_qk_rmsnorm_amd as A
    import numpy as np
    from _harness import errors, oracle_forward, redo_table
    _say("case huge value behind a large weight")
    lengths = [40, 300, 2, 130]
    j = 340
    inp, trig = _trigger_inputs(lengths, [j], 2.0, False)
    big = 2.0 ** 70
    v = inp["v"].clone()
    v[j] = (v[j].float() * big).to(torch.bfloat16)
    inp = dict(inp, v=v)
    dev = to_device(inp)
    ref_out, ref_lse = oracle_forward(inp, -1, False)
    c = A.Call(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], dev["sinks"], dev["qnorm_w"],
               dev["knorm_w"], -1, False, tile_config=WIDE)
    c.fwd()
    torch.cuda.synchronize()
    redo, blocks = redo_table(c)
    _say(f"  {int(redo.sum())} of {blocks} wide blocks took the exact-max rerun")
    assert int(redo.sum()) == 4          # the 2-token document, once per kv head
    doc = np.array([j, j + 1])
    rest = np.setdiff1d(np.arange(sum(lengths)), doc)
    outs = {WIDE: (c.out, c.lse)}
    outs.update({t: gpu_forward(dev, -1, False, tile_config=t) for t in (NARROW, WIDE_EXACT)})
    for t, (o, l) in outs.items():
        o = o.float().cpu().numpy().astype(np.float64)
        l = l.cpu().numpy()
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), t
        e_doc = errors(o[doc] / big, ref_out[doc] / big)
        e_rest = errors(o[rest], ref_out[rest])
        el = errors(l[:, rest], ref_lse[:, rest])
        dl = np.abs(l[:, trig[0]] - ref_lse[:, trig[0]])
        _say(f"  tile {t}: document rows out/2^70 max/mean {e_doc[0]:.3e}/{e_doc[1]:.3e}, "
             f"others {e_rest[0]:.3e}/{e_rest[1]:.3e}, trigger lse error {dl.max():.3e}")
        assert e_doc[0] <= BF16_MAX and e_doc[1] <= BF16_MEAN, (t, e_doc)
        assert e_rest[0] <= BF16_MAX and e_rest[1] <= BF16_MEAN, (t, e_rest)
        assert el[0] <= BF16_MAX and el[1] <= BF16_MEAN, (t, el)
        assert abs(l[0, j] - ref_lse[0, j]) <= BF16_MAX
        assert np.all(dl <= BF16_MAX + 2.0 ** -8 * np.abs(ref_lse[:, trig[0]]))
