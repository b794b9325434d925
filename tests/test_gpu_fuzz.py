"""Seeded fuzz tier: random varlen batches against the fp64 oracle.

Every case is drawn from its seed alone (numpy's PCG64), so a failure names a
case that reruns exactly.  Document lengths come mostly from the tile-boundary
classes of the kernels -- one below, at and one above a multiple of 16, 32, 64
(the key tile), 128 and 256, plus 0, 1, 2 -- with some uniform draws between
them; the window from {1, 2, 63, 64, 65, 512, 513, 1024, causal} (513 is
flint.config FlintConfig's default sliding window); RoPE on or off; the
sinks centred on 0 or 2; a GQA shape; and the tile configuration (automatic,
narrow or wide).  The forward is compared on every row, the backward on every
gradient element, each within the bounds of the fixed-case tests.  The same
draws, at fp16, run the fp16 I/O variant; with random padding after each
document (NaN stored in the padding rows) they run the padded-THD entry
points, whose padding rows must come back exactly (out 0, lse the sink, zero
gradients).

Bound of the bf16 forward cases.  The bf16 MFMA takes q_hat * scale * log2(e)
and k_hat rounded to bf16, and on a row with only two visible keys (W = 2)
that rounding alone moves the difference of the two scores by up to ~1e-2
nats, and out by that times w1 w2 |v1 - v2| -- up to about 1.3e-2 with |v|
near 5.  The bf16 weights add up to 2^-8 relative each (just above a power of
two), and the output rounding half an ulp, so a correct bf16 result can
exceed the 2e-2 max-abs target on such rows.  Each element must therefore be
within 2e-2 of the fp64 oracle plus the distance by which the oracle itself
moves when evaluated on those rounded operands (the oracle's normalisation
and attention functions on the rounded values); the mean-abs target 2e-3
holds unchanged.  With many visible keys the allowance is a few 1e-4."""
import os

import numpy as np
import pytest
import torch

import workloads
from _harness import (BF16_MAX, BF16_MEAN, check_bwd_parity, check_parity, custom_inputs,
                      errors, gpu_forward, oracle_forward, require_gpu, to_device)

BOUNDARY_LENGTHS = [0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129,
                    255, 256, 257, 511, 512, 513]
WINDOWS = [1, 2, 63, 64, 65, 512, 513, 1024, -1]
HEADS = [(32, 4), (32, 4), (32, 4), (16, 2), (8, 8), (32, 1), (4, 2), (16, 4), (16, 1)]
TILES = [0, 1, 2]  # automatic, narrow, wide
N_FWD, N_BWD = 96, 24  # cases per run (seeds OFFSET .. OFFSET + N - 1)
N_FP16, N_PADDED = 16, 16
# SINKATTN_FUZZ_OFFSET=k000 runs another set of draws (each test adds its own
# base to the seed, so offsets that are multiples of 1000 never repeat a case)
OFFSET = int(os.environ.get("SINKATTN_FUZZ_OFFSET", "0"))


def fuzz_case(seed: int, max_tokens: int):
    """(lengths, window, use_rope, sink_mean, (Hq, Hkv), tile) of case `seed`."""
    rng = np.random.default_rng(1000 + seed)
    n_docs = int(rng.integers(1, 13))
    lengths = []
    for _ in range(n_docs):
        if rng.random() < 0.75:
            lengths.append(int(rng.choice(BOUNDARY_LENGTHS)))
        else:
            lengths.append(int(rng.integers(1, 1100)))
    # keep the oracle's work bounded: drop documents from the end past the cap
    while sum(lengths) > max_tokens and len(lengths) > 1:
        lengths.pop()
    if sum(lengths) > max_tokens:
        lengths = [max_tokens]
    window = int(rng.choice(WINDOWS))
    use_rope = bool(rng.random() < 0.5)
    sink_mean = float(rng.choice([0.0, 2.0]))
    heads = HEADS[int(rng.integers(len(HEADS)))]
    tile = int(rng.choice(TILES))
    return lengths, window, use_rope, sink_mean, heads, tile


def padded_case(seed: int):
    """A fuzz case plus the slot of each document: its length and a random
    amount of padding (none, 1, 15, 64 or uniform in [1, 129])."""
    lengths, window, use_rope, sink_mean, heads, tile = fuzz_case(200 + seed, 1500)
    rng = np.random.default_rng(5000 + seed)
    slots = [n + int(rng.choice([0, 0, 1, 15, 64, int(rng.integers(1, 130))])) for n in lengths]
    return lengths, slots, window, use_rope, sink_mean, heads, tile


@pytest.fixture(scope="module")
def gpu():
    return require_gpu()


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even), via the fp32 bits."""
    a = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    a = ((a + 0x7FFF + ((a >> 16) & 1)) >> 16) << 16
    return a.astype(np.uint32).view(np.float32).astype(np.float64)


def oracle_on_bf16_operands(q, k, v, cu, sinks, qnorm_w, knorm_w, window, use_rope):
    """The fp64 oracle's attention on the operands the bf16 MFMA consumes:
    q_hat * scale * log2(e) and k_hat rounded to bf16 (q_hat divided back)."""
    import oracle.oracle as O
    d = q.shape[2]
    scale = 1.0 / np.sqrt(d)
    c = scale * np.log2(np.e)
    qh = O.rmsnorm_rope(q, cu, qnorm_w, use_rope=use_rope)
    kh = O.rmsnorm_rope(k, cu, knorm_w, use_rope=use_rope)
    return O.attention(bf16_round(qh * c) / c, bf16_round(kh), v, cu, sinks, window=window,
                       scale=scale)


def check_bf16_forward(got_out, got_lse, ref_out, ref_lse, floor_out, floor_lse, label):
    """Element-wise: |got - ref| <= 2e-2 + |floor - ref| (out and lse); mean-abs
    within 2e-3."""
    assert np.all(np.isfinite(got_out)), f"{label}: non-finite output"
    assert got_out.shape == ref_out.shape and got_lse.shape == ref_lse.shape, label
    if got_out.size == 0:  # T = 0: nothing to compare
        return
    eo, el = errors(got_out, ref_out), errors(got_lse, ref_lse)
    allow_o = BF16_MAX + np.abs(floor_out - ref_out)
    allow_l = BF16_MAX + np.abs(floor_lse - ref_lse)
    excess_o = np.abs(got_out - ref_out) - allow_o
    excess_l = np.abs(got_lse - ref_lse) - allow_l
    print(f"  {label}: out max/mean {eo[0]:.3e}/{eo[1]:.3e} lse max/mean {el[0]:.3e}/{el[1]:.3e}; "
          f"operand-rounding allowance max {float(np.max(allow_o) - BF16_MAX):.2e}",
          flush=True)
    assert excess_o.max() <= 0 and eo[1] <= BF16_MEAN, (label, eo, float(excess_o.max()))
    assert excess_l.max() <= 0 and el[1] <= BF16_MEAN, (label, el, float(excess_l.max()))


def _describe(kind, seed, case):
    lengths, window, use_rope, sink_mean, heads, tile = case
    return (f"case fuzz {kind} seed={seed} T={sum(lengths)} docs={len(lengths)} "
            f"lengths={lengths} W={window} rope={use_rope} sinks~N({sink_mean},1) "
            f"heads={heads} tile={tile}")


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(OFFSET, OFFSET + N_FWD))
def test_forward_fuzz(gpu, seed):
    case = fuzz_case(seed, max_tokens=2500)
    lengths, window, use_rope, sink_mean, (hq, hkv), tile = case
    print(_describe("fwd", seed, case), flush=True)
    inp = custom_inputs(lengths, Hq=hq, Hkv=hkv, sink_mean=sink_mean, seed=seed)
    out, lse = gpu_forward(to_device(inp), window, use_rope, tile_config=tile)
    ref_out, ref_lse = oracle_forward(inp, window, use_rope)
    f = lambda t: t.double().numpy()  # noqa: E731
    fl_out, fl_lse = oracle_on_bf16_operands(f(inp["q"]), f(inp["k"]), f(inp["v"]),
                                             inp["cu_seqlens"].numpy(), f(inp["sinks"]),
                                             f(inp["qnorm_w"]), f(inp["knorm_w"]), window,
                                             use_rope)
    check_bf16_forward(out.float().cpu().numpy().astype(np.float64),
                       lse.cpu().numpy().astype(np.float64), ref_out, ref_lse, fl_out, fl_lse,
                       f"fuzz fwd {seed}")


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(OFFSET, OFFSET + N_BWD))
def test_backward_fuzz(gpu, seed):
    case = fuzz_case(100 + seed, max_tokens=1200)
    lengths, window, use_rope, sink_mean, (hq, hkv), _ = case
    print(_describe("bwd", seed, case), flush=True)
    inp = custom_inputs(lengths, Hq=hq, Hkv=hkv, sink_mean=sink_mean, seed=seed)
    check_bwd_parity(inp, window, use_rope, label=f"fuzz bwd {seed}")


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(OFFSET, OFFSET + N_FP16))
def test_forward_fuzz_fp16(gpu, seed):
    case = fuzz_case(300 + seed, max_tokens=2000)
    lengths, window, use_rope, sink_mean, (hq, hkv), tile = case
    print(_describe("fwd fp16", seed, case), flush=True)
    inp = custom_inputs(lengths, Hq=hq, Hkv=hkv, dtype="f16", sink_mean=sink_mean, seed=seed)
    check_parity(inp, window, use_rope, label=f"fuzz fwd fp16 {seed}", tile_config=tile)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(OFFSET, OFFSET + N_PADDED))
def test_padded_fuzz(gpu, seed):
    import attention_qk_rmsnorm_amd as A
    from test_gpu_padded import _check_grads, _oracle_bwd, _oracle_fwd, _padded_inputs
    lengths, slots, window, use_rope, sink_mean, (hq, hkv), tile = padded_case(seed)
    print(f"case fuzz padded seed={seed} lengths={lengths} slots={slots} W={window} "
          f"rope={use_rope} heads={(hq, hkv)} tile={tile}", flush=True)
    inp, rows, pad = _padded_inputs(lengths, slots, Hq=hq, Hkv=hkv, seed=seed)
    dev = to_device(inp)
    out, lse = A.sink_attn_fwd(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], dev["sinks"],
                               dev["qnorm_w"], dev["knorm_w"], window, use_rope,
                               cu_seqlens_padded=dev["cu_seqlens_padded"], tile_config=tile)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    lz = lse.cpu().numpy().astype(np.float64)
    # padding rows exactly: out 0, lse the sink
    assert np.all(o[pad] == 0.0)
    assert np.array_equal(lz[:, pad], np.repeat(inp["sinks"].numpy()[:, None], len(pad), 1)
                          .astype(np.float64))
    ref_out, ref_lse = _oracle_fwd(inp, window, use_rope, rows)
    # the operand floor on the real rows, packed as an unpadded batch
    f = lambda t: t.double().numpy()  # noqa: E731
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    fl_out, fl_lse = oracle_on_bf16_operands(f(inp["q"])[rows], f(inp["k"])[rows],
                                             f(inp["v"])[rows], cu, f(inp["sinks"]),
                                             f(inp["qnorm_w"]), f(inp["knorm_w"]), window,
                                             use_rope)
    check_bf16_forward(o[rows], lz[:, rows], ref_out[rows], ref_lse[:, rows], fl_out, fl_lse,
                       f"fuzz padded fwd {seed}")
    if seed % 2 == 0:  # the backward on half of them
        T = sum(slots)
        dout = workloads.make_grad_output(workloads.Workload("g", (T,), hq, hkv), seed)
        if len(pad):
            dout[torch.from_numpy(pad)] = float("nan")
        g = A.sink_attn_bwd(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], dev["sinks"],
                            dev["qnorm_w"], dev["knorm_w"], window, use_rope, out, lse,
                            dout.to("cuda:0"), cu_seqlens_padded=dev["cu_seqlens_padded"])
        torch.cuda.synchronize()
        _check_grads(g, _oracle_bwd(inp, window, use_rope, rows, dout), rows, pad,
                     f"fuzz padded bwd {seed}")


def test_cases_reach_the_boundary_classes():
    # (host logic only, runs without a GPU) the drawn cases cover every window
    # and tile choice, empty documents and both sides of the 64-key tile edge
    fwd = [fuzz_case(s, 2500) for s in range(N_FWD)]
    cases = fwd + [fuzz_case(100 + s, 1200) for s in range(N_BWD)]
    lengths = {n for c in cases for n in c[0]}
    assert set(BOUNDARY_LENGTHS) <= lengths, sorted(set(BOUNDARY_LENGTHS) - lengths)
    assert {c[1] for c in fwd} == set(WINDOWS)
    assert {c[5] for c in fwd} == set(TILES)
    assert {c[4] for c in fwd} == set(HEADS)
    padded = [padded_case(s) for s in range(N_PADDED)]
    assert all(sl >= n for c in padded for n, sl in zip(c[0], c[1]))
    assert any(sl > n for c in padded for n, sl in zip(c[0], c[1]))
    assert any(c[2] for c in cases) and not all(c[2] for c in cases)
