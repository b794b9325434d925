"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Small cases compare every output element; the full-size workloads (the sizes
and launch configuration the benchmark times) compare a deterministic sample of
rows the oracle computes one by one: each document's first and last 64 tokens,
the tokens around the window edge and seeded random tokens."""
import math

import numpy as np
import pytest
import torch

import workloads
from _harness import (BF16_MAX, check_parity, custom_inputs, errors, gpu_forward,
                      oracle_forward, require_gpu, to_device)

pytestmark = pytest.mark.gpu

RAGGED = [1, 2, 3, 17, 63, 64, 65, 127, 128, 129, 200, 0, 31]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    return require_gpu()


def _say(msg):
    print(msg, flush=True)


# ------------------------------------------------------------ fp32 debug ---

def test_tiny_reference_fp32():
    w = workloads.named_workloads()["tiny"]
    _say(f"case tiny fp32 {w.lengths}")
    check_parity(workloads.make_inputs(w), w.window, w.use_rope, label="tiny")


@pytest.mark.parametrize("d,heads,window,use_rope", [
    (128, (8, 2), -1, True), (128, (8, 2), 5, False), (64, (4, 1), 33, True),
    (64, (6, 3), -1, False),
])
def test_fp32_path_ragged(d, heads, window, use_rope):
    _say(f"case fp32 d={d} heads={heads} W={window} rope={use_rope}")
    inp = custom_inputs([5, 1, 40, 0, 77], Hq=heads[0], Hkv=heads[1], d=d, dtype="f32")
    check_parity(inp, window, use_rope, label="fp32")


# ------------------------------------------------------------- bf16 path ---

@pytest.mark.parametrize("window", [-1, 1, 2, 63, 64, 65, 100, 512])
@pytest.mark.parametrize("use_rope", [False, True])
def test_bf16_ragged_documents(window, use_rope):
    _say(f"case bf16 ragged W={window} rope={use_rope}")
    inp = custom_inputs(RAGGED)
    check_parity(inp, window, use_rope, label=f"ragged W={window}")


# The pages' default sliding window, 513 = 8 * 64 + 1 (flint.config
# FlintConfig sliding_window): a window edge one key past a tile boundary, on
# documents longer than the window (shorter ones see the whole causal range).
W513_LENGTHS = [1100, 513, 514, 37, 1040, 2]


@pytest.mark.parametrize("use_rope", [False, True])
@pytest.mark.parametrize("tile", [0, 1, 2])  # automatic, narrow, wide
def test_bf16_default_window_513(tile, use_rope):
    _say(f"case bf16 W=513 rope={use_rope} tile={tile}")
    check_parity(custom_inputs(W513_LENGTHS), 513, use_rope, label=f"W=513 tile={tile}",
                 tile_config=tile)


# 80 empty documents inside one 64-token key tile (more document starts than
# tokens: the prologue's per-tile document lookup leaves its window of 65
# starts and searches memory) and 4,315 documents in all (more than the 4,096
# starts the schedule keeps in LDS, and a third level of the lookup's search)
MANY_DOCS = [37] + [0] * 80 + [1] * 20 + [0] * 3 + [5] * 10 + [2, 0, 3] * 1400 + [90]


@pytest.mark.parametrize("window,use_rope", [(-1, False), (3, True)])
@pytest.mark.parametrize("tile", [1, 2])  # narrow, wide
def test_bf16_many_and_empty_documents(window, use_rope, tile):
    _say(f"case bf16 many documents ({len(MANY_DOCS)}) W={window} rope={use_rope} tile={tile}")
    inp = custom_inputs(MANY_DOCS)
    check_parity(inp, window, use_rope, label=f"many docs W={window} tile={tile}",
                 tile_config=tile)


def test_bf16_forty_thousand_documents():
    # 40,002 documents of 0-2 tokens: more than 32,768, so the document
    # lookups take their deepest search levels
    lengths = [1, 2, 0] * 13334
    _say(f"case bf16 {len(lengths)} documents")
    inp = custom_inputs(lengths)
    check_parity(inp, -1, False, label="40k docs causal")
    check_parity(inp, 2, True, label="40k docs W=2")


@pytest.mark.parametrize("heads", [(32, 4), (8, 8), (16, 4), (32, 1), (16, 1), (4, 2)])
def test_bf16_group_sizes(heads):
    _say(f"case bf16 heads={heads}")
    inp = custom_inputs([150, 33, 290], Hq=heads[0], Hkv=heads[1])
    check_parity(inp, 100, True, label=f"heads={heads}")
    check_parity(inp, -1, False, label=f"heads={heads}")


def test_bf16_long_document_multi_tile():
    _say("case bf16 one doc 1500")
    inp = custom_inputs([1500])
    check_parity(inp, -1, False, label="1500 causal")
    check_parity(inp, 300, True, label="1500 W=300")


def test_bf16_sink_minus_inf_and_denominator_dominant():
    inp = custom_inputs([70, 130])
    _say("case bf16 sink -inf")
    check_parity(dict(inp, sinks=torch.full((32,), float("-inf"))), 40, True, label="-inf")
    _say("case bf16 sink N(2,1)")
    check_parity(custom_inputs([70, 130], sink_mean=2.0), -1, False, label="N(2,1)")
    _say("case bf16 sink 8")
    check_parity(dict(inp, sinks=torch.full((32,), 8.0)), -1, True, label="sink 8")


def test_bf16_huge_sink_gives_zero_output():
    _say("case bf16 sink 1e4")
    inp = custom_inputs([50, 90])
    out, lse = gpu_forward(to_device(dict(inp, sinks=torch.full((32,), 1e4))), -1, False)
    assert torch.all(out == 0)
    assert torch.allclose(lse, torch.full_like(lse, 1e4))


def test_bf16_softmax_scale_override():
    # the bf16 rounding error of q_hat and k_hat grows with the scale; 0.06
    # (below the default 1/sqrt(128)) keeps the default tolerance meaningful
    # while a scale that is ignored or misapplied still fails it
    _say("case bf16 scale 0.06")
    inp = custom_inputs([120, 45])
    check_parity(inp, 50, True, label="scale", softmax_scale=0.06)


@pytest.mark.parametrize("scale", [0.2, 0.3])
@pytest.mark.parametrize("tile", [1, 2])
def test_bf16_large_softmax_scale_scaled_bound(scale, tile):
    # a score's error from rounding q_hat and k_hat to bf16 is proportional to
    # softmax_scale (and to the norm weights, near 1 here), so the bounds that
    # hold at Flint's default scale 1/sqrt(128) are taken times
    # scale * sqrt(128): 2.26x at 0.2, 3.39x at 0.3
    f = scale * math.sqrt(128)
    _say(f"case bf16 scale {scale} tile={tile} bounds x{f:.2f}")
    check_parity(custom_inputs([120, 45, 300]), 50, True, label=f"scale {scale} tile={tile}",
                 bound_scale=f, softmax_scale=scale, tile_config=tile)


def test_bf16_window_at_least_length_equals_causal():
    _say("case bf16 W >= S")
    inp = to_device(custom_inputs([300, 77]))
    a = gpu_forward(inp, -1, True)
    b = gpu_forward(inp, 300, True)
    c = gpu_forward(inp, 100000, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[0], c[0])
    assert torch.equal(a[1], b[1]) and torch.equal(a[1], c[1])


def test_bf16_packed_equals_per_document():
    # key tiles start at multiples of 64 of the packed token index, so packing
    # changes how keys group into tiles, hence the running max each P is
    # rounded to bf16 against (the denominator sums those same bf16 weights):
    # equal up to that rounding, not bitwise
    _say("case bf16 packed vs per-doc")
    lengths = [130, 7, 64, 300]
    inp = custom_inputs(lengths)
    dev = to_device(inp)
    out, lse = gpu_forward(dev, 100, True)
    cu = inp["cu_seqlens"].tolist()
    for n, L in enumerate(lengths):
        a, b = cu[n], cu[n + 1]
        one = dict(dev, q=dev["q"][a:b].contiguous(), k=dev["k"][a:b].contiguous(),
                   v=dev["v"][a:b].contiguous(),
                   cu_seqlens=torch.tensor([0, L], dtype=torch.int32, device="cuda"))
        o1, l1 = gpu_forward(one, 100, True)
        diff = (out[a:b].float() - o1.float()).abs()
        assert diff.max().item() <= 1e-2 and diff.mean().item() <= 1e-3
        assert torch.allclose(lse[:, a:b], l1, rtol=0, atol=1e-3)


def test_bf16_deterministic_and_fully_written():
    _say("case bf16 determinism + poison")
    inp = to_device(custom_inputs([333, 1, 90]))
    T = 424
    base = torch.full((T + 64, 32, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    guard = torch.full((32, T + 64), float("nan"), dtype=torch.float32, device="cuda")
    out = base[32:32 + T]
    lse = guard[:, :T].contiguous()
    o1, l1 = gpu_forward(inp, 64, True, out=out, lse=lse)
    assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
    assert torch.isnan(base[:32].float()).all() and torch.isnan(base[32 + T:].float()).all()
    o2, l2 = gpu_forward(inp, 64, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_bf16_stages_equal_forward():
    _say("case bf16 stages")
    import attention_qk_rmsnorm_amd as A
    inp = to_device(custom_inputs([200, 55]))
    ref = gpu_forward(inp, 33, True)
    c = A.sink_attn_prologue(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], inp["sinks"],
                             inp["qnorm_w"], inp["knorm_w"], 33, True)
    c.attention()
    torch.cuda.synchronize()
    assert torch.equal(c.out, ref[0]) and torch.equal(c.lse, ref[1])


def test_bf16_lse_optional_and_empty_batch():
    _say("case bf16 lse=None, T=0")
    inp = to_device(custom_inputs([40]))
    out, lse = gpu_forward(inp, -1, False, return_lse=False)
    ref, _ = gpu_forward(inp, -1, False)
    assert lse is None and torch.equal(out, ref)
    empty = to_device(custom_inputs([0, 0]))
    out, lse = gpu_forward(empty, -1, False)
    assert out.shape == (0, 32, 128)


# ------------------------------------------------- full-size workloads ---

def _sampled(name, n_random):
    w = workloads.named_workloads()[name]
    _say(f"case {name} T={w.total_tokens} D={w.num_docs} W={w.window} rope={w.use_rope}")
    inp = workloads.make_inputs(w)
    rows = workloads.sample_rows(w.lengths, w.window, n_random)
    eo, el = check_parity(inp, w.window, w.use_rope, rows=rows, label=name)
    _say(f"  {name}: rows={len(rows)} out max/mean {eo[0]:.3e}/{eo[1]:.3e} "
         f"lse max/mean {el[0]:.3e}/{el[1]:.3e}")


def test_sliding_all_rows():
    w = workloads.named_workloads()["sliding"]
    _say(f"case sliding all rows T={w.total_tokens}")
    inp = workloads.make_inputs(w)
    eo, el = check_parity(inp, w.window, w.use_rope, label="sliding")
    _say(f"  sliding: out max/mean {eo[0]:.3e}/{eo[1]:.3e} lse {el[0]:.3e}/{el[1]:.3e}")


# Full and Long: every document's first and last 64 rows, the rows around the
# window edge and 4,096 seeded random rows; Mixed (whose rows are short):
# the same edges and 1,024 random rows.
@pytest.mark.parametrize("name,n_random", [("full", 4096), ("long", 4096),
                                           ("mixed_sliding", 1024), ("mixed_causal", 1024)])
def test_full_size_sampled_rows(name, n_random):
    _sampled(name, n_random)


def test_sliding_workload_at_window_513_all_rows():
    # the sliding workload's documents (8 x U[256, 4096], RoPE) at the pages'
    # default window of 513 instead of its 1024, every row
    w = workloads.named_workloads()["sliding"]
    _say(f"case sliding W=513 all rows T={w.total_tokens}")
    inp = workloads.make_inputs(w)
    check_parity(inp, 513, w.use_rope, label="sliding W=513")
