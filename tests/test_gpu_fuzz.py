"""Seeded fuzz tier: random varlen batches against the fp64 oracle.

Every case is drawn from its seed alone (numpy's PCG64), so a failure names a
case that reruns exactly.  Document lengths come mostly from the tile-boundary
classes of the kernels -- one below, at and one above a multiple of 16, 32, 64
(the key tile), 128 and 256, plus 0, 1, 2 -- with some uniform draws between
them; the window from {1, 2, 63, 64, 65, 512, 513, 1024, causal} (513 is
flint.config FlintConfig's default sliding window); RoPE on or off; the
sinks centred on 0 or 2; a GQA shape; and the tile configuration (automatic,
narrow or wide).  The forward is compared on every row, the backward on every
gradient element, each within the bounds of the fixed-case tests."""
import numpy as np
import pytest

from _harness import check_bwd_parity, check_parity, custom_inputs, require_gpu

BOUNDARY_LENGTHS = [0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129,
                    255, 256, 257, 511, 512, 513]
WINDOWS = [1, 2, 63, 64, 65, 512, 513, 1024, -1]
HEADS = [(32, 4), (32, 4), (32, 4), (16, 2), (8, 8), (32, 1), (4, 2)]
TILES = [0, 1, 2]  # automatic, narrow, wide
N_FWD, N_BWD = 96, 24  # cases per run (seeds 0 .. N - 1)


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


@pytest.fixture(scope="module")
def gpu():
    return require_gpu()


def _describe(kind, seed, case):
    lengths, window, use_rope, sink_mean, heads, tile = case
    return (f"case fuzz {kind} seed={seed} T={sum(lengths)} docs={len(lengths)} "
            f"lengths={lengths} W={window} rope={use_rope} sinks~N({sink_mean},1) "
            f"heads={heads} tile={tile}")


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(N_FWD))
def test_forward_fuzz(gpu, seed):
    case = fuzz_case(seed, max_tokens=2500)
    lengths, window, use_rope, sink_mean, (hq, hkv), tile = case
    print(_describe("fwd", seed, case), flush=True)
    inp = custom_inputs(lengths, Hq=hq, Hkv=hkv, sink_mean=sink_mean, seed=seed)
    check_parity(inp, window, use_rope, label=f"fuzz fwd {seed}", tile_config=tile)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(N_BWD))
def test_backward_fuzz(gpu, seed):
    case = fuzz_case(100 + seed, max_tokens=1200)
    lengths, window, use_rope, sink_mean, (hq, hkv), _ = case
    print(_describe("bwd", seed, case), flush=True)
    inp = custom_inputs(lengths, Hq=hq, Hkv=hkv, sink_mean=sink_mean, seed=seed)
    check_bwd_parity(inp, window, use_rope, label=f"fuzz bwd {seed}")


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
    assert any(c[2] for c in cases) and not all(c[2] for c in cases)
