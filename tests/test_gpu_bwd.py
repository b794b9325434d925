"""GPU parity of the backward pass (sink_attn_bwd) against the fp64 backward
oracle on the same bf16 inputs, output gradient and forward results.

Every gradient tensor is compared element by element; the tolerance is
relative to the tensor's own scale because gradient magnitudes grow with the
number of (token, head) terms a key collects (see _harness.BWD_REL_MAX)."""
import numpy as np
import pytest
import torch

from _harness import check_bwd_parity, custom_inputs, gpu_backward, require_gpu, to_device

pytestmark = pytest.mark.gpu

RAGGED = [1, 2, 3, 17, 63, 64, 65, 127, 128, 129, 200, 0, 31, 300]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    return require_gpu()


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("window,use_rope", [(-1, False), (1, True), (65, False), (100, True),
                                             (512, True)])
def test_ragged_documents(window, use_rope):
    _say(f"case bwd ragged W={window} rope={use_rope}")
    check_bwd_parity(custom_inputs(RAGGED), window, use_rope, label=f"W={window}")


@pytest.mark.parametrize("use_rope", [False, True])
def test_default_window_513(use_rope):
    # the pages' default sliding window (flint.config FlintConfig
    # sliding_window = 513 = 8 * 64 + 1) on documents longer than it
    _say(f"case bwd W=513 rope={use_rope}")
    check_bwd_parity(custom_inputs([1100, 513, 514, 37, 1040, 2]), 513, use_rope,
                     label=f"W=513 rope={use_rope}")


def test_causal_document_of_8192_tokens():
    # one causal document of 8,192 tokens against the fp64 backward oracle,
    # every element: key blocks deep in the document walk up to 2,048 column
    # tiles through the dK/dV ring, and dQ blocks up to 128 key tiles.  One
    # kv head with its 8 query heads (group size 8, as Flint's 32 / 4): the
    # kernels treat every kv head alike and on their own.
    _say("case bwd one causal doc 8192, 8q/1kv")
    check_bwd_parity(custom_inputs([8192], Hq=8, Hkv=1), -1, False, label="causal 8192")


def test_outputs_fully_written():
    # NaN guard bands around dq, dk, dv and the parameter gradients: every
    # element is written, nothing outside
    _say("case bwd poison guards")
    import attention_qk_rmsnorm_amd as A
    inp = to_device(custom_inputs([333, 1, 90, 0, 700]))
    T = 1124
    nan = float("nan")
    ref = gpu_backward(inp, 64, True)
    out, lse = A.sink_attn_fwd(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], inp["sinks"],
                               inp["qnorm_w"], inp["knorm_w"], 64, True)
    grads, bufs = {}, {}
    for key, shape, dt in (("dq", (T, 32, 128), torch.bfloat16),
                           ("dk", (T, 4, 128), torch.bfloat16),
                           ("dv", (T, 4, 128), torch.bfloat16),
                           ("dsinks", (32,), torch.float32),
                           ("dqnorm_w", (128,), torch.float32),
                           ("dknorm_w", (128,), torch.float32)):
        n = int(np.prod(shape))
        buf = torch.full((n + 256,), nan, dtype=dt, device="cuda:0")
        bufs[key] = (buf, n)
        grads[key] = buf[128:128 + n].view(shape)
    import workloads
    dout = workloads.make_grad_output(workloads.Workload("g", (T,), 32, 4, 128, "bf16"), 0)
    g = A.sink_attn_bwd(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], inp["sinks"],
                        inp["qnorm_w"], inp["knorm_w"], 64, True, out, lse,
                        dout.to("cuda:0"), grads=grads)
    torch.cuda.synchronize()
    for key, (buf, n) in bufs.items():
        assert torch.isfinite(g[key].float()).all(), key
        assert torch.isnan(buf[:128].float()).all(), key
        assert torch.isnan(buf[128 + n:].float()).all(), key
        assert torch.equal(g[key], ref[key]), key


def test_many_and_empty_documents():
    # a run of 80 empty documents inside one key tile and 4,315 documents in all
    lengths = [37] + [0] * 80 + [1] * 20 + [0] * 3 + [5] * 10 + [2, 0, 3] * 1400 + [90]
    _say(f"case bwd many documents ({len(lengths)})")
    check_bwd_parity(custom_inputs(lengths), 3, True, label="many docs W=3")


def test_forty_thousand_documents():
    # 40,002 documents of 0-2 tokens (more than 32,768: the deepest levels of
    # the wave-level document lookup)
    lengths = [1, 2, 0] * 13334
    _say(f"case bwd {len(lengths)} documents")
    check_bwd_parity(custom_inputs(lengths), -1, True, label="40k docs")


@pytest.mark.parametrize("heads", [(32, 4), (8, 8), (32, 1), (4, 2), (16, 16)])
def test_group_sizes(heads):
    _say(f"case bwd heads={heads}")
    inp = custom_inputs([150, 33, 290], Hq=heads[0], Hkv=heads[1])
    check_bwd_parity(inp, 100, True, label=f"{heads} W=100")
    check_bwd_parity(inp, -1, False, label=f"{heads} causal")


def test_long_document():
    _say("case bwd one doc 1500")
    inp = custom_inputs([1500])
    check_bwd_parity(inp, -1, False, label="causal 1500")
    check_bwd_parity(inp, 700, True, label="W=700 1500")


def test_sinks():
    _say("case bwd sinks")
    inp = custom_inputs([70, 130])
    g = check_bwd_parity(dict(inp, sinks=torch.full((32,), float("-inf"))), 40, True,
                         label="sink -inf")
    assert torch.all(g["dsinks"] == 0)
    check_bwd_parity(custom_inputs([70, 130], sink_mean=3.0), -1, False, label="sinks N(3,1)")


def test_norm_weights_and_scale():
    _say("case bwd norm weights, softmax scale, eps")
    inp = custom_inputs([90, 200], seed=3)
    g = torch.Generator().manual_seed(11)
    inp = dict(inp, qnorm_w=1 + 0.3 * torch.randn(128, generator=g),
               knorm_w=1 + 0.3 * torch.randn(128, generator=g))
    check_bwd_parity(inp, 50, True, label="weights N(1,0.3)")
    check_bwd_parity(inp, -1, True, label="scale 0.05", softmax_scale=0.05)
    check_bwd_parity(inp, -1, False, label="eps 1e-2", rms_eps=1e-2)


def test_determinism_and_empty_batch():
    _say("case bwd determinism + T=0")
    import attention_qk_rmsnorm_amd as A
    inp = to_device(custom_inputs([333, 1, 900]))
    a = gpu_backward(inp, 64, True)
    b = gpu_backward(inp, 64, True)
    for key in a:
        assert torch.equal(a[key], b[key]), key
    e = to_device(custom_inputs([0]))
    z = {k: torch.full_like(v, 7.0) for k, v in a.items() if k.startswith("ds") or "norm" in k}
    dq = torch.empty_like(e["q"])
    out = torch.empty_like(e["q"])
    lse = torch.empty((32, 0), dtype=torch.float32, device="cuda:0")
    grads = dict(z, dq=dq, dk=torch.empty_like(e["k"]), dv=torch.empty_like(e["v"]))
    A.sink_attn_bwd(e["q"], e["k"], e["v"], e["cu_seqlens"], e["sinks"], e["qnorm_w"],
                    e["knorm_w"], -1, False, out, lse, out, grads=grads)
    torch.cuda.synchronize()
    for key in ("dsinks", "dqnorm_w", "dknorm_w"):
        assert torch.all(grads[key] == 0), key


def test_dq_workgroup_sizes_agree():
    # the dQ kernel's two workgroup sizes (forced through tile_config): every
    # wave walks the same key tiles in the same order, so dq is bitwise equal;
    # dqnorm_w is summed over other workgroups, so only its rounding differs
    _say("case bwd dQ workgroups 128 vs 256 columns")
    import attention_qk_rmsnorm_amd as A
    inp = to_device(custom_inputs([333, 1, 900, 64, 1500], seed=4))
    res = {}
    for tile in (A.SINK_ATTN_TILE_NARROW, A.SINK_ATTN_TILE_WIDE):
        res[tile] = gpu_backward(inp, 300, True, bwd_tile_config=tile)
    a, b = res[A.SINK_ATTN_TILE_NARROW], res[A.SINK_ATTN_TILE_WIDE]
    for key in ("dq", "dk", "dv", "dsinks", "dknorm_w"):
        assert torch.equal(a[key], b[key]), key
    d = (a["dqnorm_w"] - b["dqnorm_w"]).abs().max().item()
    assert d <= 1e-5 * b["dqnorm_w"].abs().max().item(), d
    check_bwd_parity(custom_inputs([333, 1, 900, 64, 1500], seed=4), 300, True,
                     label="dQ 128 columns", bwd_tile_config=A.SINK_ATTN_TILE_NARROW)
    check_bwd_parity(custom_inputs([333, 1, 900, 64, 1500], seed=4), 300, True,
                     label="dQ 256 columns", bwd_tile_config=A.SINK_ATTN_TILE_WIDE)


def test_sliding_layer_scale():
    # two documents of 2500 and 3500 tokens with the sliding layers' 1024-key
    # window and RoPE: many key blocks and column tiles per document
    _say("case bwd T=6000 W=1024 rope")
    check_bwd_parity(custom_inputs([2500, 3500], seed=5), 1024, True, label="T=6000 W=1024")
