"""GPU check of sink_attn_fwd_noalloc, the forward for callers that cannot
allocate device memory: called through the C ABI, it must give exactly what
sink_attn_fwd gives on the same inputs (same kernels, so bitwise), on two
calls in a row where the second is smaller than the first -- the library's
device array then still holds the first call's larger images, which the
second call must neither read nor depend on -- and with output buffers passed
in, no torch allocation may happen during the call."""
import pytest
import torch

from _harness import (BF16_MAX, BF16_MEAN, custom_inputs, errors, gpu_forward,
                      oracle_forward, require_gpu, to_device)

pytestmark = pytest.mark.gpu

WIDE = 2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    return require_gpu()


def _say(msg):
    print(msg, flush=True)


def _noalloc_vs_fwd(A, inp, window, use_rope, **kw):
    dev = to_device(inp)
    ref_out, ref_lse = gpu_forward(dev, window, use_rope, **kw)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    A.sink_attn_fwd_noalloc(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], dev["sinks"],
                            dev["qnorm_w"], dev["knorm_w"], window, use_rope, out, lse, **kw)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(out, ref_out), "out differs from sink_attn_fwd"
    assert torch.equal(lse, ref_lse), "lse differs from sink_attn_fwd"


def test_noalloc_equals_fwd_on_two_calls_second_smaller(gpu):
    A = gpu
    # first call: 4,200 tokens through the wide tiles (images of ~9 MB and the
    # redo table in the library's array)
    _say("case noalloc call 1: [2900, 1, 1299] causal, wide tiles")
    big = custom_inputs([2900, 1, 1299])
    _noalloc_vs_fwd(A, big, -1, False, tile_config=WIDE)
    # second call, smaller: narrow tiles, RoPE, window
    _say("case noalloc call 2: [300, 45, 0, 7] W=64 RoPE, automatic tiles")
    small = custom_inputs([300, 45, 0, 7])
    _noalloc_vs_fwd(A, small, 64, True)
    # and the fp32 path
    _say("case noalloc call 3: fp32 [128], 4q/1kv, d=64")
    tiny = custom_inputs([128], Hq=4, Hkv=1, d=64, dtype="f32")
    _noalloc_vs_fwd(A, tiny, -1, False)


def test_noalloc_against_oracle(gpu):
    A = gpu
    _say("case noalloc vs oracle: [513, 1, 200] W=513 RoPE")
    inp = custom_inputs([513, 1, 200])
    dev = to_device(inp)
    out, lse = A.sink_attn_fwd_noalloc(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"],
                                       dev["sinks"], dev["qnorm_w"], dev["knorm_w"], 513, True)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_forward(inp, 513, True)
    eo = errors(out.float().cpu().numpy(), ref_out)
    el = errors(lse.cpu().numpy(), ref_lse)
    _say(f"  out max/mean {eo[0]:.3e}/{eo[1]:.3e} lse max/mean {el[0]:.3e}/{el[1]:.3e}")
    assert eo[0] <= BF16_MAX and eo[1] <= BF16_MEAN
    assert el[0] <= BF16_MAX and el[1] <= BF16_MEAN


def test_noalloc_rejects_a_call_past_its_array(gpu):
    A = gpu
    # 45,000 tokens at 4 kv heads need more than the 80 MiB array: rejected
    # on the host before any launch, the outputs untouched
    T = 45000
    q = torch.zeros((T, 32, 128), dtype=torch.bfloat16, device="cuda:0")
    kv = torch.zeros((T, 4, 128), dtype=torch.bfloat16, device="cuda:0")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda:0")
    w = torch.ones(128, device="cuda:0")
    s = torch.zeros(32, device="cuda:0")
    out = torch.full_like(q, 3.0)
    with pytest.raises(A.SinkAttnError) as e:
        A.sink_attn_fwd_noalloc(q, kv, kv, cu, s, w, w, -1, False, out)
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
