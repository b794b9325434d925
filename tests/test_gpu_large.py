"""GPU checks at a batch size where byte offsets pass 2^31: 147 documents of
4096 tokens (T = 602,112; q, out, dout and dq are 4.9 GB each), the sliding
layers' 1024-key window with RoPE.  A 32-bit offset anywhere in the
prologue, the attention kernels or the backward would show up in the last
documents of the batch.

Documents are independent (positions restart at each document), so the
oracle runs on the last two documents alone and is compared with those rows
of the GPU results; every output element is checked to be finite.  The
inputs are drawn on the device by torch's generator (seeded) and the slices
the oracle needs are copied back, so the oracle sees the same bits."""
import numpy as np
import pytest
import torch

import workloads
from _harness import BF16_MAX, BF16_MEAN, BWD_REL_MAX, BWD_REL_MEAN, errors, require_gpu

pytestmark = pytest.mark.gpu

D, L, W = 147, 4096, 1024
T = D * L


@pytest.fixture(scope="module")
def batch():
    require_gpu()
    g = torch.Generator(device="cuda:0")
    g.manual_seed(7)
    dev = "cuda:0"
    bf = torch.bfloat16
    inp = {
        "q": torch.randn((T, 32, 128), generator=g, device=dev, dtype=torch.float32).to(bf),
        "k": torch.randn((T, 4, 128), generator=g, device=dev, dtype=torch.float32).to(bf),
        "v": torch.randn((T, 4, 128), generator=g, device=dev, dtype=torch.float32).to(bf),
        "sinks": torch.randn((32,), generator=g, device=dev, dtype=torch.float32),
        "qnorm_w": 1 + 0.02 * torch.randn((128,), generator=g, device=dev, dtype=torch.float32),
        "knorm_w": 1 + 0.02 * torch.randn((128,), generator=g, device=dev, dtype=torch.float32),
        "cu_seqlens": torch.arange(0, T + 1, L, dtype=torch.int32, device=dev),
    }
    return inp


def _tail(x, n_docs):
    return x[T - n_docs * L:].cpu()


def test_forward_past_2gb_offsets(batch):
    import attention_qk_rmsnorm_amd as A
    print(f"case large fwd T={T}", flush=True)
    b = batch
    out, lse = A.sink_attn_fwd(b["q"], b["k"], b["v"], b["cu_seqlens"], b["sinks"], b["qnorm_w"],
                               b["knorm_w"], W, True)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    import oracle.oracle as O
    f = lambda t: t.double().numpy()  # noqa: E731
    rows = workloads.sample_rows([L, L], W, 256, seed=3)
    q2, k2, v2 = _tail(b["q"], 2), _tail(b["k"], 2), _tail(b["v"], 2)
    ref_out, ref_lse = O.sink_attn_fwd(f(q2)[rows], f(k2), f(v2), np.array([0, L, 2 * L], np.int32),
                                       f(b["sinks"].cpu()), f(b["qnorm_w"].cpu()),
                                       f(b["knorm_w"].cpu()), W, True, rows=rows)
    got = out[T - 2 * L:].float().cpu().numpy().astype(np.float64)[rows]
    gl = lse[:, T - 2 * L:].cpu().numpy().astype(np.float64)[:, rows]
    eo, el = errors(got, ref_out), errors(gl, ref_lse)
    print(f"  large fwd: rows={len(rows)} out max/mean {eo[0]:.3e}/{eo[1]:.3e} "
          f"lse max {el[0]:.3e}", flush=True)
    assert eo[0] <= BF16_MAX and eo[1] <= BF16_MEAN and el[0] <= BF16_MAX, (eo, el)


def test_backward_past_2gb_offsets(batch):
    import attention_qk_rmsnorm_amd as A
    print(f"case large bwd T={T}", flush=True)
    b = batch
    g = torch.Generator(device="cuda:0")
    g.manual_seed(8)
    dout = torch.randn((T, 32, 128), generator=g, device="cuda:0",
                       dtype=torch.float32).to(torch.bfloat16)
    c = A.Call(b["q"], b["k"], b["v"], b["cu_seqlens"], b["sinks"], b["qnorm_w"], b["knorm_w"],
               W, True)
    c.fwd()
    grads = A.BwdCall(b["q"], b["k"], b["v"], b["cu_seqlens"], b["sinks"], b["qnorm_w"],
                      b["knorm_w"], W, True, c.out, c.lse, dout).run()
    torch.cuda.synchronize()
    for key, t in grads.items():
        assert torch.isfinite(t.float()).all(), key
    import oracle.oracle as O
    f = lambda t: t.double().numpy()  # noqa: E731
    ref = O.sink_attn_bwd(f(_tail(b["q"], 1)), f(_tail(b["k"], 1)), f(_tail(b["v"], 1)),
                          np.array([0, L], np.int32), f(b["sinks"].cpu()),
                          f(b["qnorm_w"].cpu()), f(b["knorm_w"].cpu()), W, True,
                          f(_tail(dout, 1)))
    msg = []
    for key in ("dq", "dk", "dv"):
        got = grads[key][T - L:].float().cpu().numpy().astype(np.float64)
        emax, emean = errors(got, ref[key])
        smax, smean = float(np.abs(ref[key]).max()), float(np.abs(ref[key]).mean())
        msg.append(f"{key} {emax / smax:.2e}/{emean / smean:.2e}")
        assert emax <= BWD_REL_MAX * smax and emean <= BWD_REL_MEAN * smean, (key, emax, emean)
    print("  large bwd (last document): rel max/mean " + ", ".join(msg), flush=True)
