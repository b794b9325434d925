"""GPU parity of the padded layouts against the padded-THD oracle.

* padded THD (cu_seqlens with cu_seqlens_padded) through sink_attn_fwd_padded
  with every tile configuration and the fp32 path, and through
  sink_attn_bwd_padded; NaN stored at padding rows must not reach real rows;
  padding rows come back exactly as the pages' reading fixes them (out = 0,
  lse = sink, zero gradients);
* BSHD with a trailing-padding attention mask (sink_attn_fwd_bshd /
  sink_attn_bwd_bshd); a mask with padding before real tokens is rejected;
* RMSNorm eps = 0 with a ragged token count (keys past T once came out NaN).
"""
import numpy as np
import pytest
import torch

import workloads
from _harness import (BF16_MAX, BF16_MEAN, BWD_REL_FP16, BWD_REL_MAX, BWD_REL_MEAN, GRAD_KEYS,
                      check_parity, custom_inputs, errors, fwd_bounds, require_gpu,
                      to_device)

pytestmark = pytest.mark.gpu

LENGTHS = [70, 1, 0, 200, 33, 129]
SLOTS = [128, 64, 64, 256, 40, 192]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    return require_gpu()


def _say(msg):
    print(msg, flush=True)


def _padded_inputs(lengths, slots, Hq=32, Hkv=4, d=128, dtype="bf16", seed=0, junk=True):
    inp = custom_inputs(slots, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, seed=seed)
    cu, cp = workloads.padded_boundaries(lengths, slots)
    import oracle.oracle as O
    rows = O.padded_real_rows(cu, cp)
    pad = np.setdiff1d(np.arange(sum(slots)), rows)
    if junk and len(pad):
        for key in ("q", "k", "v"):
            inp[key][torch.from_numpy(pad)] = float("nan")
    inp["cu_seqlens"] = torch.from_numpy(cu)
    inp["cu_seqlens_padded"] = torch.from_numpy(cp)
    return inp, rows, pad


def _oracle_fwd(inp, window, use_rope, rows):
    import oracle.oracle as O
    f = lambda t: t.double().numpy()  # noqa: E731
    q, k, v = f(inp["q"]), f(inp["k"]), f(inp["v"])
    pad = np.setdiff1d(np.arange(q.shape[0]), rows)
    for a in (q, k, v):
        a[pad] = 0.0  # the oracle must not see them either way
    return O.sink_attn_fwd_padded(q, k, v, inp["cu_seqlens"].numpy(),
                                  inp["cu_seqlens_padded"].numpy(), f(inp["sinks"]),
                                  f(inp["qnorm_w"]), f(inp["knorm_w"]), window, use_rope)


def _check_fwd(inp, rows, pad, out, lse, window, use_rope, label):
    ref_out, ref_lse = _oracle_fwd(inp, window, use_rope, rows)
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o[rows])) and np.all(np.isfinite(l[:, rows])), label
    eo = errors(o[rows], ref_out[rows])
    el = errors(l[:, rows], ref_lse[:, rows])
    _say(f"  {label}: out max/mean {eo[0]:.3e}/{eo[1]:.3e} lse max {el[0]:.3e}")
    bmax, bmean = fwd_bounds(inp["q"].dtype)
    if inp["q"].dtype == torch.float32:
        assert eo[0] <= bmax and el[0] <= bmax, (label, eo, el)
    else:
        assert eo[0] <= bmax and eo[1] <= bmean and el[0] <= bmax, (label, eo, el)
    assert np.all(o[pad] == 0.0), label
    assert np.array_equal(l[:, pad], np.repeat(inp["sinks"].numpy()[:, None], len(pad), 1)
                          .astype(np.float64)), label


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("tile", [0, 1, 2, 3])
@pytest.mark.parametrize("window,use_rope", [(-1, False), (50, True)])
def test_padded_thd_forward(tile, window, use_rope, dtype):
    import attention_qk_rmsnorm_amd as A
    _say(f"case padded fwd tile={tile} W={window} {dtype}")
    inp, rows, pad = _padded_inputs(LENGTHS, SLOTS, dtype=dtype)
    dev = to_device(inp)
    out, lse = A.sink_attn_fwd(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], dev["sinks"],
                               dev["qnorm_w"], dev["knorm_w"], window, use_rope,
                               cu_seqlens_padded=dev["cu_seqlens_padded"], tile_config=tile)
    torch.cuda.synchronize()
    _check_fwd(inp, rows, pad, out, lse, window, use_rope, f"tile {tile}")


def test_padded_thd_forward_fp32():
    import attention_qk_rmsnorm_amd as A
    _say("case padded fwd fp32")
    inp, rows, pad = _padded_inputs([40, 0, 77, 5], [64, 16, 96, 8], Hq=4, Hkv=1, d=64,
                                    dtype="f32")
    dev = to_device(inp)
    out, lse = A.sink_attn_fwd(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], dev["sinks"],
                               dev["qnorm_w"], dev["knorm_w"], 20, True,
                               cu_seqlens_padded=dev["cu_seqlens_padded"])
    torch.cuda.synchronize()
    _check_fwd(inp, rows, pad, out, lse, 20, True, "fp32")


def test_eps_zero_with_ragged_token_count():
    # T = 317 leaves padding keys in the last 64-key tile; with eps = 0 their
    # norm must not turn into 0 * inf
    _say("case eps=0 ragged T")
    inp = custom_inputs([200, 117])
    check_parity(inp, -1, False, label="eps 0 narrow", rms_eps=0.0, tile_config=1)
    check_parity(inp, 64, True, label="eps 0 wide", rms_eps=0.0, tile_config=2)


def _check_grads(g, ref, rows, pad, label):
    msg, bad = [], []
    rmax, rmean = BWD_REL_FP16 if g["dq"].dtype == torch.float16 else (BWD_REL_MAX, BWD_REL_MEAN)
    for key in GRAD_KEYS:
        got = g[key].float().cpu().numpy().astype(np.float64)
        r = ref[key]
        if key in ("dq", "dk", "dv"):
            assert np.all(got[pad] == 0.0), (label, key)
            got, r = got[rows], r[rows]
        assert np.all(np.isfinite(got)), (label, key)
        emax, emean = errors(got, r)
        smax, smean = float(np.abs(r).max()), float(np.abs(r).mean())
        msg.append(f"{key} {emax / smax:.2e}/{emean / smean:.2e}")
        if emax > rmax * smax or emean > rmean * smean:
            bad.append(key)
    _say(f"  {label}: rel max/mean " + ", ".join(msg))
    assert not bad, (label, bad)


def _oracle_bwd(inp, window, use_rope, rows, dout):
    import oracle.oracle as O
    f = lambda t: t.double().numpy()  # noqa: E731
    q, k, v, do = f(inp["q"]), f(inp["k"]), f(inp["v"]), f(dout)
    pad = np.setdiff1d(np.arange(q.shape[0]), rows)
    for a in (q, k, v, do):
        a[pad] = 0.0
    return O.sink_attn_bwd_padded(q, k, v, inp["cu_seqlens"].numpy(),
                                  inp["cu_seqlens_padded"].numpy(), f(inp["sinks"]),
                                  f(inp["qnorm_w"]), f(inp["knorm_w"]), window, use_rope, do)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("window,use_rope", [(-1, False), (50, True)])
def test_padded_thd_backward(window, use_rope, dtype):
    import attention_qk_rmsnorm_amd as A
    _say(f"case padded bwd W={window} {dtype}")
    inp, rows, pad = _padded_inputs(LENGTHS, SLOTS, dtype=dtype)
    T = sum(SLOTS)
    dout = workloads.make_grad_output(workloads.Workload("g", (T,), dtype=dtype), 0)
    dout[torch.from_numpy(pad)] = float("nan")
    dev = to_device(inp)
    out, lse = A.sink_attn_fwd(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], dev["sinks"],
                               dev["qnorm_w"], dev["knorm_w"], window, use_rope,
                               cu_seqlens_padded=dev["cu_seqlens_padded"])
    g = A.sink_attn_bwd(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], dev["sinks"],
                        dev["qnorm_w"], dev["knorm_w"], window, use_rope, out, lse,
                        dout.to("cuda:0"), cu_seqlens_padded=dev["cu_seqlens_padded"])
    torch.cuda.synchronize()
    _check_grads(g, _oracle_bwd(inp, window, use_rope, rows, dout), rows, pad,
                 f"padded W={window}")


def test_bshd_mask_forward_backward_and_rejection():
    import attention_qk_rmsnorm_amd as A
    _say("case bshd mask")
    B, S, lengths = 3, 300, [300, 17, 150]
    inp = custom_inputs([S] * B, seed=2)
    mask = torch.arange(S)[None, :] < torch.tensor(lengths)[:, None]
    dev = to_device(inp)
    q = dev["q"].view(B, S, 32, 128)
    k = dev["k"].view(B, S, 4, 128)
    v = dev["v"].view(B, S, 4, 128)
    out, lse = A.sink_attn_fwd_bshd(q, k, v, mask.to("cuda:0"), dev["sinks"], dev["qnorm_w"],
                                    dev["knorm_w"], 100, True)
    torch.cuda.synchronize()
    assert out.shape == (B, S, 32, 128) and lse.shape == (32, B, S)
    cu, cp = workloads.padded_boundaries(lengths, [S] * B)
    pinp = dict(inp, cu_seqlens=torch.from_numpy(cu), cu_seqlens_padded=torch.from_numpy(cp))
    import oracle.oracle as O
    rows = O.padded_real_rows(cu, cp)
    pad = np.setdiff1d(np.arange(B * S), rows)
    _check_fwd(pinp, rows, pad, out.view(B * S, 32, 128), lse.reshape(32, B * S), 100, True,
               "bshd fwd")
    dout = workloads.make_grad_output(workloads.Workload("g", (B * S,)), 1)
    g = A.sink_attn_bwd_bshd(q, k, v, mask.to("cuda:0"), dev["sinks"], dev["qnorm_w"],
                             dev["knorm_w"], 100, True, out, lse,
                             dout.to("cuda:0").view(B, S, 32, 128))
    torch.cuda.synchronize()
    flat = {key: (val.reshape(B * S, *val.shape[2:]) if val.dim() == 4 else val)
            for key, val in g.items()}
    _check_grads(flat, _oracle_bwd(pinp, 100, True, rows, dout), rows, pad, "bshd bwd")
    holes = mask.clone()
    holes[1, 3] = False  # padding before real tokens
    with pytest.raises(ValueError):
        A.sink_attn_fwd_bshd(q, k, v, holes.to("cuda:0"), dev["sinks"], dev["qnorm_w"],
                             dev["knorm_w"], 100, True)


# ------------------------------------------------- full-size padded batch ---
# The BSHD batch of 8 rows x 4096 slots with the sliding layers' real lengths
# (W = 1024, RoPE), in the launch configuration the benchmark times: the
# boundaries from the attention mask, then the padded entry points.

def _full_bshd():
    import attention_qk_rmsnorm_amd as A
    w = workloads.named_workloads()["sliding_bshd"]
    inp = workloads.make_inputs(w)
    dev = to_device(inp)
    cu, cp = A.mask_to_seqlens(dev["attention_mask"])
    assert torch.equal(cu.cpu(), inp["cu_seqlens"]) and torch.equal(cp.cpu(),
                                                                     inp["cu_seqlens_padded"])
    return A, w, inp, dev, cu, cp


def test_full_size_bshd_forward_sampled_rows():
    A, w, inp, dev, cu, cp = _full_bshd()
    _say(f"case sliding_bshd fwd rows={w.num_rows} real={w.total_tokens}")
    c = A.Call(dev["q"], dev["k"], dev["v"], cu, dev["sinks"], dev["qnorm_w"], dev["knorm_w"],
               w.window, w.use_rope, cu_seqlens_padded=cp)
    c.fwd()
    torch.cuda.synchronize()
    import oracle.oracle as O
    real = O.padded_real_rows(inp["cu_seqlens"].numpy(), inp["cu_seqlens_padded"].numpy())
    pick = real[workloads.sample_rows(w.lengths, w.window, 192)]
    pad = np.setdiff1d(np.arange(w.num_rows), real)
    pick = np.concatenate([pick, pad[:: max(1, len(pad) // 64)]])
    f = lambda t: t.double().numpy()  # noqa: E731
    ref_out, ref_lse = O.sink_attn_fwd_padded(
        f(inp["q"]), f(inp["k"]), f(inp["v"]), inp["cu_seqlens"].numpy(),
        inp["cu_seqlens_padded"].numpy(), f(inp["sinks"]), f(inp["qnorm_w"]),
        f(inp["knorm_w"]), w.window, w.use_rope, rows=pick)
    o = c.out[torch.from_numpy(pick).cuda()].float().cpu().numpy().astype(np.float64)
    l = c.lse[:, torch.from_numpy(pick).cuda()].cpu().numpy().astype(np.float64)
    eo, el = errors(o, ref_out), errors(l, ref_lse)
    _say(f"  sliding_bshd: rows={len(pick)} out max/mean {eo[0]:.3e}/{eo[1]:.3e} "
         f"lse max {el[0]:.3e}")
    assert eo[0] <= BF16_MAX and eo[1] <= BF16_MEAN and el[0] <= BF16_MAX, (eo, el)
    # every padding row, on the device: out = 0, lse = the sink
    padt = torch.from_numpy(pad).cuda()
    assert torch.all(c.out[padt] == 0)
    assert torch.equal(c.lse[:, padt], dev["sinks"][:, None].expand(-1, len(pad)))


def test_full_size_bshd_backward():
    # every real row's dq, dk, dv and the batch-wide sums (dsinks, both
    # norm-weight gradients) against the fp64 oracle on the gathered real
    # tokens (the padded call's real rows are the unpadded call on them);
    # every padding row's gradient is zero.
    A, w, inp, dev, cu, cp = _full_bshd()
    _say(f"case sliding_bshd bwd rows={w.num_rows} real={w.total_tokens}")
    dout = workloads.make_grad_output(w)
    d_dout = dout.to("cuda:0")
    c = A.Call(dev["q"], dev["k"], dev["v"], cu, dev["sinks"], dev["qnorm_w"], dev["knorm_w"],
               w.window, w.use_rope, cu_seqlens_padded=cp)
    c.fwd()
    g = A.BwdCall(dev["q"], dev["k"], dev["v"], cu, dev["sinks"], dev["qnorm_w"],
                  dev["knorm_w"], w.window, w.use_rope, c.out, c.lse, d_dout,
                  cu_seqlens_padded=cp)
    g.run()
    torch.cuda.synchronize()
    grads = g.grads
    import oracle.oracle as O
    real = O.padded_real_rows(inp["cu_seqlens"].numpy(), inp["cu_seqlens_padded"].numpy())
    pad = torch.from_numpy(np.setdiff1d(np.arange(w.num_rows), real)).cuda()
    for key in ("dq", "dk", "dv"):
        assert torch.all(grads[key][pad] == 0), key
        assert torch.all(torch.isfinite(grads[key].float())), key
    f = lambda t: t.double().numpy()  # noqa: E731
    ref = O.sink_attn_bwd(f(inp["q"][real]), f(inp["k"][real]), f(inp["v"][real]),
                          inp["cu_seqlens"].numpy(), f(inp["sinks"]), f(inp["qnorm_w"]),
                          f(inp["knorm_w"]), w.window, w.use_rope, f(dout[real]))
    msg = []
    rt = torch.from_numpy(real).cuda()
    for key in ("dq", "dk", "dv", "dsinks", "dqnorm_w", "dknorm_w"):
        got = grads[key][rt] if key in ("dq", "dk", "dv") else grads[key]
        got = got.float().cpu().numpy().astype(np.float64)
        emax, emean = errors(got, ref[key])
        smax, smean = float(np.abs(ref[key]).max()), float(np.abs(ref[key]).mean())
        msg.append(f"{key} {emax / smax:.2e}/{emean / smean:.2e}")
        assert emax <= BWD_REL_MAX * smax and emean <= BWD_REL_MEAN * smean, (key, emax, emean)
    _say("  sliding_bshd bwd vs oracle: rel max/mean " + ", ".join(msg))


# tight slots: empty slots, slots that the document fills exactly and short
# padding gaps, so query blocks and key tiles span several documents
TIGHT_LENGTHS = [5, 0, 0, 3, 60, 0, 17, 1, 130, 64, 2]
TIGHT_SLOTS = [9, 0, 4, 3, 64, 0, 20, 2, 131, 64, 70]


@pytest.mark.parametrize("heads", [(32, 4), (8, 8), (32, 1)])
def test_padded_backward_tight_slots(heads):
    import attention_qk_rmsnorm_amd as A
    _say(f"case padded bwd tight slots heads={heads}")
    Hq, Hkv = heads
    inp, rows, pad = _padded_inputs(TIGHT_LENGTHS, TIGHT_SLOTS, Hq=Hq, Hkv=Hkv)
    T = sum(TIGHT_SLOTS)
    dout = workloads.make_grad_output(workloads.Workload("g", (T,), Hq, Hkv), 3)
    dout[torch.from_numpy(pad)] = float("nan")
    dev = to_device(inp)
    for window, use_rope in ((-1, False), (7, True)):
        out, lse = A.sink_attn_fwd(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"],
                                   dev["sinks"], dev["qnorm_w"], dev["knorm_w"], window,
                                   use_rope, cu_seqlens_padded=dev["cu_seqlens_padded"])
        torch.cuda.synchronize()
        _check_fwd(inp, rows, pad, out, lse, window, use_rope, f"tight fwd W={window}")
        g = A.sink_attn_bwd(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], dev["sinks"],
                            dev["qnorm_w"], dev["knorm_w"], window, use_rope, out, lse,
                            dout.to("cuda:0"), cu_seqlens_padded=dev["cu_seqlens_padded"])
        torch.cuda.synchronize()
        _check_grads(g, _oracle_bwd(inp, window, use_rope, rows, dout), rows, pad,
                     f"tight {heads} W={window}")


@pytest.mark.parametrize("batch,seq", [(1, 1), (3, 5), (300, 77), (700, 1), (2, 1000)])
def test_mask_to_seqlens_shapes(batch, seq):
    import attention_qk_rmsnorm_amd as A
    _say(f"case mask_to_seqlens {batch}x{seq}")
    rng = np.random.default_rng(batch * 1000 + seq)
    lengths = rng.integers(0, seq + 1, size=batch)
    mask = torch.from_numpy(np.arange(seq)[None, :] < lengths[:, None])
    cu, cp = A.mask_to_seqlens(mask.to("cuda:0"))
    ref_cu, ref_cp = workloads.padded_boundaries(lengths, [seq] * batch)
    assert np.array_equal(cu.cpu().numpy(), ref_cu) and np.array_equal(cp.cpu().numpy(), ref_cp)
    if seq > 2:
        holes = mask.clone()
        hit = np.nonzero(lengths >= 2)[0][:5]
        for b in hit:
            holes[b, 0] = False  # a gap before real tokens
        if len(hit):
            lib = A.load_library()
            m = holes.to("cuda:0").view(torch.uint8).contiguous()
            c = torch.empty(batch + 1, dtype=torch.int32, device="cuda:0")
            p = torch.empty_like(c)
            bad = torch.full((1,), -7, dtype=torch.int32, device="cuda:0")
            import ctypes
            rc = lib.sink_attn_mask_to_seqlens(
                ctypes.c_void_p(m.data_ptr()), batch, seq, ctypes.c_void_p(c.data_ptr()),
                ctypes.c_void_p(p.data_ptr()), ctypes.c_void_p(bad.data_ptr()),
                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            torch.cuda.synchronize()
            assert rc == 0 and int(bad.item()) == len(hit)
