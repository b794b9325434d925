"""Pins of the padded-THD oracle (oracle.py sink_attn_fwd_padded /
sink_attn_bwd_padded) to facts outside its own code.

flint.layers FlintAttention.forward (attention_mask): padded queries and keys
are excluded from the real attention and the sink stays valid; attention.utils:
packed inputs carry cu_seqlens (real lengths) and cu_seqlens_padded.

* real rows equal torch scaled_dot_product_attention run on a BSHD batch with
  a boolean mask built from causality, the window and a key-padding mask (sink
  disabled, norm by torch F.rms_norm, GQA by repeat_interleave);
* padding query rows: the sink is the whole softmax, so out = 0 and
  lse = sink exactly;
* values stored at padding rows (huge, inf, NaN) change nothing;
* without padding the padded entry equals the unpadded oracle bitwise;
* backward: central finite differences of the padded loss, including
  coordinates of padding rows (whose gradient is exactly zero).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.oracle as O


def _batch(seed, B, S, lengths, Hq=4, Hkv=2, d=16):
    rng = np.random.default_rng(seed)
    T = B * S
    p = dict(q=rng.normal(size=(T, Hq, d)), k=rng.normal(size=(T, Hkv, d)),
             v=rng.normal(size=(T, Hkv, d)), sinks=rng.normal(size=Hq),
             qw=1 + 0.2 * rng.normal(size=d), kw=1 + 0.2 * rng.normal(size=d))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cp = (np.arange(B + 1) * S).astype(np.int32)
    return p, cu, cp


def _fwd(p, cu, cp, window, rope, sinks=None, eps=1e-6, theta=100.0):
    return O.sink_attn_fwd_padded(p["q"], p["k"], p["v"], cu, cp,
                                  p["sinks"] if sinks is None else sinks, p["qw"], p["kw"],
                                  window, rope, eps=eps, theta=theta)


@pytest.mark.parametrize("window", [-1, 5])
def test_real_rows_match_sdpa_with_key_padding_mask(window):
    B, S, lengths = 3, 24, (24, 13, 1)
    p, cu, cp = _batch(1, B, S, lengths)
    Hq, Hkv, d = 4, 2, 16
    out, lse = _fwd(p, cu, cp, window, False, sinks=np.full(Hq, -np.inf), eps=1e-6)
    t = {k: torch.tensor(v) for k, v in p.items()}
    qh = F.rms_norm(t["q"], (d,), t["qw"], eps=1e-6).view(B, S, Hq, d).transpose(1, 2)
    kh = F.rms_norm(t["k"], (d,), t["kw"], eps=1e-6).view(B, S, Hkv, d).transpose(1, 2)
    vv = t["v"].view(B, S, Hkv, d).transpose(1, 2)
    kh = kh.repeat_interleave(Hq // Hkv, dim=1)
    vv = vv.repeat_interleave(Hq // Hkv, dim=1)
    valid = torch.arange(S)[None, :] < torch.tensor(lengths)[:, None]          # [B, S]
    i, j = torch.arange(S)[:, None], torch.arange(S)[None, :]
    vis = (j <= i) & valid[:, None, :]                                         # [B, S, S]
    if window > 0:
        vis &= (i - j) < window
    ref = F.scaled_dot_product_attention(qh, kh, vv, attn_mask=vis[:, None])   # [B, Hq, S, d]
    ref = ref.transpose(1, 2).reshape(B * S, Hq, d).numpy()
    rows = O.padded_real_rows(cu, cp)
    assert np.allclose(out[rows], ref[rows], rtol=0, atol=1e-12)


def test_padding_rows_hold_the_sink_alone():
    B, S, lengths = 2, 20, (7, 20)
    p, cu, cp = _batch(2, B, S, lengths)
    out, lse = _fwd(p, cu, cp, -1, True)
    pad = np.setdiff1d(np.arange(B * S), O.padded_real_rows(cu, cp))
    assert len(pad) == 13
    assert np.all(out[pad] == 0.0)
    assert np.all(lse[:, pad] == p["sinks"][:, None])


def test_padding_values_do_not_matter():
    B, S, lengths = 3, 16, (3, 16, 9)
    p, cu, cp = _batch(3, B, S, lengths)
    pad = np.setdiff1d(np.arange(B * S), O.padded_real_rows(cu, cp))
    ref = _fwd(p, cu, cp, 4, True)
    junk = dict(p)
    for key in ("q", "k", "v"):
        junk[key] = p[key].copy()
        junk[key][pad] = np.nan
        junk[key][pad[::2]] = 1e300
    got = _fwd(junk, cu, cp, 4, True)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def test_no_padding_equals_unpadded():
    lengths = (5, 11, 1, 8)
    rng = np.random.default_rng(4)
    T = sum(lengths)
    q, k, v = rng.normal(size=(T, 4, 16)), rng.normal(size=(T, 2, 16)), rng.normal(size=(T, 2, 16))
    s, qw, kw = rng.normal(size=4), 1 + 0.1 * rng.normal(size=16), 1 + 0.1 * rng.normal(size=16)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    a = O.sink_attn_fwd_padded(q, k, v, cu, cu, s, qw, kw, 6, True, theta=100.0)
    b = O.sink_attn_fwd(q, k, v, cu, s, qw, kw, 6, True, theta=100.0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_backward_finite_differences_with_padding():
    B, S, lengths = 2, 12, (5, 12)
    p, cu, cp = _batch(5, B, S, lengths)
    rng = np.random.default_rng(9)
    dout = rng.normal(size=p["q"].shape)
    g = O.sink_attn_bwd_padded(p["q"], p["k"], p["v"], cu, cp, p["sinks"], p["qw"], p["kw"],
                               4, True, dout, theta=100.0)
    rows = O.padded_real_rows(cu, cp)
    pad = np.setdiff1d(np.arange(B * S), rows)
    for key in ("dq", "dk", "dv"):
        assert np.all(g[key][pad] == 0.0)

    def loss(pp):
        out, _ = _fwd(pp, cu, cp, 4, True)
        return float((out * dout).sum())

    h = 1e-6
    names = {"q": "dq", "k": "dk", "v": "dv", "sinks": "dsinks", "qw": "dqnorm_w",
             "kw": "dknorm_w"}
    for name, key in names.items():
        arr = p[name]
        for trial in range(6):
            if arr.ndim == 3:
                t = int(rows[trial % len(rows)] if trial % 2 == 0 else pad[trial % len(pad)])
                idx = (t,) + tuple(int(rng.integers(0, s)) for s in arr.shape[1:])
            else:
                idx = (int(rng.integers(0, arr.shape[0])),)
            plus = dict(p, **{name: arr.copy()})
            plus[name][idx] += h
            minus = dict(p, **{name: arr.copy()})
            minus[name][idx] -= h
            fd = (loss(plus) - loss(minus)) / (2 * h)
            assert abs(fd - g[key][idx]) <= 1e-5 * max(1.0, abs(fd)), (name, idx, fd, g[key][idx])


def test_selected_rows_equal_the_whole_batch():
    B, S, lengths = 3, 16, (3, 16, 9)
    p, cu, cp = _batch(6, B, S, lengths)
    whole = _fwd(p, cu, cp, 5, True)
    rows = np.array([0, 2, 3, 15, 16, 31, 32, 40, 41, 47])
    part = O.sink_attn_fwd_padded(p["q"], p["k"], p["v"], cu, cp, p["sinks"], p["qw"], p["kw"],
                                  5, True, theta=100.0, rows=rows)
    assert np.array_equal(part[0], whole[0][rows]) and np.array_equal(part[1], whole[1][:, rows])
