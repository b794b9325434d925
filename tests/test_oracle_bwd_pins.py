"""Pins of the backward oracle (oracle.c, oracle_sink_attn_bwd) to facts that do
not come from its own formulas:

* central finite differences of the forward oracle's loss sum(dout * out) at
  random coordinates of every input (q, k, v, sinks, both norm weights), with
  and without RoPE, windows, packed documents (one of length 1, one empty)
  and a disabled sink;
* torch.autograd in float64 through a dense masked-softmax formulation of
  the forward (its forward is first checked against the forward oracle), on
  every element, also with a dout that is zero on most rows (rows the oracle
  skips);
* exact identities: RMSNorm's scale invariance makes every (token, head) row
  of dq orthogonal to the raw q row (and dk to k) when eps = 0; out is linear
  in v, so sum(dv * v) = sum(dout * out); a disabled sink has zero gradient;
* the W = 1 closed form: out_t = sigma_t v_t with
  sigma_t = 1 / (1 + exp(sink - s_tt)), so dv_t = sum_h sigma dout_t and
  dsink_h = -sum_t sigma (1 - sigma) <dout_t, v_t>.
"""
import numpy as np
import pytest
import torch

import oracle.oracle as O


def _problem(seed=1, lengths=(9, 14), Hq=4, Hkv=2, d=8, sink=None):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    p = dict(q=rng.normal(size=(T, Hq, d)), k=rng.normal(size=(T, Hkv, d)),
             v=rng.normal(size=(T, Hkv, d)),
             sinks=rng.normal(size=Hq) if sink is None else np.full(Hq, sink),
             qw=1 + 0.2 * rng.normal(size=d), kw=1 + 0.2 * rng.normal(size=d))
    dout = rng.normal(size=(T, Hq, d))
    return cu, p, dout


def _loss(cu, p, dout, window, rope, theta, eps):
    out, _ = O.sink_attn_fwd(p["q"], p["k"], p["v"], cu, p["sinks"], p["qw"], p["kw"],
                             window, rope, eps=eps, theta=theta)
    return float((out * dout).sum())


def _grads(cu, p, dout, window, rope, theta, eps):
    return O.sink_attn_bwd(p["q"], p["k"], p["v"], cu, p["sinks"], p["qw"], p["kw"],
                           window, rope, dout, eps=eps, theta=theta)


KEYS = {"q": "dq", "k": "dk", "v": "dv", "sinks": "dsinks", "qw": "dqnorm_w",
        "kw": "dknorm_w"}


@pytest.mark.parametrize("lengths, window, rope, sink", [
    ((9, 14), -1, False, None),
    ((9, 14), 5, True, None),
    ((1, 12, 0, 7), 3, True, None),
    ((20,), -1, True, float("-inf")),
    ((6, 6), 1, False, None),
])
def test_finite_differences(lengths, window, rope, sink):
    cu, p, dout = _problem(lengths=lengths, sink=sink)
    theta, eps, h = 100.0, 1e-6, 1e-6
    g = _grads(cu, p, dout, window, rope, theta, eps)
    rng = np.random.default_rng(7)
    for name, key in KEYS.items():
        if name == "sinks" and sink is not None:
            continue
        arr = p[name]
        for _ in range(8):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            plus = dict(p, **{name: arr.copy()})
            plus[name][idx] += h
            minus = dict(p, **{name: arr.copy()})
            minus[name][idx] -= h
            fd = (_loss(cu, plus, dout, window, rope, theta, eps)
                  - _loss(cu, minus, dout, window, rope, theta, eps)) / (2 * h)
            an = g[key][idx]
            assert abs(fd - an) <= 1e-5 * max(1.0, abs(fd)), (name, idx, fd, an)


def _torch_forward(cu, p, window, rope, theta, eps, scale):
    q, k, v = p["q"], p["k"], p["v"]
    T, Hq, d = q.shape
    Hkv = k.shape[1]

    def norm(x, w):
        return w * x / torch.sqrt((x * x).mean(-1, keepdim=True) + eps)

    doc = torch.repeat_interleave(torch.arange(len(cu) - 1), torch.diff(torch.as_tensor(cu)))
    pos = (torch.arange(T) - torch.as_tensor(cu)[doc]).double()

    def rot(x):
        if not rope:
            return x
        i = torch.arange(d // 2, dtype=torch.float64)
        ang = pos[:, None] * theta ** (-2.0 * i / d)
        c, s = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]
        a, b = x[..., : d // 2], x[..., d // 2:]
        return torch.cat([a * c - b * s, b * c + a * s], -1)

    qh = rot(norm(q, p["qw"]))
    kh = rot(norm(k, p["kw"])).repeat_interleave(Hq // Hkv, dim=1)
    vv = v.repeat_interleave(Hq // Hkv, dim=1)
    s = scale * torch.einsum("thd,uhd->htu", qh, kh)
    t_idx, u_idx = torch.arange(T)[:, None], torch.arange(T)[None, :]
    vis = (doc[:, None] == doc[None, :]) & (u_idx <= t_idx)
    if window > 0:
        vis &= (t_idx - u_idx) < window
    s = s.masked_fill(~vis[None], float("-inf"))
    full = torch.cat([s, p["sinks"][:, None, None].expand(Hq, T, 1)], -1)
    P = torch.softmax(full, -1)[..., :T]
    return torch.einsum("htu,uhd->thd", P, vv)


@pytest.mark.parametrize("window, rope", [(-1, False), (4, True)])
def test_autograd_every_element(window, rope):
    cu, p, dout = _problem(seed=3, lengths=(5, 11, 1, 8))
    theta, eps = 100.0, 1e-6
    tp = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in p.items()}
    out = _torch_forward(cu, tp, window, rope, theta, eps, 1.0 / np.sqrt(8))
    ref, _ = O.sink_attn_fwd(p["q"], p["k"], p["v"], cu, p["sinks"], p["qw"], p["kw"],
                             window, rope, eps=eps, theta=theta)
    assert np.allclose(out.detach().numpy(), ref, rtol=0, atol=1e-12)
    (out * torch.tensor(dout)).sum().backward()
    g = _grads(cu, p, dout, window, rope, theta, eps)
    for name, key in KEYS.items():
        assert np.allclose(g[key], tp[name].grad.numpy(), rtol=1e-9, atol=1e-11), name


@pytest.mark.parametrize("window, rope", [(-1, False), (4, True)])
def test_autograd_sparse_dout(window, rope):
    # dout non-zero on a few (token, head) rows only, some tokens with a single
    # live head: the oracle skips the zero rows in both of its passes, and
    # every gradient must still be autograd's on every element
    cu, p, dout = _problem(seed=4, lengths=(5, 11, 1, 8))
    T, Hq, _ = dout.shape
    live = np.zeros((T, Hq), dtype=bool)
    live[[0, 4, 9, 15, 16, 24], :] = True
    live[[2, 12, 20], [1, 3, 0]] = True
    dout = np.where(live[:, :, None], dout, 0.0)
    theta, eps = 100.0, 1e-6
    tp = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in p.items()}
    out = _torch_forward(cu, tp, window, rope, theta, eps, 1.0 / np.sqrt(8))
    (out * torch.tensor(dout)).sum().backward()
    g = _grads(cu, p, dout, window, rope, theta, eps)
    for name, key in KEYS.items():
        assert np.allclose(g[key], tp[name].grad.numpy(), rtol=1e-9, atol=1e-11), name
    assert np.all(g["dq"][~live] == 0.0)


def test_norm_scale_invariance_and_value_linearity():
    cu, p, dout = _problem(seed=5, lengths=(13, 10))
    g = _grads(cu, p, dout, 6, True, 100.0, 0.0)       # eps = 0: exact scale invariance
    dots_q = np.einsum("thd,thd->th", g["dq"], p["q"])
    dots_k = np.einsum("thd,thd->th", g["dk"], p["k"])
    assert np.abs(dots_q).max() < 1e-12 and np.abs(dots_k).max() < 1e-12
    out, _ = O.sink_attn_fwd(p["q"], p["k"], p["v"], cu, p["sinks"], p["qw"], p["kw"], 6,
                             True, eps=0.0, theta=100.0)
    assert np.isclose((g["dv"] * p["v"]).sum(), (out * dout).sum(), rtol=1e-12)


def test_disabled_sink_has_no_gradient():
    cu, p, dout = _problem(seed=6, sink=float("-inf"))
    g = _grads(cu, p, dout, -1, False, 1e6, 1e-6)
    assert np.all(g["dsinks"] == 0.0)


def test_window_one_closed_form():
    cu, p, dout = _problem(seed=8, lengths=(7, 5))
    g = _grads(cu, p, dout, 1, True, 100.0, 1e-6)
    qh = O.rmsnorm_rope(p["q"], cu, p["qw"], eps=1e-6, theta=100.0, use_rope=True)
    kh = O.rmsnorm_rope(p["k"], cu, p["kw"], eps=1e-6, theta=100.0, use_rope=True)
    T, Hq, d = p["q"].shape
    Hkv = p["k"].shape[1]
    G = Hq // Hkv
    s_tt = np.einsum("thd,thd->th", qh, np.repeat(kh, G, axis=1)) / np.sqrt(d)
    sig = 1.0 / (1.0 + np.exp(p["sinks"][None, :] - s_tt))           # [T, Hq]
    vrep = np.repeat(p["v"], G, axis=1)
    dov = np.einsum("thd,thd->th", dout, vrep)
    dv = (sig[:, :, None] * dout).reshape(T, Hkv, G, d).sum(2)
    assert np.allclose(g["dv"], dv, rtol=1e-12, atol=1e-13)
    assert np.allclose(g["dsinks"], -(sig * (1 - sig) * dov).sum(0), rtol=1e-11, atol=1e-13)
