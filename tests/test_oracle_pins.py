"""Pins of the fp64 oracle to facts the pages and the mathematics fix.

None of these tests retypes the oracle's arithmetic: each compares it with a
library routine (torch rms_norm, torch scaled_dot_product_attention, scipy
logsumexp), a closed form, an invariant, or a second formulation built from
different primitives (dense masked matrices and rotation matrices).

Sources: NeMo AutoModel API pages "flint.layers" (FlintAttention,
_FlintSinkParameters), "flint.config" (FlintConfig docstring and fields) and
"attention.utils" (preprocess_args_and_kwargs_for_attn).
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

EPS = 1e-6
THETA = 1e6


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _cu(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return cu


def _torch_rmsnorm(x, w, eps=EPS):
    return F.rms_norm(torch.from_numpy(np.ascontiguousarray(x)), (x.shape[-1],),
                      torch.from_numpy(np.ascontiguousarray(w)), eps).numpy()


# ---------------------------------------------------------------- RMSNorm ---
# flint.layers FlintAttention: per-head RMSNorm (q_norm / k_norm);
# flint.config FlintConfig.rms_norm_eps = 1e-6.

@pytest.mark.parametrize("magnitude", [1.0, 1e-4])
def test_rmsnorm_is_torch_rms_norm(oracle_mod, magnitude):
    # the small magnitude makes mean(x^2) ~ eps, so a dropped eps fails
    rng = np.random.default_rng(1)
    x = magnitude * _rand(rng, 7, 3, 16)
    w = 1 + 0.1 * _rand(rng, 16)
    y = oracle_mod.rmsnorm_rope(x, [0, 7], w, eps=EPS, use_rope=False)
    np.testing.assert_allclose(y, _torch_rmsnorm(x, w), rtol=1e-13, atol=1e-15)


def test_rmsnorm_unit_weight_mean_square(oracle_mod):
    rng = np.random.default_rng(2)
    x = _rand(rng, 5, 2, 32) * np.array([1e-3, 1.0])[None, :, None]
    y = oracle_mod.rmsnorm_rope(x, [0, 5], np.ones(32), eps=EPS, use_rope=False)
    m = (x ** 2).mean(-1)
    np.testing.assert_allclose((y ** 2).mean(-1), m / (m + EPS), rtol=1e-12)


def test_rmsnorm_scale_invariant_without_eps(oracle_mod):
    rng = np.random.default_rng(3)
    x = _rand(rng, 4, 2, 16)
    w = 1 + 0.1 * _rand(rng, 16)
    a = oracle_mod.rmsnorm_rope(x, [0, 4], w, eps=0.0, use_rope=False)
    b = oracle_mod.rmsnorm_rope(37.5 * x, [0, 4], w, eps=0.0, use_rope=False)
    np.testing.assert_allclose(a, b, rtol=1e-13)


# ------------------------------------------------------------------- RoPE ---
# flint.layers FlintAttention._apply_rope: rotate corresponding channels in the
# two halves of each head; flint.config: NeoX RoPE over all head channels;
# forward: THD positions are document-local and zero-based.

def test_rope_position_zero_is_identity(oracle_mod):
    rng = np.random.default_rng(4)
    lengths = [5, 3, 6]
    x = _rand(rng, 14, 2, 16)
    w = 1 + 0.1 * _rand(rng, 16)
    a = oracle_mod.rmsnorm_rope(x, _cu(lengths), w, use_rope=True)
    b = oracle_mod.rmsnorm_rope(x, _cu(lengths), w, use_rope=False)
    starts = [0, 5, 8]
    for t in range(14):
        if t in starts:
            assert np.array_equal(a[t], b[t])
        else:
            assert not np.allclose(a[t], b[t])


def _basis_doc(d, i, n_tokens, lengths):
    x = np.zeros((n_tokens, 1, d))
    x[:, 0, i] = 1.0
    return x


@pytest.mark.parametrize("i, inv_freq", [
    (0, 1.0),                      # theta^0
    (16, 10.0 ** -1.5),            # theta^(-32/128) = (1e6)^(-1/4)
    (32, 1e-3),                    # theta^(-64/128) = (1e6)^(-1/2)
    (48, 10.0 ** -4.5),            # theta^(-96/128) = (1e6)^(-3/4)
])
def test_rope_pair_closed_form(oracle_mod, i, inv_freq):
    d, half = 128, 64
    lengths = [700, 1300]               # the second document restarts at 0
    T = sum(lengths)
    scale_n = 1.0 / math.sqrt(1.0 / d + EPS)   # RMSNorm of a basis vector
    pos = np.concatenate([np.arange(L) for L in lengths]).astype(np.float64)
    # first-half basis vector e_i -> cos(phi) e_i + sin(phi) e_{i+64}
    y = oracle_mod.rmsnorm_rope(_basis_doc(d, i, T, lengths), _cu(lengths),
                                np.ones(d), eps=EPS, theta=THETA, use_rope=True)
    phi = pos * inv_freq
    np.testing.assert_allclose(y[:, 0, i], scale_n * np.cos(phi), atol=1e-11)
    np.testing.assert_allclose(y[:, 0, i + half], scale_n * np.sin(phi), atol=1e-11)
    others = np.delete(y[:, 0, :], [i, i + half], axis=1)
    assert np.all(others == 0.0)
    # second-half basis vector e_{i+64} -> -sin(phi) e_i + cos(phi) e_{i+64}
    y2 = oracle_mod.rmsnorm_rope(_basis_doc(d, i + half, T, lengths), _cu(lengths),
                                 np.ones(d), eps=EPS, theta=THETA, use_rope=True)
    np.testing.assert_allclose(y2[:, 0, i], -scale_n * np.sin(phi), atol=1e-11)
    np.testing.assert_allclose(y2[:, 0, i + half], scale_n * np.cos(phi), atol=1e-11)


def test_rope_relative_position_and_norm(oracle_mod):
    rng = np.random.default_rng(5)
    d, L = 64, 40
    x = np.repeat(_rand(rng, 1, 1, d), L, axis=0)
    y = oracle_mod.rmsnorm_rope(x, [0, L], np.ones(d), use_rope=True)[:, 0, :]
    norms = np.linalg.norm(y, axis=1)
    np.testing.assert_allclose(norms, norms[0], rtol=1e-13)
    for a, b, c in [(3, 7, 11), (0, 20, 5), (10, 2, 17)]:
        np.testing.assert_allclose(y[a] @ y[b], y[a + c] @ y[b + c], rtol=1e-11, atol=1e-12)


# ------------------------------------------------------ attention and sink ---

def _mask_from_library(lengths, window):
    """Block-diagonal (document ids) band mask built with torch.block_diag,
    torch.tril and torch.triu: True where a key is visible."""
    blocks = []
    for L in lengths:
        ones = torch.ones((L, L), dtype=torch.bool)
        band = torch.tril(ones)
        if window > 0:
            band = band & torch.triu(ones, diagonal=-(window - 1))
        blocks.append(band)
    return torch.block_diag(*blocks) if blocks else torch.zeros((0, 0), dtype=torch.bool)


@pytest.mark.parametrize("window", [-1, 1, 3, 100])
def test_sink_minus_inf_is_torch_sdpa(oracle_mod, window):
    # sink = -inf removes the sink category: ordinary softmax attention
    rng = np.random.default_rng(6)
    lengths = [7, 0, 12, 5]
    T, Hq, Hkv, d = sum(lengths), 8, 2, 16
    G = Hq // Hkv
    qh, kh, v = _rand(rng, T, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d)
    out, lse = oracle_mod.attention(qh, kh, v, _cu(lengths), np.full(Hq, -np.inf),
                                    window=window)
    tq = torch.from_numpy(qh).permute(1, 0, 2)
    tk = torch.from_numpy(kh).repeat_interleave(G, dim=1).permute(1, 0, 2)
    tv = torch.from_numpy(v).repeat_interleave(G, dim=1).permute(1, 0, 2)
    mask = _mask_from_library(lengths, window)
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                         scale=1.0 / math.sqrt(d))
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    # lse at sink = -inf is the logsumexp over the visible scores
    s = np.einsum("thd,uhd->htu", qh, np.repeat(kh, G, axis=1)) / math.sqrt(d)
    s = np.where(mask.numpy()[None], s, -np.inf)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=1e-12)


def test_sink_minus_inf_single_doc_is_sdpa_is_causal(oracle_mod):
    # causal direction and scale against SDPA's own causal mask
    rng = np.random.default_rng(7)
    T, Hq, Hkv, d = 23, 4, 4, 32
    qh, kh, v = _rand(rng, T, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d)
    out, _ = oracle_mod.attention(qh, kh, v, [0, T], np.full(Hq, -np.inf), window=-1)
    ref = F.scaled_dot_product_attention(
        *(torch.from_numpy(a).permute(1, 0, 2) for a in (qh, kh, v)), is_causal=True)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def _full_inputs(rng, lengths, Hq=8, Hkv=2, d=16):
    T = sum(lengths)
    return dict(q=_rand(rng, T, Hq, d), k=_rand(rng, T, Hkv, d), v=_rand(rng, T, Hkv, d),
                cu_seqlens=_cu(lengths), sinks=_rand(rng, Hq),
                qnorm_w=1 + 0.02 * _rand(rng, d), knorm_w=1 + 0.02 * _rand(rng, d))


def test_sink_closed_form_identity(oracle_mod):
    # adding one zero-value category of logit s: out scales by the sigmoid of
    # (lse - s) and the log-normaliser becomes logaddexp(lse, s)
    rng = np.random.default_rng(8)
    inp = _full_inputs(rng, [9, 4, 13])
    base = dict(inp, sinks=np.full(8, -np.inf))
    out0, lse0 = oracle_mod.sink_attn_fwd(**base, window=5, use_rope=True)
    out1, lse1 = oracle_mod.sink_attn_fwd(**inp, window=5, use_rope=True)
    s = inp["sinks"][:, None]
    np.testing.assert_allclose(lse1, np.logaddexp(lse0, s), rtol=1e-13)
    sig = scipy.special.expit(lse0 - s)            # [Hq, T]
    np.testing.assert_allclose(out1, out0 * sig.T[:, :, None], rtol=1e-12, atol=1e-14)


def test_huge_sink_zeroes_output(oracle_mod):
    rng = np.random.default_rng(9)
    inp = _full_inputs(rng, [6, 10])
    inp["sinks"] = np.full(8, 1e4)
    out, lse = oracle_mod.sink_attn_fwd(**inp, window=-1, use_rope=True)
    assert np.all(out == 0.0)
    assert np.all(lse == 1e4)


def test_sink_is_not_scaled(oracle_mod):
    # one visible key (W = 1): lse = logaddexp(s_tt, sink) with the sink used
    # as given, not multiplied by 1/sqrt(d)
    rng = np.random.default_rng(10)
    inp = _full_inputs(rng, [4])
    out, lse = oracle_mod.sink_attn_fwd(**inp, window=1, use_rope=False)
    qn = _torch_rmsnorm(inp["q"], inp["qnorm_w"])
    kn = _torch_rmsnorm(inp["k"], inp["knorm_w"])
    G = 4
    s = np.einsum("thd,thd->ht", qn, np.repeat(kn, G, axis=1)) / 4.0
    np.testing.assert_allclose(lse, np.logaddexp(s, inp["sinks"][:, None]), rtol=1e-13)


@pytest.mark.parametrize("use_rope", [False, True])
def test_window_one_closed_form(oracle_mod, use_rope):
    # W = 1: only the query's own key is visible; RoPE cancels at equal
    # positions, so out_t = v_t * sigmoid(s_tt - sink)
    rng = np.random.default_rng(11)
    lengths = [5, 1, 8]
    inp = _full_inputs(rng, lengths)
    out, lse = oracle_mod.sink_attn_fwd(**inp, window=1, use_rope=use_rope)
    qn = _torch_rmsnorm(inp["q"], inp["qnorm_w"])
    kn = _torch_rmsnorm(inp["k"], inp["knorm_w"])
    kn_rep = np.repeat(kn, 4, axis=1)
    v_rep = np.repeat(inp["v"], 4, axis=1)
    s = np.einsum("thd,thd->th", qn, kn_rep) / 4.0                   # [T, Hq]
    sig = scipy.special.expit(s - inp["sinks"][None, :])
    np.testing.assert_allclose(out, v_rep * sig[:, :, None], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse.T, np.logaddexp(s, inp["sinks"][None, :]), rtol=1e-12)


@pytest.mark.parametrize("use_rope", [False, True])
def test_window_at_least_doc_length_is_causal(oracle_mod, use_rope):
    rng = np.random.default_rng(12)
    lengths = [11, 3, 17]
    inp = _full_inputs(rng, lengths)
    causal = oracle_mod.sink_attn_fwd(**inp, window=-1, use_rope=use_rope)
    for W in (17, 18, 1000):
        wide = oracle_mod.sink_attn_fwd(**inp, window=W, use_rope=use_rope)
        assert np.array_equal(causal[0], wide[0]) and np.array_equal(causal[1], wide[1])
    narrow = oracle_mod.sink_attn_fwd(**inp, window=16, use_rope=use_rope)
    assert not np.array_equal(causal[0], narrow[0])


@pytest.mark.parametrize("window,use_rope", [(-1, False), (4, True)])
def test_packed_equals_per_document(oracle_mod, window, use_rope):
    rng = np.random.default_rng(13)
    lengths = [9, 1, 14, 0, 6]
    inp = _full_inputs(rng, lengths)
    out, lse = oracle_mod.sink_attn_fwd(**inp, window=window, use_rope=use_rope)
    cu = inp["cu_seqlens"]
    for n, L in enumerate(lengths):
        a, b = cu[n], cu[n + 1]
        one = dict(inp, q=inp["q"][a:b], k=inp["k"][a:b], v=inp["v"][a:b],
                   cu_seqlens=np.array([0, L], dtype=np.int32))
        o1, l1 = oracle_mod.sink_attn_fwd(**one, window=window, use_rope=use_rope)
        assert np.array_equal(out[a:b], o1) and np.array_equal(lse[:, a:b], l1)
    # permuting documents permutes the outputs
    perm = [2, 0, 4, 3, 1]
    idx = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in perm]).astype(int)
    plen = [lengths[n] for n in perm]
    pinp = dict(inp, q=inp["q"][idx], k=inp["k"][idx], v=inp["v"][idx], cu_seqlens=_cu(plen))
    po, pl = oracle_mod.sink_attn_fwd(**pinp, window=window, use_rope=use_rope)
    assert np.array_equal(po, out[idx]) and np.array_equal(pl, lse[:, idx])


def test_gqa_is_mha_with_repeated_kv(oracle_mod):
    # query head h reads kv head h // G, i.e. torch.repeat_interleave of K/V
    rng = np.random.default_rng(14)
    lengths = [10, 7]
    inp = _full_inputs(rng, lengths, Hq=8, Hkv=2)
    gqa = oracle_mod.sink_attn_fwd(**inp, window=6, use_rope=True)
    mha_in = dict(inp, k=np.repeat(inp["k"], 4, axis=1), v=np.repeat(inp["v"], 4, axis=1))
    mha = oracle_mod.sink_attn_fwd(**mha_in, window=6, use_rope=True)
    assert np.array_equal(gqa[0], mha[0]) and np.array_equal(gqa[1], mha[1])
    # permuting query heads inside one group permutes the outputs
    perm = [3, 1, 0, 2, 4, 5, 6, 7]
    pin = dict(inp, q=inp["q"][:, perm], sinks=inp["sinks"][perm])
    po, pl = oracle_mod.sink_attn_fwd(**pin, window=6, use_rope=True)
    assert np.array_equal(po, gqa[0][:, perm]) and np.array_equal(pl, gqa[1][perm])


def test_constant_keys_closed_form(oracle_mod):
    # equal keys in a document give equal scores s_t, so
    # out_t = sum_J v / (|J| + exp(sink - s_t))
    rng = np.random.default_rng(15)
    lengths = [6, 9]
    inp = _full_inputs(rng, lengths, Hq=4, Hkv=1)
    cu = inp["cu_seqlens"]
    for n in range(2):
        inp["k"][cu[n]:cu[n + 1]] = inp["k"][cu[n]]
    W = 4
    out, _ = oracle_mod.sink_attn_fwd(**inp, window=W, use_rope=False)
    qn = _torch_rmsnorm(inp["q"], inp["qnorm_w"])
    kn = _torch_rmsnorm(inp["k"], inp["knorm_w"])
    for n in range(2):
        for t in range(cu[n], cu[n + 1]):
            J = np.arange(max(cu[n], t - W + 1), t + 1)
            for h in range(4):
                s = qn[t, h] @ kn[t, 0] / 4.0
                exp = inp["v"][J, 0].sum(0) / (len(J) + math.exp(inp["sinks"][h] - s))
                np.testing.assert_allclose(out[t, h], exp, rtol=1e-11, atol=1e-13)


# ---------------------------------------------- second formulation (dense) ---

def _rotation_matrix(d, p, theta):
    half = d // 2
    R = np.zeros((d, d))
    for i in range(half):
        ang = p * theta ** (-2.0 * i / d)
        c, s = math.cos(ang), math.sin(ang)
        R[i, i], R[i, i + half] = c, -s
        R[i + half, i], R[i + half, i + half] = s, c
    return R


def _dense_reference(inp, window, use_rope, theta=THETA):
    """Dense formulation: torch rms_norm, rotation matrices, a T x T score
    matrix per head with a library-built mask, the sink appended as one extra
    column whose value row is zero, scipy softmax / logsumexp over it."""
    q, k, v = inp["q"], inp["k"], inp["v"]
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    cu = inp["cu_seqlens"]
    lengths = np.diff(cu)
    pos = np.concatenate([np.arange(L) for L in lengths]) if T else np.zeros(0)
    qn = _torch_rmsnorm(q, inp["qnorm_w"])
    kn = _torch_rmsnorm(k, inp["knorm_w"])
    if use_rope:
        Rs = np.stack([_rotation_matrix(d, p, theta) for p in pos])
        qn = np.einsum("tij,thj->thi", Rs, qn)
        kn = np.einsum("tij,thj->thi", Rs, kn)
    mask = _mask_from_library(list(lengths), window).numpy()
    out = np.zeros_like(q)
    lse = np.zeros((Hq, T))
    for h in range(Hq):
        g = h // G
        S = qn[:, h] @ kn[:, g].T / math.sqrt(d)
        S = np.where(mask, S, -np.inf)
        S_ext = np.concatenate([S, np.full((T, 1), inp["sinks"][h])], axis=1)
        P = scipy.special.softmax(S_ext, axis=1)
        V_ext = np.concatenate([v[:, g], np.zeros((1, d))], axis=0)
        out[:, h] = P @ V_ext
        lse[h] = scipy.special.logsumexp(S_ext, axis=1)
    return out, lse


@pytest.mark.parametrize("window,use_rope,heads", [
    (-1, False, (8, 2)), (3, True, (8, 2)), (7, True, (4, 1)), (-1, True, (6, 3)),
])
def test_dense_second_formulation(oracle_mod, window, use_rope, heads):
    rng = np.random.default_rng(16)
    lengths = [12, 1, 0, 9, 5]
    inp = _full_inputs(rng, lengths, Hq=heads[0], Hkv=heads[1], d=16)
    out, lse = oracle_mod.sink_attn_fwd(**inp, window=window, use_rope=use_rope)
    ref_out, ref_lse = _dense_reference(inp, window, use_rope)
    np.testing.assert_allclose(out, ref_out, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-13)


def test_lse_normalises_probabilities(oracle_mod):
    # with lse the full log-normaliser (sink included), the visible softmax
    # weights plus the sink weight sum to one
    rng = np.random.default_rng(17)
    lengths = [10, 6]
    inp = _full_inputs(rng, lengths)
    _, lse = oracle_mod.sink_attn_fwd(**inp, window=4, use_rope=True)
    qh = oracle_mod.rmsnorm_rope(inp["q"], inp["cu_seqlens"], inp["qnorm_w"], use_rope=True)
    kh = oracle_mod.rmsnorm_rope(inp["k"], inp["cu_seqlens"], inp["knorm_w"], use_rope=True)
    mask = _mask_from_library(lengths, 4).numpy()
    S = np.einsum("thd,uhd->htu", qh, np.repeat(kh, 4, axis=1)) / 4.0
    S = np.where(mask[None], S, -np.inf)
    total = np.exp(S - lse[:, :, None]).sum(-1) + np.exp(inp["sinks"][:, None] - lse)
    np.testing.assert_allclose(total, 1.0, rtol=1e-13)


# ------------------------------------------------------- worked examples ---

def test_worked_example_hand_derived(oracle_mod):
    """d = 4, one document of two tokens, eps = 0, unit weights, sink 0,
    scale 1/2.  q0 = k0 = (1,1,1,1) normalise to themselves; q1 = (2,0,0,0)
    and k1 = (0,2,0,0) also have mean square 1.  v0 = e0, v1 = e1.
    Without RoPE: s00 = 2; s10 = 1; s11 = 0.
      out0 = sigmoid(2) e0,            lse0 = log(1 + e^2)
      out1 = (e e0 + e1) / (2 + e),    lse1 = log(2 + e)
    With RoPE (theta = 1e6, so pairs (0,2) and (1,3) turn by p and p/1000):
    token 1 sits at position 1, so q1 -> (2cos1, 0, 2sin1, 0) and
    k1 -> (0, 2cos(1e-3), 0, 2sin(1e-3)); s11 = 0 still and
    s10 = cos1 + sin1."""
    q = np.array([[[1, 1, 1, 1]], [[2, 0, 0, 0]]], dtype=np.float64)
    k = np.array([[[1, 1, 1, 1]], [[0, 2, 0, 0]]], dtype=np.float64)
    v = np.array([[[1, 0, 0, 0]], [[0, 1, 0, 0]]], dtype=np.float64)
    common = dict(q=q, k=k, v=v, cu_seqlens=[0, 2], sinks=[0.0], qnorm_w=np.ones(4),
                  knorm_w=np.ones(4), eps=0.0, window=-1)
    out, lse = oracle_mod.sink_attn_fwd(**common, use_rope=False)
    e = math.e
    np.testing.assert_allclose(out[0, 0], [1 / (1 + math.exp(-2)), 0, 0, 0], rtol=1e-15)
    np.testing.assert_allclose(out[1, 0], [e / (2 + e), 1 / (2 + e), 0, 0], rtol=1e-15)
    np.testing.assert_allclose(lse[0], [math.log(1 + e * e), math.log(2 + e)], rtol=1e-15)
    out, lse = oracle_mod.sink_attn_fwd(**common, use_rope=True)
    s10 = math.cos(1.0) + math.sin(1.0)
    z1 = 2 + math.exp(s10)
    np.testing.assert_allclose(out[0, 0], [1 / (1 + math.exp(-2)), 0, 0, 0], rtol=1e-15)
    np.testing.assert_allclose(out[1, 0], [math.exp(s10) / z1, 1 / z1, 0, 0], rtol=1e-14,
                               atol=1e-16)
    np.testing.assert_allclose(lse[0], [math.log(1 + e * e), math.log(z1)], rtol=1e-14)


def _closed_form(expr):
    """Evaluate a closed-form expression of the golden fixture (numbers,
    + - * / and exp, log, cos, sin, e only)."""
    import ast
    allowed = {"exp": math.exp, "log": math.log, "cos": math.cos, "sin": math.sin, "e": math.e}
    tree = ast.parse(expr, mode="eval")
    for node in ast.walk(tree):
        if isinstance(node, ast.Name) and node.id not in allowed:
            raise ValueError(f"unexpected name {node.id} in {expr!r}")
        if not isinstance(node, (ast.Expression, ast.BinOp, ast.UnaryOp, ast.Call, ast.Name,
                                 ast.Load, ast.Constant, ast.Add, ast.Sub, ast.Mult, ast.Div,
                                 ast.USub)):
            raise ValueError(f"unexpected syntax in {expr!r}")
    return float(eval(compile(tree, "<golden>", "eval"), {"__builtins__": {}}, allowed))


def test_golden_fixture(oracle_mod):
    """The stored hand-worked example under tests/golden: inputs, closed-form
    expected values and their derivation."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "worked_example_d4.json")
    with open(path) as f:
        g = json.load(f)
    for case in g["cases"]:
        out, lse = oracle_mod.sink_attn_fwd(
            q=np.array(g["q"], dtype=np.float64), k=np.array(g["k"], dtype=np.float64),
            v=np.array(g["v"], dtype=np.float64), cu_seqlens=g["cu_seqlens"],
            sinks=g["sinks"], qnorm_w=g["qnorm_w"], knorm_w=g["knorm_w"], eps=g["eps"],
            theta=g["theta"], window=case["window"], use_rope=case["use_rope"])
        exp_out = np.vectorize(_closed_form)(np.array(case["out"], dtype=object)).astype(float)
        exp_lse = np.vectorize(_closed_form)(np.array(case["lse"], dtype=object)).astype(float)
        np.testing.assert_allclose(out, exp_out, rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(lse, exp_lse, rtol=1e-14)


# ------------------------------------------------------------ edge cases ---

def test_empty_and_zero_length_documents(oracle_mod):
    z = np.zeros((0, 2, 8))
    out, lse = oracle_mod.sink_attn_fwd(q=np.zeros((0, 4, 8)), k=z, v=z, cu_seqlens=[0, 0, 0],
                                        sinks=np.zeros(4), qnorm_w=np.ones(8),
                                        knorm_w=np.ones(8), window=-1, use_rope=True)
    assert out.shape == (0, 4, 8) and lse.shape == (4, 0)


def test_row_subset_matches_full(oracle_mod):
    rng = np.random.default_rng(18)
    lengths = [20, 11]
    inp = _full_inputs(rng, lengths)
    out, lse = oracle_mod.sink_attn_fwd(**inp, window=5, use_rope=True)
    rows = np.array([0, 3, 19, 20, 30], dtype=np.int32)
    sub = dict(inp, q=inp["q"][rows])
    o2, l2 = oracle_mod.sink_attn_fwd(**sub, window=5, use_rope=True, rows=rows)
    assert np.array_equal(o2, out[rows]) and np.array_equal(l2, lse[:, rows])


def test_invalid_arguments_rejected(oracle_mod):
    rng = np.random.default_rng(19)
    inp = _full_inputs(rng, [4, 4])
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.sink_attn_fwd(**inp, window=0, use_rope=False)
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.sink_attn_fwd(**dict(inp, cu_seqlens=[0, 5, 4]), window=-1, use_rope=False)
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.sink_attn_fwd(**dict(inp, cu_seqlens=[0, 4, 9]), window=-1, use_rope=False)
