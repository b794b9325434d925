"""ctypes front end of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg import this module.  The product package never does, and this
module imports nothing from the product package.

All arrays are numpy float64 / int32, C-contiguous.  Inputs are widened from
their storage dtype exactly (bf16 -> fp64 and fp32 -> fp64 are exact) by the
caller; the oracle then follows the definition in oracle.c step by step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.environ.get("SINKATTN_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True, src: str = _SRC, out: str | None = None) -> str:
    """Compile oracle.c (or another copy of it) into a shared library with
    plain gcc and OpenMP; by default into liboracle.so next to it."""
    out = out or LIB_PATH
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.oracle_rmsnorm_rope.argtypes = [I, I, P, I, I, P, P, D, D, I, P]
    lib.oracle_rmsnorm_rope.restype = I
    lib.oracle_attention.argtypes = [I, I, P, I, I, I, P, P, P, P, D, I, P, I,
                                     P, P, I]
    lib.oracle_attention.restype = I
    lib.oracle_sink_attn_fwd.argtypes = [I, I, P, I, I, I, P, P, P, P, P, P,
                                         D, D, D, I, I, P, I, P, P, I]
    lib.oracle_sink_attn_fwd.restype = I
    lib.oracle_sink_attn_bwd.argtypes = [I, I, P, I, I, I, P, P, P, P, P, P,
                                         D, D, D, I, I, P, P, P, P, P, P, P, I]
    lib.oracle_sink_attn_bwd.restype = I
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = I
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class OracleError(ValueError):
    pass


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def rmsnorm_rope(x, cu_seqlens, w, eps=1e-6, theta=1e6, use_rope=True):
    """Per-head RMSNorm then (optionally) NeoX RoPE of a THD tensor [T, H, d]."""
    x = _f64(x)
    T, H, d = x.shape
    cu = _i32(cu_seqlens)
    w = _f64(w)
    y = np.empty_like(x)
    rc = _load().oracle_rmsnorm_rope(T, len(cu) - 1, _ptr(cu), H, d, _ptr(x),
                                     _ptr(w), float(eps), float(theta),
                                     int(bool(use_rope)), _ptr(y))
    if rc:
        raise OracleError(f"oracle_rmsnorm_rope rejected its arguments ({rc})")
    return y


def attention(qh, kh, v, cu_seqlens, sinks, window=-1, scale=None, rows=None,
              nthreads=0):
    """Sink attention on already normalised/rotated rows.

    qh [n_rows, Hq, d] (rows of the listed tokens, or all T tokens),
    kh / v [T, Hkv, d].  Returns (out [n_rows, Hq, d], lse [Hq, n_rows]).
    """
    qh, kh, v = _f64(qh), _f64(kh), _f64(v)
    T, Hkv, d = kh.shape
    n_rows, Hq, _ = qh.shape
    cu = _i32(cu_seqlens)
    sinks = _f64(sinks)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.empty((n_rows, Hq, d), dtype=np.float64)
    lse = np.empty((Hq, n_rows), dtype=np.float64)
    rows_arr = None if rows is None else _i32(rows)
    rc = _load().oracle_attention(
        T, len(cu) - 1, _ptr(cu), Hq, Hkv, d, _ptr(qh), _ptr(kh), _ptr(v),
        _ptr(sinks), float(scale), int(window),
        None if rows_arr is None else _ptr(rows_arr), n_rows, _ptr(out),
        _ptr(lse), int(nthreads))
    if rc:
        raise OracleError(f"oracle_attention rejected its arguments ({rc})")
    return out, lse


def sink_attn_fwd(q, k, v, cu_seqlens, sinks, qnorm_w, knorm_w, window,
                  use_rope, eps=1e-6, theta=1e6, scale=None, rows=None,
                  nthreads=0):
    """The whole forward pass in fp64.

    q [n_rows, Hq, d] holds the raw queries of the tokens listed in rows (all
    T tokens when rows is None); k, v [T, Hkv, d].  Returns
    (out [n_rows, Hq, d], lse [Hq, n_rows]) as float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, Hkv, d = k.shape
    n_rows, Hq, _ = q.shape
    cu = _i32(cu_seqlens)
    out = np.empty((n_rows, Hq, d), dtype=np.float64)
    lse = np.empty((Hq, n_rows), dtype=np.float64)
    rows_arr = None if rows is None else _i32(rows)
    if rows_arr is None and n_rows != T:
        raise OracleError("q must hold all T tokens when rows is None")
    rc = _load().oracle_sink_attn_fwd(
        T, len(cu) - 1, _ptr(cu), Hq, Hkv, d, _ptr(q), _ptr(k), _ptr(v),
        _ptr(_f64(sinks)), _ptr(_f64(qnorm_w)), _ptr(_f64(knorm_w)),
        float(eps), float(theta), float(scale) if scale else 0.0, int(window),
        int(bool(use_rope)), None if rows_arr is None else _ptr(rows_arr),
        n_rows, _ptr(out), _ptr(lse), int(nthreads))
    if rc:
        raise OracleError(f"oracle_sink_attn_fwd rejected its arguments ({rc})")
    return out, lse


def sink_attn_bwd(q, k, v, cu_seqlens, sinks, qnorm_w, knorm_w, window, use_rope,
                  dout, eps=1e-6, theta=1e6, scale=None, nthreads=0):
    """Gradients of sum(dout * out) of the whole forward pass, in fp64.

    q, dout [T, Hq, d]; k, v [T, Hkv, d].  Returns a dict with dq, dk, dv (the
    shapes of q, k, v), dsinks [Hq], dqnorm_w and dknorm_w [d], as float64.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    T, Hkv, d = k.shape
    Hq = q.shape[1]
    if q.shape[0] != T or dout.shape != q.shape:
        raise OracleError("q and dout must be [T, Hq, d]")
    cu = _i32(cu_seqlens)
    res = {"dq": np.empty_like(q), "dk": np.empty_like(k), "dv": np.empty_like(v),
           "dsinks": np.empty(Hq), "dqnorm_w": np.empty(d), "dknorm_w": np.empty(d)}
    rc = _load().oracle_sink_attn_bwd(
        T, len(cu) - 1, _ptr(cu), Hq, Hkv, d, _ptr(q), _ptr(k), _ptr(v),
        _ptr(_f64(sinks)), _ptr(_f64(qnorm_w)), _ptr(_f64(knorm_w)),
        float(eps), float(theta), float(scale) if scale else 0.0, int(window),
        int(bool(use_rope)), _ptr(dout), _ptr(res["dq"]), _ptr(res["dk"]),
        _ptr(res["dv"]), _ptr(res["dsinks"]), _ptr(res["dqnorm_w"]),
        _ptr(res["dknorm_w"]), int(nthreads))
    if rc:
        raise OracleError(f"oracle_sink_attn_bwd rejected its arguments ({rc})")
    return res


# ---- padded THD --------------------------------------------------------------
# Padded THD (attention.utils: cu_seqlens with cu_seqlens_padded): document n's
# real tokens are [cu_padded[n], cu_padded[n] + cu[n+1] - cu[n]) of the packed
# tensors, the rest of [cu_padded[n], cu_padded[n+1]) is padding.  flint.layers
# FlintAttention.forward (attention_mask): padded queries and keys are excluded
# from the real attention and the sink stays valid.  The oracle takes that
# literally: the real tokens, gathered into an unpadded batch, go through the
# definitions above unchanged; a padding query's softmax holds the sink alone
# (out = 0, lse = sink), and no gradient reaches a padding row.

def padded_real_rows(cu_seqlens, cu_seqlens_padded) -> np.ndarray:
    """Indices of the real tokens of a padded-THD batch, in order."""
    cu = _i32(cu_seqlens)
    cp = _i32(cu_seqlens_padded)
    if cu.shape != cp.shape:
        raise OracleError("cu_seqlens and cu_seqlens_padded must have the same shape")
    parts = [np.arange(cp[n], cp[n] + (cu[n + 1] - cu[n])) for n in range(len(cu) - 1)]
    rows = np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
    for n in range(len(cu) - 1):
        if cu[n + 1] - cu[n] > cp[n + 1] - cp[n]:
            raise OracleError("a document's real tokens do not fit its padded slot")
    return rows.astype(np.int64)


def sink_attn_fwd_padded(q, k, v, cu_seqlens, cu_seqlens_padded, sinks, qnorm_w, knorm_w,
                         window, use_rope, eps=1e-6, theta=1e6, scale=None, rows=None):
    """Forward over a padded-THD batch: (out [T, Hq, d], lse [Hq, T]), or,
    when rows (padded-batch indices) is given, (out [n, Hq, d], lse [Hq, n])
    of those rows only.  q, k, v always hold all T rows."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, Hq, d = q.shape
    real = padded_real_rows(cu_seqlens, cu_seqlens_padded)
    want = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    packed = np.full(T, -1, dtype=np.int64)      # padded row -> index among the real rows
    packed[real] = np.arange(len(real))
    out = np.zeros((len(want), Hq, d))
    lse = np.repeat(_f64(sinks)[:, None], len(want), axis=1)
    hit = np.nonzero(packed[want] >= 0)[0]
    if len(hit):
        o, l = sink_attn_fwd(q[want[hit]], k[real], v[real], _i32(cu_seqlens), sinks, qnorm_w,
                             knorm_w, window, use_rope, eps=eps, theta=theta, scale=scale,
                             rows=None if rows is None else packed[want[hit]])
        out[hit] = o
        lse[:, hit] = l
    return out, lse


def sink_attn_bwd_padded(q, k, v, cu_seqlens, cu_seqlens_padded, sinks, qnorm_w, knorm_w,
                         window, use_rope, dout, eps=1e-6, theta=1e6, scale=None):
    """Gradients of sum(dout * out) for the padded-THD forward; padding rows
    of dq, dk, dv are zero (a padding row's out is the constant 0)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    rows = padded_real_rows(cu_seqlens, cu_seqlens_padded)
    res = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
           "dsinks": np.zeros(q.shape[1]), "dqnorm_w": np.zeros(q.shape[2]),
           "dknorm_w": np.zeros(q.shape[2])}
    if len(rows):
        g = sink_attn_bwd(q[rows], k[rows], v[rows], _i32(cu_seqlens), sinks, qnorm_w, knorm_w,
                          window, use_rope, dout[rows], eps=eps, theta=theta, scale=scale)
        for key in ("dq", "dk", "dv"):
            res[key][rows] = g[key]
        for key in ("dsinks", "dqnorm_w", "dknorm_w"):
            res[key] = g[key]
    return res
