"""Thin Python binding of libsinkattn (the C ABI of include/sink_attn.h).

Argument marshalling only: this module turns torch tensors into device
pointers and the current HIP stream, allocates outputs and the workspace with
torch when the caller does not pass them, and raises on a non-zero status.
Every step of the computation runs in the library's HIP kernels; there is no
other path.  The library must have been built (attention_qk_rmsnorm_amd.build).
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

from .build import LIB_PATH

SINK_ATTN_BF16 = 0
SINK_ATTN_F32 = 1
SINK_ATTN_F16 = 2

SINK_ATTN_TILE_AUTO = 0
SINK_ATTN_TILE_NARROW = 1
SINK_ATTN_TILE_WIDE = 2
SINK_ATTN_TILE_WIDE_EXACT = 3

_DTYPES = {torch.bfloat16: SINK_ATTN_BF16, torch.float32: SINK_ATTN_F32,
           torch.float16: SINK_ATTN_F16}


class SinkAttnDesc(ctypes.Structure):
    _fields_ = [
        ("total_tokens", ctypes.c_int32),
        ("num_docs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32),
        ("tile_config", ctypes.c_int32),
        ("rms_eps", ctypes.c_double),
        ("rope_theta", ctypes.c_double),
        ("softmax_scale", ctypes.c_double),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class SinkAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def library_path() -> str:
    """The library this process loads: libsinkattn.so next to the package, or
    another build of the same C ABI named by SINKATTN_LIBRARY."""
    return os.environ.get("SINKATTN_LIBRARY") or LIB_PATH


def load_library():
    """Load libsinkattn.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with attention_qk_rmsnorm_amd.build.build() "
            "(hipcc --offload-arch=gfx950); there is no fallback path")
    lib = ctypes.CDLL(path)
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    DP = ctypes.POINTER(SinkAttnDesc)
    lib.sink_attn_workspace_bytes.argtypes = [DP]
    lib.sink_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.sink_attn_fwd.argtypes = [DP, P, P, P, P, P, P, P, I32, I32, P, P, P]
    lib.sink_attn_fwd.restype = ctypes.c_int
    lib.sink_attn_prologue.argtypes = [DP, P, P, P, P, I32, P]
    lib.sink_attn_prologue.restype = ctypes.c_int
    lib.sink_attn_attention.argtypes = [DP, P, P, P, P, I32, I32, P, P, P]
    lib.sink_attn_attention.restype = ctypes.c_int
    lib.sink_attn_tile_config.argtypes = [DP, I32]
    lib.sink_attn_tile_config.restype = ctypes.c_int
    lib.sink_attn_fwd_noalloc.argtypes = [DP, P, P, P, P, P, P, P, I32, I32, P, P, P]
    lib.sink_attn_fwd_noalloc.restype = ctypes.c_int
    lib.sink_attn_fwd_padded.argtypes = [DP, P, P, P, P, P, P, P, P, I32, I32, P, P, P]
    lib.sink_attn_fwd_padded.restype = ctypes.c_int
    lib.sink_attn_bwd_padded.argtypes = [DP, P, P, P, P, P, P, P, P, I32, I32, P, P, P, P, P, P,
                                         P, P, P, P]
    lib.sink_attn_bwd_padded.restype = ctypes.c_int
    lib.sink_attn_mask_to_seqlens.argtypes = [P, I32, I32, P, P, P, P]
    lib.sink_attn_mask_to_seqlens.restype = ctypes.c_int
    lib.sink_attn_bwd_workspace_bytes.argtypes = [DP]
    lib.sink_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.sink_attn_bwd.argtypes = [DP, P, P, P, P, P, P, P, I32, I32, P, P, P, P, P, P, P, P, P, P]
    lib.sink_attn_bwd.restype = ctypes.c_int
    lib.sink_attn_status_string.argtypes = [ctypes.c_int]
    lib.sink_attn_status_string.restype = ctypes.c_char_p
    lib.sink_attn_version.argtypes = []
    lib.sink_attn_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().sink_attn_status_string(int(status)).decode()


def header_functions() -> list:
    """Names of the functions include/sink_attn.h declares."""
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(os.path.dirname(here), "include", "sink_attn.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^[A-Za-z_][\w \*]*?\b(sink_attn_\w+)\s*\(", text, flags=re.M)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def make_desc(total_tokens, num_docs, num_q_heads, num_kv_heads, head_dim, dtype,
              rms_eps=1e-6, rope_theta=1e6, softmax_scale=0.0, workspace=None,
              max_seqlen=0, tile_config=SINK_ATTN_TILE_AUTO) -> SinkAttnDesc:
    d = SinkAttnDesc()
    d.total_tokens = int(total_tokens)
    d.num_docs = int(num_docs)
    d.num_q_heads = int(num_q_heads)
    d.num_kv_heads = int(num_kv_heads)
    d.head_dim = int(head_dim)
    d.dtype = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    d.max_seqlen = int(max_seqlen)
    d.tile_config = int(tile_config)
    d.rms_eps = float(rms_eps)
    d.rope_theta = float(rope_theta)
    d.softmax_scale = float(softmax_scale or 0.0)
    if workspace is not None:
        d.workspace = workspace.data_ptr()
        d.workspace_bytes = workspace.numel() * workspace.element_size()
    return d


def workspace_bytes(desc: SinkAttnDesc) -> int:
    return int(load_library().sink_attn_workspace_bytes(ctypes.byref(desc)))


def tile_config(desc: SinkAttnDesc, window: int) -> int:
    """The bf16 tile configuration the attention stage uses for this call
    (SINK_ATTN_TILE_NARROW / _WIDE), 0 for fp32; raises on invalid input."""
    rc = int(load_library().sink_attn_tile_config(ctypes.byref(desc), int(window)))
    if rc < 0:
        raise SinkAttnError(rc, "sink_attn_tile_config")
    return rc


def _check_tensor(name, t, dtype, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Call:
    """Marshalled arguments of one forward call (shared by the three entry points)."""

    def __init__(self, q, k, v, cu_seqlens, sinks, qnorm_w, knorm_w, window, use_rope,
                 out=None, lse=None, *, rms_eps=1e-6, rope_theta=1e6, softmax_scale=None,
                 workspace=None, stream=None, return_lse=True, tile_config=SINK_ATTN_TILE_AUTO,
                 cu_seqlens_padded=None, library_scratch=False):
        if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
            raise ValueError("q, k, v must be THD tensors [tokens, heads, head_dim]")
        dev = q.device
        T, Hq, d = q.shape
        Hkv = k.shape[1]
        if k.shape != (T, Hkv, d) or v.shape != k.shape:
            raise ValueError("k and v must be [T, Hkv, head_dim] with q's T and head_dim")
        if q.dtype not in _DTYPES:
            raise ValueError(f"unsupported dtype {q.dtype}")
        for name, t in (("k", k), ("v", v)):
            _check_tensor(name, t, q.dtype, dev)
        _check_tensor("cu_seqlens", cu_seqlens, torch.int32, dev)
        if cu_seqlens_padded is not None:
            _check_tensor("cu_seqlens_padded", cu_seqlens_padded, torch.int32, dev)
            if cu_seqlens_padded.shape != cu_seqlens.shape:
                raise ValueError("cu_seqlens_padded must have cu_seqlens' shape")
        for name, t in (("sinks", sinks), ("qnorm_w", qnorm_w), ("knorm_w", knorm_w)):
            _check_tensor(name, t, torch.float32, dev)
        self.desc = make_desc(T, cu_seqlens.numel() - 1, Hq, Hkv, d, q.dtype, rms_eps,
                              rope_theta, softmax_scale or 0.0, tile_config=tile_config)
        self.cu_padded = cu_seqlens_padded
        # library_scratch: the call goes to sink_attn_fwd_noalloc, which works in
        # the library's own device array, so no workspace is allocated here
        need = 0 if library_scratch else workspace_bytes(self.desc)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        if workspace is not None:
            self.desc.workspace = workspace.data_ptr()
            self.desc.workspace_bytes = workspace.numel() * workspace.element_size()
        if out is None:
            out = torch.empty_like(q)
        else:
            _check_tensor("out", out, q.dtype, dev)
        if lse is None and return_lse:
            lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
        elif lse is not None:
            _check_tensor("lse", lse, torch.float32, dev)
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        elif isinstance(stream, torch.cuda.Stream):
            stream = stream.cuda_stream
        self.q, self.k, self.v, self.cu = q, k, v, cu_seqlens
        self.sinks, self.qnorm_w, self.knorm_w = sinks, qnorm_w, knorm_w
        self.window, self.use_rope = int(window), int(bool(use_rope))
        self.out, self.lse, self.workspace = out, lse, workspace
        self.stream = ctypes.c_void_p(stream)

    def fwd(self):
        lib = load_library()
        if self.cu_padded is not None:
            rc = lib.sink_attn_fwd_padded(
                ctypes.byref(self.desc), _ptr(self.q), _ptr(self.k), _ptr(self.v),
                _ptr(self.cu), _ptr(self.cu_padded), _ptr(self.sinks), _ptr(self.qnorm_w),
                _ptr(self.knorm_w), self.window, self.use_rope, _ptr(self.out), _ptr(self.lse),
                self.stream)
            if rc:
                raise SinkAttnError(rc, "sink_attn_fwd_padded")
            return
        rc = lib.sink_attn_fwd(
            ctypes.byref(self.desc), _ptr(self.q), _ptr(self.k), _ptr(self.v), _ptr(self.cu),
            _ptr(self.sinks), _ptr(self.qnorm_w), _ptr(self.knorm_w), self.window,
            self.use_rope, _ptr(self.out), _ptr(self.lse), self.stream)
        if rc:
            raise SinkAttnError(rc, "sink_attn_fwd")

    def fwd_noalloc(self):
        """The forward through sink_attn_fwd_noalloc (unpadded THD only)."""
        if self.cu_padded is not None:
            raise ValueError("sink_attn_fwd_noalloc takes unpadded THD only")
        rc = load_library().sink_attn_fwd_noalloc(
            ctypes.byref(self.desc), _ptr(self.q), _ptr(self.k), _ptr(self.v), _ptr(self.cu),
            _ptr(self.sinks), _ptr(self.qnorm_w), _ptr(self.knorm_w), self.window,
            self.use_rope, _ptr(self.out), _ptr(self.lse), self.stream)
        if rc:
            raise SinkAttnError(rc, "sink_attn_fwd_noalloc")

    def prologue(self):
        if self.cu_padded is not None:
            raise ValueError("the two-stage entry points take unpadded THD only")
        rc = load_library().sink_attn_prologue(
            ctypes.byref(self.desc), _ptr(self.k), _ptr(self.v), _ptr(self.cu),
            _ptr(self.knorm_w), self.use_rope, self.stream)
        if rc:
            raise SinkAttnError(rc, "sink_attn_prologue")

    def attention(self):
        if self.cu_padded is not None:
            raise ValueError("the two-stage entry points take unpadded THD only")
        rc = load_library().sink_attn_attention(
            ctypes.byref(self.desc), _ptr(self.q), _ptr(self.cu), _ptr(self.sinks),
            _ptr(self.qnorm_w), self.window, self.use_rope, _ptr(self.out), _ptr(self.lse),
            self.stream)
        if rc:
            raise SinkAttnError(rc, "sink_attn_attention")


def sink_attn_fwd(q, k, v, cu_seqlens, sinks, qnorm_w, knorm_w, window, use_rope,
                  out=None, lse=None, **kw):
    """Forward pass on the current stream.  Returns (out, lse); lse is None
    when return_lse=False and no lse buffer is given."""
    c = Call(q, k, v, cu_seqlens, sinks, qnorm_w, knorm_w, window, use_rope, out, lse, **kw)
    c.fwd()
    return c.out, c.lse


def sink_attn_fwd_noalloc(q, k, v, cu_seqlens, sinks, qnorm_w, knorm_w, window, use_rope,
                          out=None, lse=None, **kw):
    """Forward pass through sink_attn_fwd_noalloc: the library works in its own
    device array (SINK_ATTN_NOALLOC_SCRATCH_BYTES per device) instead of a
    workspace.  Pass out (and lse) to keep the call free of allocations; torch
    allocates them here otherwise.  Returns (out, lse)."""
    c = Call(q, k, v, cu_seqlens, sinks, qnorm_w, knorm_w, window, use_rope, out, lse,
             library_scratch=True, **kw)
    c.fwd_noalloc()
    return c.out, c.lse


NOALLOC_SCRATCH_BYTES = 80 << 20   # SINK_ATTN_NOALLOC_SCRATCH_BYTES of include/sink_attn.h


def sink_attn_prologue(q, k, v, cu_seqlens, sinks, qnorm_w, knorm_w, window, use_rope,
                       **kw) -> Call:
    """Run the first stage; returns the Call whose .attention() runs the second."""
    c = Call(q, k, v, cu_seqlens, sinks, qnorm_w, knorm_w, window, use_rope, **kw)
    c.prologue()
    return c


def sink_attn_workspace_bytes(total_tokens, num_docs, num_q_heads, num_kv_heads, head_dim,
                              dtype=torch.bfloat16) -> int:
    return workspace_bytes(make_desc(total_tokens, num_docs, num_q_heads, num_kv_heads,
                                     head_dim, dtype))


def sink_attn_tile_config(total_tokens, num_docs, num_q_heads, num_kv_heads, head_dim, window,
                          dtype=torch.bfloat16, tile_config=SINK_ATTN_TILE_AUTO) -> int:
    """Tile configuration the attention stage picks for these shapes and window."""
    return globals()["tile_config"](
        make_desc(total_tokens, num_docs, num_q_heads, num_kv_heads, head_dim, dtype,
                  tile_config=tile_config), window)


def bwd_workspace_bytes(desc: SinkAttnDesc) -> int:
    return int(load_library().sink_attn_bwd_workspace_bytes(ctypes.byref(desc)))


class BwdCall:
    """Marshalled arguments of one backward call (sink_attn_bwd)."""

    def __init__(self, q, k, v, cu_seqlens, sinks, qnorm_w, knorm_w, window, use_rope, out,
                 lse, dout, *, rms_eps=1e-6, rope_theta=1e6, softmax_scale=None,
                 workspace=None, stream=None, grads=None, cu_seqlens_padded=None,
                 tile_config=SINK_ATTN_TILE_AUTO):
        if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
            raise ValueError("q, k, v must be THD tensors [tokens, heads, head_dim]")
        if q.dtype not in (torch.bfloat16, torch.float16):
            raise ValueError("the backward takes bf16 or fp16 q, k, v, out and dout")
        dev = q.device
        T, Hq, d = q.shape
        Hkv = k.shape[1]
        if k.shape != (T, Hkv, d) or v.shape != k.shape:
            raise ValueError("k and v must be [T, Hkv, head_dim] with q's T and head_dim")
        if out.shape != q.shape or dout.shape != q.shape:
            raise ValueError("out and dout must have q's shape")
        for name, t in (("k", k), ("v", v), ("out", out), ("dout", dout)):
            _check_tensor(name, t, q.dtype, dev)
        _check_tensor("cu_seqlens", cu_seqlens, torch.int32, dev)
        if cu_seqlens_padded is not None:
            _check_tensor("cu_seqlens_padded", cu_seqlens_padded, torch.int32, dev)
            if cu_seqlens_padded.shape != cu_seqlens.shape:
                raise ValueError("cu_seqlens_padded must have cu_seqlens' shape")
        self.cu_padded = cu_seqlens_padded
        for name, t in (("sinks", sinks), ("qnorm_w", qnorm_w), ("knorm_w", knorm_w),
                        ("lse", lse)):
            _check_tensor(name, t, torch.float32, dev)
        if lse.shape != (Hq, T):
            raise ValueError("lse must be [Hq, T]")
        # tile_config: narrow / wide force the dQ kernel's small / large
        # workgroups (automatic by default)
        self.desc = make_desc(T, cu_seqlens.numel() - 1, Hq, Hkv, d, q.dtype, rms_eps,
                              rope_theta, softmax_scale or 0.0, tile_config=tile_config)
        need = bwd_workspace_bytes(self.desc)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        if workspace is not None:
            self.desc.workspace = workspace.data_ptr()
            self.desc.workspace_bytes = workspace.numel() * workspace.element_size()
        if grads is None:
            grads = {"dq": torch.empty_like(q), "dk": torch.empty_like(k),
                     "dv": torch.empty_like(v),
                     "dsinks": torch.empty(Hq, dtype=torch.float32, device=dev),
                     "dqnorm_w": torch.empty(d, dtype=torch.float32, device=dev),
                     "dknorm_w": torch.empty(d, dtype=torch.float32, device=dev)}
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        elif isinstance(stream, torch.cuda.Stream):
            stream = stream.cuda_stream
        self.args = (q, k, v, cu_seqlens, sinks, qnorm_w, knorm_w)
        self.window, self.use_rope = int(window), int(bool(use_rope))
        self.out, self.lse, self.dout = out, lse, dout
        self.grads, self.workspace = grads, workspace
        self.stream = ctypes.c_void_p(stream)

    def run(self):
        g = self.grads
        tail = (self.window, self.use_rope, _ptr(self.out), _ptr(self.lse), _ptr(self.dout),
                _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dsinks"]),
                _ptr(g["dqnorm_w"]), _ptr(g["dknorm_w"]), self.stream)
        a = [_ptr(t) for t in self.args]
        if self.cu_padded is not None:
            rc = load_library().sink_attn_bwd_padded(
                ctypes.byref(self.desc), *a[:4], _ptr(self.cu_padded), *a[4:], *tail)
            name = "sink_attn_bwd_padded"
        else:
            rc = load_library().sink_attn_bwd(ctypes.byref(self.desc), *a, *tail)
            name = "sink_attn_bwd"
        if rc:
            raise SinkAttnError(rc, name)
        return g


def sink_attn_bwd(q, k, v, cu_seqlens, sinks, qnorm_w, knorm_w, window, use_rope, out, lse,
                  dout, **kw) -> dict:
    """Backward pass on the current stream: gradients of sum(dout * out) as a
    dict with dq, dk, dv (bf16, shapes of q, k, v), dsinks [Hq], dqnorm_w and
    dknorm_w [d] (fp32).  out and lse are what the forward returned."""
    return BwdCall(q, k, v, cu_seqlens, sinks, qnorm_w, knorm_w, window, use_rope, out, lse,
                   dout, **kw).run()


def sink_attn_bwd_workspace_bytes(total_tokens, num_docs, num_q_heads, num_kv_heads, head_dim,
                                  dtype=torch.bfloat16) -> int:
    return bwd_workspace_bytes(make_desc(total_tokens, num_docs, num_q_heads, num_kv_heads,
                                         head_dim, dtype))


def mask_to_seqlens(attention_mask, stream=None):
    """Padded-THD boundaries (cu_seqlens, cu_seqlens_padded) of a BSHD
    attention mask [batch, seq] (True / nonzero = real token), computed on the
    device by sink_attn_mask_to_seqlens.  Raises ValueError when a row's
    padding does not trail (such inputs have to be packed as THD); that check
    synchronises the stream."""
    if attention_mask.dim() != 2:
        raise ValueError("attention_mask must be [batch, seq]")
    dev = attention_mask.device
    m = attention_mask
    if m.dtype == torch.bool:
        m = m.view(torch.uint8)
    if m.dtype != torch.uint8:
        raise ValueError("attention_mask must be bool or uint8")
    m = m.contiguous()
    B, S = m.shape
    cu = torch.empty(B + 1, dtype=torch.int32, device=dev)
    cu_padded = torch.empty(B + 1, dtype=torch.int32, device=dev)
    bad = torch.empty(1, dtype=torch.int32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = load_library().sink_attn_mask_to_seqlens(_ptr(m), B, S, _ptr(cu), _ptr(cu_padded),
                                                  _ptr(bad), ctypes.c_void_p(stream))
    if rc:
        raise SinkAttnError(rc, "sink_attn_mask_to_seqlens")
    if int(bad.item()):
        raise ValueError(f"{int(bad.item())} row(s) of attention_mask have padding before "
                         "real tokens; BSHD takes trailing padding only, pack such inputs "
                         "as THD")
    return cu, cu_padded


def _bshd_to_thd(x):
    if x.dim() != 4:
        raise ValueError("BSHD tensors are [batch, seq, heads, head_dim]")
    if not x.is_contiguous():
        raise ValueError("BSHD tensors must be contiguous")
    B, S, H, d = x.shape
    return x.view(B * S, H, d)


def sink_attn_fwd_bshd(q, k, v, attention_mask, sinks, qnorm_w, knorm_w, window, use_rope,
                       **kw):
    """Forward on BSHD tensors [batch, seq, heads, d] with a trailing-padding
    attention mask [batch, seq].  Returns (out [batch, seq, Hq, d],
    lse [Hq, batch, seq]); padding rows get out = 0 and lse = the sink."""
    B, S = q.shape[0], q.shape[1]
    cu, cu_padded = mask_to_seqlens(attention_mask)
    out, lse = sink_attn_fwd(_bshd_to_thd(q), _bshd_to_thd(k), _bshd_to_thd(v), cu, sinks,
                             qnorm_w, knorm_w, window, use_rope, cu_seqlens_padded=cu_padded,
                             **kw)
    return out.view(q.shape), (None if lse is None else lse.view(lse.shape[0], B, S))


def sink_attn_bwd_bshd(q, k, v, attention_mask, sinks, qnorm_w, knorm_w, window, use_rope,
                       out, lse, dout, **kw) -> dict:
    """Backward of sink_attn_fwd_bshd; dq, dk, dv come back in BSHD shapes."""
    cu, cu_padded = mask_to_seqlens(attention_mask)
    Hq = q.shape[2]
    g = sink_attn_bwd(_bshd_to_thd(q), _bshd_to_thd(k), _bshd_to_thd(v), cu, sinks, qnorm_w,
                      knorm_w, window, use_rope, _bshd_to_thd(out),
                      lse.reshape(Hq, -1), _bshd_to_thd(dout), cu_seqlens_padded=cu_padded, **kw)
    g["dq"] = g["dq"].view(q.shape)
    g["dk"] = g["dk"].view(k.shape)
    g["dv"] = g["dv"].view(v.shape)
    return g
