"""The C ABI without a GPU: every declared symbol is exported, the workspace
query is pure host arithmetic, and every invalid argument is rejected on the
host with its status code before any HIP call (so these run on a CPU-only
machine).  Rejecting what cannot be consumed, instead of falling back, follows
flint.layers _validate_backend and attention.utils (ValueError on a layout a
backend cannot consume)."""
import ctypes

import pytest

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, ELAUNCH, ESCRATCH = 0, -1, -2, -3, -4, -5


@pytest.fixture(scope="module")
def A():
    import os
    import attention_qk_rmsnorm_amd as A
    if not os.path.exists(A.library_path()):
        from attention_qk_rmsnorm_amd.build import build
        build()
    return A


def test_every_declared_symbol_is_exported(A):
    lib = A.load_library()
    names = A.header_functions()
    assert set(names) >= {"sink_attn_fwd", "sink_attn_workspace_bytes",
                          "sink_attn_status_string", "sink_attn_prologue",
                          "sink_attn_attention", "sink_attn_version", "sink_attn_tile_config",
                          "sink_attn_bwd", "sink_attn_bwd_workspace_bytes", "sink_attn_fwd_padded",
                          "sink_attn_bwd_padded", "sink_attn_mask_to_seqlens",
                          "sink_attn_fwd_noalloc"}
    for n in names:
        assert hasattr(lib, n), n


def test_descriptor_layout_matches_header(A):
    # 8 int32, 3 doubles, pointer, size_t
    assert ctypes.sizeof(A.SinkAttnDesc) == 8 * 4 + 3 * 8 + 8 + 8
    assert A.SinkAttnDesc.rms_eps.offset == 32
    assert A.SinkAttnDesc.workspace.offset == 56


def test_status_strings(A):
    for code in (OK, EINVAL, EUNSUPPORTED, EWORKSPACE, ELAUNCH, ESCRATCH, 12345):
        s = A.status_string(code)
        assert isinstance(s, str) and s
    assert A.status_string(12345) == "unknown status"


def _desc(A, T=256, D=2, Hq=32, Hkv=4, d=128, dtype=0, ws_bytes=None, **kw):
    desc = A.make_desc(T, D, Hq, Hkv, d, dtype, **kw)
    need = A.workspace_bytes(desc)
    desc.workspace = 0x10000000 if need else None
    desc.workspace_bytes = need if ws_bytes is None else ws_bytes
    return desc


def test_workspace_bytes(A):
    assert A.sink_attn_workspace_bytes(0, 0, 32, 4, 128) == 0
    a = A.sink_attn_workspace_bytes(1000, 3, 32, 4, 128)
    b = A.sink_attn_workspace_bytes(100000, 3, 32, 4, 128)
    assert 0 < a < b and a % 256 == 0 and b % 256 == 0
    # k_hat + V^T for 4 kv heads over keys padded to 64 dominate
    assert b >= 2 * 4 * 100032 * 128 * 2
    assert A.sink_attn_workspace_bytes(128, 1, 4, 1, 64, A.SINK_ATTN_F32) > 0
    assert A.load_library().sink_attn_workspace_bytes(None) == 0
    assert A.sink_attn_workspace_bytes(100, 1, 32, 5, 128) == 0     # invalid: 32 % 5


FAKE = 0x7f0000000000   # 256-byte aligned, never dereferenced: the checks fail first


def _fwd(A, desc, window=-1, use_rope=0, q=FAKE, k=FAKE, v=FAKE, cu=FAKE, sinks=FAKE,
         qw=FAKE, kw=FAKE, out=FAKE, lse=FAKE):
    lib = A.load_library()
    P = ctypes.c_void_p
    return lib.sink_attn_fwd(ctypes.byref(desc) if desc is not None else None, P(q), P(k),
                             P(v), P(cu), P(sinks), P(qw), P(kw), window, use_rope, P(out),
                             P(lse), None)


@pytest.mark.parametrize("case, expected", [
    ("null_desc", EINVAL),
    ("window_zero", EINVAL),
    ("use_rope_two", EINVAL),
    ("heads_not_divisible", EINVAL),
    ("negative_tokens", EINVAL),
    ("tokens_without_docs", EINVAL),
    ("tile_config_4", EINVAL),
    ("tile_config_negative", EINVAL),
    ("negative_eps", EINVAL),
    ("theta_zero", EINVAL),
    ("nan_scale", EINVAL),
    ("null_q", EINVAL),
    ("null_out", EINVAL),
    ("null_cu", EINVAL),
    ("null_sinks", EINVAL),
    ("misaligned_q", EINVAL),
    ("misaligned_out", EINVAL),
    ("head_dim_96", EUNSUPPORTED),
    ("bf16_head_dim_64", EUNSUPPORTED),
    ("group_3", EUNSUPPORTED),
    ("group_64", EUNSUPPORTED),
    ("dtype_7", EUNSUPPORTED),
    ("no_workspace", EWORKSPACE),
    ("small_workspace", EWORKSPACE),
    ("misaligned_workspace", EWORKSPACE),
])
def test_invalid_arguments_rejected_before_any_launch(A, case, expected):
    kwargs = {}
    desc = _desc(A)
    if case == "null_desc":
        desc = None
    elif case == "window_zero":
        kwargs["window"] = 0
    elif case == "use_rope_two":
        kwargs["use_rope"] = 2
    elif case == "heads_not_divisible":
        desc = _desc(A, Hq=30, Hkv=4, ws_bytes=1 << 30)
    elif case == "negative_tokens":
        desc = _desc(A, T=-5)
    elif case == "tokens_without_docs":
        desc = _desc(A, D=0, ws_bytes=1 << 30)
    elif case == "tile_config_4":
        desc.tile_config = 4
    elif case == "tile_config_negative":
        desc.tile_config = -1
    elif case == "negative_eps":
        desc.rms_eps = -1.0
    elif case == "theta_zero":
        desc.rope_theta = 0.0
    elif case == "nan_scale":
        desc.softmax_scale = float("nan")
    elif case == "null_q":
        kwargs["q"] = 0
    elif case == "null_out":
        kwargs["out"] = 0
    elif case == "null_cu":
        kwargs["cu"] = 0
    elif case == "null_sinks":
        kwargs["sinks"] = 0
    elif case == "misaligned_q":
        kwargs["q"] = FAKE + 2
    elif case == "misaligned_out":
        kwargs["out"] = FAKE + 8
    elif case == "head_dim_96":
        desc = _desc(A, d=96, ws_bytes=1 << 30)
    elif case == "bf16_head_dim_64":
        desc = _desc(A, d=64, ws_bytes=1 << 30)
    elif case == "group_3":
        desc = _desc(A, Hq=12, Hkv=4, ws_bytes=1 << 30)
    elif case == "group_64":
        desc = _desc(A, Hq=64, Hkv=1, ws_bytes=1 << 30)
    elif case == "dtype_7":
        desc = _desc(A, dtype=7, ws_bytes=1 << 30)
    elif case == "no_workspace":
        desc.workspace = None
    elif case == "small_workspace":
        desc.workspace_bytes -= 256
    elif case == "misaligned_workspace":
        desc.workspace = 0x10000000 + 128
    assert _fwd(A, desc, **kwargs) == expected


def test_stage_entry_points_validate_too(A):
    lib = A.load_library()
    P = ctypes.c_void_p
    desc = _desc(A)
    assert lib.sink_attn_attention(ctypes.byref(desc), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 0,
                                   0, P(FAKE), P(FAKE), None) == EINVAL
    assert lib.sink_attn_prologue(ctypes.byref(desc), P(FAKE), P(0), P(FAKE), P(FAKE), 0,
                                  None) == EINVAL
    small = _desc(A, ws_bytes=1024)
    assert lib.sink_attn_prologue(ctypes.byref(small), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 1,
                                  None) == EWORKSPACE


def test_empty_batch_is_a_no_op(A):
    # T == 0: nothing to compute, nothing launched, no workspace needed
    desc = _desc(A, T=0, D=0)
    assert desc.workspace_bytes == 0
    assert _fwd(A, desc, q=0, k=0, v=0, sinks=0, qw=0, kw=0, out=0, lse=0) == OK
    desc = _desc(A, T=0, D=3)
    assert _fwd(A, desc, q=0, k=0, v=0, sinks=0, qw=0, kw=0, out=0, lse=0) == OK


@pytest.mark.parametrize("T, D, window, expected", [
    (32768, 1, -1, 2),      # one long causal document: wide tiles
    (131072, 2, 4096, 2),   # long documents, 4096-key window: wide
    (12450, 8, 1024, 1),    # 1024-key window: narrow
    (111378, 512, -1, 1),   # short documents: narrow
    (8192, 1, 1024, 1),     # long document, 1024-key window: 960 keys, narrow
    (32768, 1, 1536, 2),    # long document, 1536-key window: 1500 keys, wide
    (4096, 2, -1, 2),       # two 2048-token causal documents: wide (1024 keys)
    (4094, 2, -1, 1),       # just under: narrow
    (1024, 1, 2048, 1),     # window past the document: causal estimate (512 keys)
])
def test_automatic_tile_choice(A, T, D, window, expected):
    assert A.sink_attn_tile_config(T, D, 32, 4, 128, window) == expected


def test_forced_tile_choice_and_fp32(A):
    assert A.sink_attn_tile_config(100, 1, 32, 4, 128, -1, tile_config=A.SINK_ATTN_TILE_WIDE) == 2
    assert A.sink_attn_tile_config(10 ** 6, 1, 32, 4, 128, -1,
                                   tile_config=A.SINK_ATTN_TILE_NARROW) == 1
    assert A.sink_attn_tile_config(128, 1, 4, 1, 64, -1, dtype=A.SINK_ATTN_F32) == 0
    with pytest.raises(A.SinkAttnError):
        A.sink_attn_tile_config(128, 1, 32, 4, 128, 0)
    assert A.sink_attn_tile_config(100, 1, 32, 4, 128, -1, tile_config=3) == 3
    with pytest.raises(A.SinkAttnError):
        A.sink_attn_tile_config(128, 1, 32, 4, 128, -1, tile_config=5)


def test_bwd_workspace_bytes(A):
    assert A.sink_attn_bwd_workspace_bytes(0, 0, 32, 4, 128) == 0
    assert A.sink_attn_bwd_workspace_bytes(128, 1, 4, 1, 64, A.SINK_ATTN_F32) == 0
    assert A.sink_attn_bwd_workspace_bytes(100, 1, 32, 5, 128) == 0     # invalid: 32 % 5
    assert A.load_library().sink_attn_bwd_workspace_bytes(None) == 0
    a = A.sink_attn_bwd_workspace_bytes(1000, 3, 32, 4, 128)
    T = 32768
    b = A.sink_attn_bwd_workspace_bytes(T, 1, 32, 4, 128)
    assert 0 < a < b and a % 256 == 0 and b % 256 == 0
    # per kv head: 32 KiB per 64 keys, 16.25 KiB per 32 query columns (4 tokens at G = 8)
    images = 4 * (T // 64) * 32 * 1024 + 4 * (T // 4) * (16 * 1024 + 256)
    assert images <= b < 1.05 * images


def _bwd(A, desc, window=-1, use_rope=0, **ptrs):
    names = ["q", "k", "v", "cu", "sinks", "qw", "kw", "out", "lse", "dout", "dq", "dk", "dv",
             "dsinks", "dqw", "dkw"]
    p = {n: FAKE for n in names}
    p.update(ptrs)
    P = ctypes.c_void_p
    a = [P(p[n]) for n in names]
    return A.load_library().sink_attn_bwd(ctypes.byref(desc) if desc is not None else None,
                                          *a[:7], window, use_rope, *a[7:], None)


def _bwd_desc(A, **kw):
    desc = _desc(A, **kw)
    need = A.bwd_workspace_bytes(desc)
    desc.workspace = 0x10000000 if need else None
    desc.workspace_bytes = need
    return desc


@pytest.mark.parametrize("case, expected", [
    ("null_desc", EINVAL), ("window_zero", EINVAL), ("use_rope_two", EINVAL),
    ("null_lse", EINVAL), ("null_dout", EINVAL), ("null_dq", EINVAL), ("null_dsinks", EINVAL),
    ("null_dknorm_w", EINVAL), ("misaligned_dk", EINVAL), ("misaligned_lse", EINVAL),
    ("fp32", EUNSUPPORTED), ("group_3", EUNSUPPORTED), ("no_workspace", EWORKSPACE),
    ("fwd_sized_workspace", EWORKSPACE), ("misaligned_workspace", EWORKSPACE),
])
def test_bwd_invalid_arguments_rejected(A, case, expected):
    desc = _bwd_desc(A)
    kw = {}
    if case == "null_desc":
        desc = None
    elif case == "window_zero":
        kw["window"] = 0
    elif case == "use_rope_two":
        kw["use_rope"] = 2
    elif case.startswith("null_"):
        kw[{"null_dknorm_w": "dkw"}.get(case, case[5:])] = 0
    elif case == "misaligned_dk":
        kw["dk"] = FAKE + 4
    elif case == "misaligned_lse":
        kw["lse"] = FAKE + 2
    elif case == "fp32":
        desc = _desc(A, dtype=1, ws_bytes=1 << 30)
    elif case == "group_3":
        desc = _desc(A, Hq=12, Hkv=4, ws_bytes=1 << 30)
    elif case == "no_workspace":
        desc.workspace = None
    elif case == "fwd_sized_workspace":
        desc.workspace_bytes = A.workspace_bytes(desc)
    elif case == "misaligned_workspace":
        desc.workspace = 0x10000000 + 64
    assert _bwd(A, desc, **kw) == expected


def _padded_fwd(A, desc, cu_padded=FAKE, window=-1, **ptrs):
    names = ["q", "k", "v", "cu", "sinks", "qw", "kw", "out", "lse"]
    p = {n: FAKE for n in names}
    p.update(ptrs)
    P = ctypes.c_void_p
    return A.load_library().sink_attn_fwd_padded(
        ctypes.byref(desc), P(p["q"]), P(p["k"]), P(p["v"]), P(p["cu"]), P(cu_padded),
        P(p["sinks"]), P(p["qw"]), P(p["kw"]), window, 0, P(p["out"]), P(p["lse"]), None)


def test_padded_entry_points_validate(A):
    desc = _desc(A)
    assert _padded_fwd(A, desc, cu_padded=0) == EINVAL          # padded boundaries required
    assert _padded_fwd(A, desc, cu_padded=FAKE + 2) == EINVAL   # misaligned
    assert _padded_fwd(A, desc, window=0) == EINVAL
    small = _desc(A, ws_bytes=1024)
    assert _padded_fwd(A, small) == EWORKSPACE
    lib = A.load_library()
    P = ctypes.c_void_p
    bdesc = _bwd_desc(A)
    args = [P(FAKE)] * 4 + [P(0)] + [P(FAKE)] * 3
    tail = [-1, 0] + [P(FAKE)] * 9 + [None]
    assert lib.sink_attn_bwd_padded(ctypes.byref(bdesc), *args, *tail) == EINVAL
    # the workspace query covers the document-end table the padded calls keep
    assert A.sink_attn_workspace_bytes(1000, 3, 32, 4, 128) < \
        A.sink_attn_workspace_bytes(1000, 300, 32, 4, 128)


def test_mask_to_seqlens_validates(A):
    lib = A.load_library()
    P = ctypes.c_void_p
    assert lib.sink_attn_mask_to_seqlens(P(FAKE), -1, 4, P(FAKE), P(FAKE), P(FAKE), None) == EINVAL
    assert lib.sink_attn_mask_to_seqlens(P(0), 2, 4, P(FAKE), P(FAKE), P(FAKE), None) == EINVAL
    assert lib.sink_attn_mask_to_seqlens(P(FAKE), 2, 4, P(0), P(FAKE), P(FAKE), None) == EINVAL
    assert lib.sink_attn_mask_to_seqlens(P(FAKE), 1 << 16, 1 << 16, P(FAKE), P(FAKE), P(FAKE),
                                         None) == EINVAL


def test_fp16_descriptor(A):
    # the fp16 I/O variant shares the bf16 layout: same workspaces, same
    # tile rule, same shape limits; the backward accepts it too
    f16 = A.SINK_ATTN_F16
    for args in ((12450, 8), (32768, 1), (111378, 512)):
        assert A.sink_attn_workspace_bytes(*args, 32, 4, 128, dtype=f16) == \
            A.sink_attn_workspace_bytes(*args, 32, 4, 128)
        assert A.sink_attn_bwd_workspace_bytes(*args, 32, 4, 128, dtype=f16) == \
            A.sink_attn_bwd_workspace_bytes(*args, 32, 4, 128)
    assert A.sink_attn_tile_config(32768, 1, 32, 4, 128, -1, dtype=f16) == 2
    assert A.sink_attn_tile_config(12450, 8, 32, 4, 128, 1024, dtype=f16) == 1
    assert _fwd(A, _desc(A, dtype=f16, d=64, ws_bytes=1 << 30)) == EUNSUPPORTED
    assert _fwd(A, _desc(A, dtype=f16, Hq=12, Hkv=4, ws_bytes=1 << 30)) == EUNSUPPORTED
    assert _fwd(A, _desc(A, dtype=f16), q=FAKE + 8) == EINVAL   # 16-byte alignment
    assert _fwd(A, _desc(A, dtype=f16, ws_bytes=1024)) == EWORKSPACE


def _noalloc(A, desc, window=-1, **ptrs):
    names = ["q", "k", "v", "cu", "sinks", "qw", "kw", "out", "lse"]
    p = {n: FAKE for n in names}
    p.update(ptrs)
    P = ctypes.c_void_p
    return A.load_library().sink_attn_fwd_noalloc(
        ctypes.byref(desc) if desc is not None else None, P(p["q"]), P(p["k"]), P(p["v"]),
        P(p["cu"]), P(p["sinks"]), P(p["qw"]), P(p["kw"]), window, 0, P(p["out"]),
        P(p["lse"]), None)


def test_noalloc_entry_point_validates_before_any_hip_call(A):
    # the no-alloc forward ignores the descriptor's workspace, checks every
    # argument as sink_attn_fwd does, and rejects a call whose workspace would
    # exceed the library's scratch array -- all before touching the device
    limit = A.NOALLOC_SCRATCH_BYTES
    import os
    import re
    with open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "include", "sink_attn.h")) as f:
        m = re.search(r"#define SINK_ATTN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)",
                      f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == limit
    fits = _desc(A, T=36000, D=1)
    assert 0 < A.workspace_bytes(fits) <= limit
    too_big = _desc(A, T=45000, D=1)
    assert A.workspace_bytes(too_big) > limit
    assert _noalloc(A, too_big) == ESCRATCH
    assert "scratch" in A.status_string(ESCRATCH)
    f32 = _desc(A, T=30000, D=1, Hq=4, Hkv=4, dtype=A.SINK_ATTN_F32)
    assert A.workspace_bytes(f32) > limit and _noalloc(A, f32) == ESCRATCH
    assert _noalloc(A, None) == EINVAL
    assert _noalloc(A, _desc(A), window=0) == EINVAL
    assert _noalloc(A, _desc(A), q=0) == EINVAL
    assert _noalloc(A, _desc(A), out=FAKE + 8) == EINVAL
    assert _noalloc(A, _desc(A, d=96)) == EUNSUPPORTED
    # argument errors win over the size check
    assert _noalloc(A, too_big, cu=0) == EINVAL
    # an empty batch needs nothing and enqueues nothing
    assert _noalloc(A, _desc(A, T=0, D=0), q=0, k=0, v=0, sinks=0, qw=0, kw=0, out=0,
                    lse=0) == OK
