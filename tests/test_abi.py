"""C ABI checks that need no GPU: the library loads, exports every function
declared in include/bca.h, and rejects bad arguments on the host before any
launch (fake device pointers are never dereferenced on these paths)."""
import ctypes
import os
import re

import pytest

from block_causal_transformer_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bca.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


@pytest.fixture(scope="module")
def lib():
    return ops.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(ops.EXPORTED) == set(names), names
    raw = ctypes.CDLL(ops.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), "libbca.so does not export %s" % n


def test_version_and_status_strings(lib):
    assert ops.bca_abi_version() == ops.ABI_VERSION
    assert ops.bca_status_string(0) == "BCA_OK"
    assert ops.bca_status_string(1) == "BCA_ERR_INVALID_ARG"
    assert ops.bca_status_string(2) == "BCA_ERR_UNSUPPORTED"
    assert ops.bca_status_string(3) == "BCA_ERR_HIP"
    assert ops.bca_status_string(99) == "BCA_UNKNOWN_STATUS"


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation


def good_shape(**kw):
    d = dict(B=1, T=4, N=10, Hq=4, Hkv=2, D=64, dtype=ops.BCA_BF16)
    d.update(kw)
    return ops.BcaShape(d["B"], d["T"], d["N"], d["Hq"], d["Hkv"], d["D"], d["dtype"])


def fwd_call(op, shape, mask, ptrs=None):
    p = ptrs or [FAKE] * 5
    f = ops.space_attn_fwd if op == "space" else ops.time_attn_fwd
    return f(shape, mask, *p)


def bwd_call(op, shape, mask, ptrs=None, ws=None, ws_bytes=0):
    p = ptrs or [FAKE] * 9
    f = ops.space_attn_bwd if op == "space" else ops.time_attn_bwd
    return f(shape, mask, *p, ws, ws_bytes)


SPACE_MASK = ops.BcaMask(0, 0, 9, 1, 0.0)
TIME_MASK = ops.BcaMask(1, 3, 0, 0, 0.0)


@pytest.mark.parametrize("field,value", [("B", 0), ("T", -1), ("N", 0), ("Hq", 0), ("Hkv", 0), ("D", 0)])
def test_non_positive_sizes(lib, field, value):
    for op, m in (("space", SPACE_MASK), ("time", TIME_MASK)):
        assert fwd_call(op, good_shape(**{field: value}), m) == ops.BCA_ERR_INVALID_ARG
        assert bwd_call(op, good_shape(**{field: value}), m) == ops.BCA_ERR_INVALID_ARG
        assert "size" in ops.bca_last_error()


def test_group_divisibility(lib):
    assert fwd_call("space", good_shape(Hq=5, Hkv=2), SPACE_MASK) == ops.BCA_ERR_INVALID_ARG
    assert "multiple" in ops.bca_last_error()


@pytest.mark.parametrize("D", [16, 48, 128])
def test_unsupported_head_dim(lib, D):
    assert fwd_call("space", good_shape(D=D), SPACE_MASK) == ops.BCA_ERR_UNSUPPORTED
    assert bwd_call("time", good_shape(D=D), TIME_MASK) == ops.BCA_ERR_UNSUPPORTED


def test_unknown_dtype(lib):
    assert fwd_call("space", good_shape(dtype=7), SPACE_MASK) == ops.BCA_ERR_UNSUPPORTED


def test_null_and_misaligned_pointers(lib):
    for i in range(5):
        p = [FAKE] * 5
        p[i] = 0
        assert fwd_call("space", good_shape(), SPACE_MASK, p) == ops.BCA_ERR_INVALID_ARG
        assert "NULL" in ops.bca_last_error()
        p[i] = FAKE + 8
        assert fwd_call("time", good_shape(), TIME_MASK, p) == ops.BCA_ERR_INVALID_ARG
        assert "aligned" in ops.bca_last_error()
    for i in range(9):
        p = [FAKE] * 9
        p[i] = 0
        assert bwd_call("space", good_shape(), SPACE_MASK, p) == ops.BCA_ERR_INVALID_ARG


def test_mask_descriptor_rules(lib):
    s = good_shape()
    # space op: no causality, no window
    assert fwd_call("space", s, ops.BcaMask(1, 0, 0, 0, 0.0)) == ops.BCA_ERR_UNSUPPORTED
    assert fwd_call("space", s, ops.BcaMask(0, 4, 0, 0, 0.0)) == ops.BCA_ERR_UNSUPPORTED
    # time op must be causal
    assert fwd_call("time", s, ops.BcaMask(0, 4, 0, 0, 0.0)) == ops.BCA_ERR_UNSUPPORTED
    # window < 0
    assert fwd_call("time", s, ops.BcaMask(1, -1, 0, 0, 0.0)) == ops.BCA_ERR_INVALID_ARG
    # agent range outside [0, N]
    for ab, ac in ((-1, 1), (9, 2), (0, -1), (11, 0)):
        assert fwd_call("space", s, ops.BcaMask(0, 0, ab, ac, 0.0)) == ops.BCA_ERR_INVALID_ARG
    # non-finite scale
    assert fwd_call("space", s, ops.BcaMask(0, 0, 0, 0, float("nan"))) == ops.BCA_ERR_INVALID_ARG
    assert fwd_call("space", s, ops.BcaMask(0, 0, 0, 0, float("inf"))) == ops.BCA_ERR_INVALID_ARG
    assert fwd_call("space", None, SPACE_MASK) == ops.BCA_ERR_INVALID_ARG


def test_workspace_query_and_check(lib):
    # one key block per problem (at most 320 positions): the fused MFMA
    # backward and the short kernels need no workspace
    assert ops.bca_bwd_workspace_bytes(ops.BCA_OP_SPACE, good_shape(N=290)) == 0
    assert ops.bca_bwd_workspace_bytes(ops.BCA_OP_TIME, good_shape(T=256)) == 0
    assert ops.bca_bwd_workspace_bytes(ops.BCA_OP_SPACE, good_shape(N=320)) == 0
    assert ops.bca_bwd_workspace_bytes(ops.BCA_OP_TIME, good_shape(T=16, N=1432, Hq=16, Hkv=16)) == 0
    # longer problems: one fp32 Delta per (query, head)
    assert ops.bca_bwd_workspace_bytes(ops.BCA_OP_SPACE, good_shape(N=321)) == 1 * 4 * 321 * 4 * 4
    # ... except windowed time attention, which runs as segments of at least
    # 128 positions whose fp32 dK, dV partials (keys of the segment's range,
    # at most 320, x 128) take more: the query takes no window and returns
    # the most any window needs (segments of exactly 128 positions): 10 slots
    # x 2 KV heads x 8 segments x 320 keys x 512 bytes
    assert ops.bca_bwd_workspace_bytes(ops.BCA_OP_TIME, good_shape(T=1024)) == 10 * 2 * 8 * 320 * 512
    # at 330 frames (3 segments of 128; a segment's range is the 320 keys
    # before its end), still more than Delta's 330 * 10 * 4 * 4 bytes
    assert ops.bca_bwd_workspace_bytes(ops.BCA_OP_TIME, good_shape(T=330)) == 10 * 2 * 3 * 320 * 512
    # the space op's length is N and the time op's T
    assert ops.bca_bwd_workspace_bytes(ops.BCA_OP_TIME, good_shape(N=1432, T=8)) == 0
    # the generic VALU path (head_dim 32, fp32) always uses it
    assert ops.bca_bwd_workspace_bytes(ops.BCA_OP_SPACE, good_shape(D=32)) == 1 * 4 * 10 * 4 * 4
    s = good_shape(N=1432, T=2)
    need = ops.bca_bwd_workspace_bytes(ops.BCA_OP_SPACE, s)
    assert need == 1 * 2 * 1432 * 4 * 4
    assert ops.bca_bwd_workspace_bytes(ops.BCA_OP_SPACE, good_shape(dtype=ops.BCA_F32)) == 1 * 4 * 10 * 4 * 4
    assert ops.bca_bwd_workspace_bytes(ops.BCA_OP_SPACE, good_shape(B=0)) == 0
    assert ops.bca_bwd_workspace_bytes(5, good_shape()) == 0
    rc = bwd_call("space", s, ops.BcaMask(0, 0, 0, 0, 0.0), ws=FAKE, ws_bytes=need - 1)
    assert rc == ops.BCA_ERR_INVALID_ARG and "workspace" in ops.bca_last_error()
    rc = bwd_call("space", s, ops.BcaMask(0, 0, 0, 0, 0.0), ws=None, ws_bytes=need)
    assert rc == ops.BCA_ERR_INVALID_ARG
    # a call needs what its own window needs: with a 192-frame window the
    # segments' partials (the query's figure), unbounded causal only Delta
    t = good_shape(T=1024)
    seg = 10 * 2 * 8 * 320 * 512
    rc = bwd_call("time", t, ops.BcaMask(1, 192, 0, 0, 0.0), ws=FAKE, ws_bytes=seg - 1)
    assert rc == ops.BCA_ERR_INVALID_ARG and str(seg) in ops.bca_last_error()
    rc = bwd_call("time", t, ops.BcaMask(1, 0, 0, 0, 0.0), ws=FAKE, ws_bytes=1024 * 10 * 4 * 4 - 1)
    assert rc == ops.BCA_ERR_INVALID_ARG and str(1024 * 10 * 4 * 4) in ops.bca_last_error()
    # a window too long for segments of 128 positions: Delta
    rc = bwd_call("time", t, ops.BcaMask(1, 200, 0, 0, 0.0), ws=FAKE, ws_bytes=1024 * 10 * 4 * 4 - 1)
    assert rc == ops.BCA_ERR_INVALID_ARG and str(1024 * 10 * 4 * 4) in ops.bca_last_error()


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(ops, "_lib", None)
    with pytest.raises(RuntimeError, match="not found"):
        ops.load(str(tmp_path / "missing.so"))


def decode_call(shape, mask, cache_frames, q_frame0, ptrs=None):
    p = ptrs or [FAKE] * 5
    return ops.time_attn_decode_fwd(shape, mask, p[0], p[1], p[2], cache_frames, q_frame0, p[3], p[4])


@pytest.mark.parametrize("T,window,cache,q0,ok", [
    (1, 192, 191, 500, False),   # window 192 needs 192 cached frames
    (1, 192, 192, 500, True),
    (1, 192, 100, 99, True),     # frames 0..99 only
    (1, 192, 99, 99, False),
    (4, 8, 10, 30, False),       # 4 new frames with window 8 read 11 frames
    (4, 8, 11, 30, True),
    (2, 0, 12, 10, True),        # unbounded window: frames 0..11
    (2, 0, 11, 10, False),
])
def test_decode_cache_must_hold_every_frame_read(lib, T, window, cache, q0, ok):
    """The size check runs before any launch; valid sizes are only checked
    for the message (not called: the pointers are fake)."""
    shape = good_shape(T=T)
    mask = ops.make_mask("time", window=window)
    if ok:
        return
    assert decode_call(shape, mask, cache, q0) == ops.BCA_ERR_INVALID_ARG
    assert "cannot hold" in ops.bca_last_error()


def test_decode_rejects_bad_arguments(lib):
    shape = good_shape(T=1)
    mask = ops.make_mask("time", window=4)
    assert decode_call(shape, mask, 0, 3) == ops.BCA_ERR_INVALID_ARG
    assert decode_call(shape, mask, 4, -1) == ops.BCA_ERR_INVALID_ARG
    assert decode_call(shape, ops.make_mask("space"), 4, 3) == ops.BCA_ERR_UNSUPPORTED
    assert decode_call(shape, mask, 4, 3, [FAKE, 0, FAKE, FAKE, FAKE]) == ops.BCA_ERR_INVALID_ARG
    assert "k_cache" in ops.bca_last_error()
    assert decode_call(shape, mask, 4, 3, [FAKE, FAKE, FAKE + 8, FAKE, FAKE]) == ops.BCA_ERR_INVALID_ARG
    assert "v_cache" in ops.bca_last_error()
    assert decode_call(good_shape(T=1, D=48), mask, 4, 3) == ops.BCA_ERR_UNSUPPORTED
    assert decode_call(good_shape(T=2), mask, 8, 2 ** 31 - 1) == ops.BCA_ERR_INVALID_ARG
    assert "overflows" in ops.bca_last_error()


def proj_shape(M=300, d_model=1920, Hq=30, Hkv=3, D=64):
    return ops.BcaProjShape(M, d_model, Hq, Hkv, D)


def qkv_call(shape, eps=1e-6, ptrs=None, rstd=None, ws_bytes=None):
    p = ptrs or [FAKE] * 7
    need = ops.bca_qkv_workspace_bytes(shape) if ws_bytes is None else ws_bytes
    return ops.rmsnorm_qkv_fwd(shape, p[0], p[1], eps, p[2], p[3], p[4], p[5], rstd, p[6], need)


def test_projection_workspace_query(lib):
    # the gain-folded weights ((30 + 2 * 3) * 64 rows of 1920, 256-byte aligned),
    # then an fp32 rstd per row
    wbytes = (30 + 2 * 3) * 64 * 1920 * 2
    assert ops.bca_qkv_workspace_bytes(proj_shape()) == (wbytes + 255) // 256 * 256 + 300 * 4
    assert ops.bca_qkv_workspace_bytes(proj_shape(M=7, d_model=72, Hq=2, Hkv=1, D=8)) == \
        ((2 + 2) * 8 * 72 * 2 + 255) // 256 * 256 + 7 * 4
    assert ops.bca_qkv_workspace_bytes(proj_shape(M=0)) == 0
    assert ops.bca_qkv_workspace_bytes(proj_shape(d_model=100)) == 0
    assert ops.bca_qkv_workspace_bytes(None) == 0


@pytest.mark.parametrize("field,value", [("M", 0), ("M", -3), ("d_model", 0), ("Hq", 0),
                                         ("Hkv", -1), ("D", 0)])
def test_projection_non_positive_sizes(lib, field, value):
    s = proj_shape(**{field: value})
    assert qkv_call(s, ws_bytes=1 << 20) == ops.BCA_ERR_INVALID_ARG
    assert "non-positive" in ops.bca_last_error()
    assert ops.out_proj_fwd(s, FAKE, FAKE, None, FAKE) == ops.BCA_ERR_INVALID_ARG


def test_projection_widths_must_be_multiples_of_8(lib):
    assert qkv_call(proj_shape(d_model=1916), ws_bytes=1 << 30) == ops.BCA_ERR_UNSUPPORTED
    assert "multiples of 8" in ops.bca_last_error()
    assert ops.out_proj_fwd(proj_shape(D=60), FAKE, FAKE, None, FAKE) == ops.BCA_ERR_UNSUPPORTED


def test_projection_rejects_bad_arguments(lib):
    s = proj_shape()
    assert ops.rmsnorm_qkv_fwd(None, FAKE, FAKE, 1e-6, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30) \
        == ops.BCA_ERR_INVALID_ARG
    for eps in (-1e-3, float("nan"), float("inf")):
        assert qkv_call(s, eps=eps) == ops.BCA_ERR_INVALID_ARG
        assert "eps" in ops.bca_last_error()
    names = ("x", "gain", "w_qkv", "q", "k", "v", "workspace")
    for i, name in enumerate(names):
        p = [FAKE] * 7
        p[i] = 0
        assert qkv_call(s, ptrs=p) == ops.BCA_ERR_INVALID_ARG
        assert name in ops.bca_last_error() and "NULL" in ops.bca_last_error()
        p[i] = FAKE + 8
        assert qkv_call(s, ptrs=p) == ops.BCA_ERR_INVALID_ARG
        assert "aligned" in ops.bca_last_error()
    assert qkv_call(s, rstd=FAKE + 4) == ops.BCA_ERR_INVALID_ARG
    assert "rstd" in ops.bca_last_error()
    rc = qkv_call(s, ws_bytes=ops.bca_qkv_workspace_bytes(s) - 1)
    assert rc == ops.BCA_ERR_INVALID_ARG and "workspace" in ops.bca_last_error()
    for i, name in enumerate(("o", "w_o", "y")):
        p = [FAKE] * 3
        p[i] = 0
        assert ops.out_proj_fwd(s, p[0], p[1], None, p[2]) == ops.BCA_ERR_INVALID_ARG
        assert name in ops.bca_last_error()
    assert ops.out_proj_fwd(s, FAKE, FAKE, FAKE + 2, FAKE) == ops.BCA_ERR_INVALID_ARG
    assert "residual" in ops.bca_last_error()


def test_projection_too_large(lib):
    assert qkv_call(proj_shape(M=2 ** 40), ws_bytes=2 ** 62) == ops.BCA_ERR_INVALID_ARG
    assert "too large" in ops.bca_last_error()


def test_size_limits_of_the_kernels_are_validated(lib):
    """Shapes past the kernels' folded-row limits (G <= 256 query heads per KV
    head, fewer than 2^21 rows position * G + head per problem) are refused
    by validation with UNSUPPORTED, before any launch."""
    for op, m in (("space", ops.BcaMask(0, 0, 0, 0, 0.0)), ("time", TIME_MASK)):
        assert fwd_call(op, good_shape(Hq=257, Hkv=1), m) == ops.BCA_ERR_UNSUPPORTED
        assert "per KV head" in ops.bca_last_error()
        assert bwd_call(op, good_shape(Hq=514, Hkv=2), m) == ops.BCA_ERR_UNSUPPORTED
    # G = 256 with 2^13 positions is exactly 2^21 rows: refused; one fewer passes validation
    assert fwd_call("space", good_shape(N=8192, Hq=256, Hkv=1), ops.BcaMask(0, 0, 0, 0, 0.0)) \
        == ops.BCA_ERR_UNSUPPORTED
    assert "rows per problem" in ops.bca_last_error()
    assert fwd_call("time", good_shape(T=69906, Hq=30, Hkv=1), TIME_MASK) == ops.BCA_ERR_UNSUPPORTED
    assert bwd_call("time", good_shape(T=69906, Hq=30, Hkv=1), TIME_MASK) == ops.BCA_ERR_UNSUPPORTED
    # the workspace query returns 0 for a shape the calls refuse
    assert ops.bca_bwd_workspace_bytes(ops.BCA_OP_SPACE, good_shape(Hq=257, Hkv=1)) == 0
    # decode: the frames read times G is the per-problem row count
    shape = good_shape(T=1, Hq=256, Hkv=1)
    assert decode_call(shape, ops.make_mask("time", window=0), 9000, 8191) == ops.BCA_ERR_UNSUPPORTED
    assert "rows per problem" in ops.bca_last_error()
