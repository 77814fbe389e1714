"""The C ABI on the host: libharp.so loads, exports every function that
include/harp.h declares, and rejects bad arguments with the documented
status before any HIP call (no compute call is made here; pointers are
fake but never dereferenced because every call below fails validation or
has M == 0)."""
import ctypes
import os
import re

import pytest

from rotated_bit_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "harp.h")

FAKE = 0x10000           # 256-byte aligned, never dereferenced
MISALIGNED = 0x10004


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(harp_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    decl = declared_functions()
    assert decl == sorted(L.EXPORTED)


def test_every_declared_symbol_is_exported():
    for name in declared_functions():
        assert hasattr(L.lib, name), name
        assert ctypes.cast(getattr(L.lib, name), ctypes.c_void_p).value


def rot(dim=256, block=256, cs=FAKE, sb=FAKE, codes=0, step=0.0):
    return L.harp_rotation(dim, block, cs, sb, codes, step)


def rot8(codes=FAKE, step=0.01, cs=0, **kw):
    return rot(cs=cs, codes=codes, step=step, **kw)


def qw(N=256, K=256, bits=2, group=64, q=FAKE, s=FAKE, z=FAKE):
    return L.harp_qweight(N, K, bits, group, q, s, z)


def rot_in(R, x=FAKE, xdt=0, xt=FAKE, xtdt=0, M=1):
    return L.lib.harp_rotate_in(ctypes.byref(R) if R is not None else None,
                                x, xdt, xt, xtdt, M, None)


@pytest.mark.parametrize("R,expect", [
    (rot(cs=0), L.HARP_ERR_NULL),
    (rot(sb=0), L.HARP_ERR_NULL),
    (rot(block=3), L.HARP_ERR_SHAPE),
    (rot(block=1), L.HARP_ERR_SHAPE),
    (rot(block=0), L.HARP_ERR_SHAPE),
    (rot(block=-4), L.HARP_ERR_SHAPE),
    (rot(dim=16384, block=16384), L.HARP_ERR_UNSUPPORTED),
    (rot(dim=300, block=256), L.HARP_ERR_SHAPE),
    (rot(dim=0, block=2), L.HARP_ERR_SHAPE),
    (rot(dim=262144 * 2, block=256), L.HARP_ERR_SHAPE),
    (rot(cs=MISALIGNED), L.HARP_ERR_ALIGN),
    (rot(sb=MISALIGNED), L.HARP_ERR_ALIGN),
    # int8-stored angles: exactly one angle format, a finite step
    (rot8(codes=0), L.HARP_ERR_NULL),
    (rot8(cs=FAKE), L.HARP_ERR_SHAPE),
    (rot8(step=float("nan")), L.HARP_ERR_SHAPE),
    (rot8(step=float("inf")), L.HARP_ERR_SHAPE),
    (rot8(codes=MISALIGNED), L.HARP_ERR_ALIGN),
    (rot8(sb=0), L.HARP_ERR_NULL),
    (rot8(block=3), L.HARP_ERR_SHAPE),
])
def test_rotation_checks(R, expect):
    assert rot_in(R) == expect


def test_int8_angle_rotation_accepted():
    # M = 0: passes every check and launches nothing
    assert rot_in(rot8(), x=0, xt=0, M=0) == L.HARP_OK
    assert rot_in(rot8(step=0.0), x=0, xt=0, M=0) == L.HARP_OK


def test_rotation_struct_layout():
    f = dict((n, getattr(L.harp_rotation, n)) for n, _ in L.harp_rotation._fields_)
    assert [f[n].offset for n in ("dim", "block", "cs", "sign_bits", "phi_codes", "phi_step")] \
        == [0, 4, 8, 16, 24, 32]
    assert ctypes.sizeof(L.harp_rotation) == 40


def test_rotate_in_other_checks():
    assert rot_in(None) == L.HARP_ERR_NULL
    assert rot_in(rot(), xdt=2) == L.HARP_ERR_DTYPE
    assert rot_in(rot(), xtdt=-1) == L.HARP_ERR_DTYPE
    assert rot_in(rot(), M=-1) == L.HARP_ERR_SHAPE
    assert rot_in(rot(), M=65537) == L.HARP_ERR_SHAPE
    assert rot_in(rot(), x=0) == L.HARP_ERR_NULL
    assert rot_in(rot(), xt=0) == L.HARP_ERR_NULL
    assert rot_in(rot(), x=MISALIGNED) == L.HARP_ERR_ALIGN
    # empty input: a no-op, NULL data allowed
    assert rot_in(rot(), x=0, xt=0, M=0) == L.HARP_OK


def test_rotate_out_checks():
    f = L.lib.harp_rotate_out
    R = rot()
    assert f(None, FAKE, FAKE, 0, 1, None) == L.HARP_ERR_NULL
    assert f(ctypes.byref(R), FAKE, FAKE, 5, 1, None) == L.HARP_ERR_DTYPE
    assert f(ctypes.byref(R), 0, FAKE, 0, 1, None) == L.HARP_ERR_NULL
    assert f(ctypes.byref(R), FAKE, MISALIGNED, 0, 1, None) == L.HARP_ERR_ALIGN
    assert f(ctypes.byref(R), 0, 0, 0, 0, None) == L.HARP_OK


@pytest.mark.parametrize("W,expect", [
    (qw(q=0), L.HARP_ERR_NULL),
    (qw(s=0), L.HARP_ERR_NULL),
    (qw(z=0), L.HARP_ERR_NULL),
    (qw(bits=1), L.HARP_ERR_UNSUPPORTED),
    (qw(bits=8), L.HARP_ERR_UNSUPPORTED),
    (qw(group=128), L.HARP_ERR_UNSUPPORTED),
    (qw(K=100), L.HARP_ERR_SHAPE),
    (qw(K=0), L.HARP_ERR_SHAPE),
    (qw(N=0), L.HARP_ERR_SHAPE),
    (qw(N=-5), L.HARP_ERR_SHAPE),
    (qw(q=MISALIGNED), L.HARP_ERR_ALIGN),
    (qw(s=FAKE + 2), L.HARP_ERR_ALIGN),
])
def test_qweight_checks(W, expect):
    assert L.lib.harp_deq_gemv(ctypes.byref(W), FAKE, FAKE, 1, None) == expect
    assert L.lib.harp_deq_gemm(ctypes.byref(W), FAKE, FAKE, 1, FAKE, 1 << 30, None) == expect
    assert L.lib.harp_dequant(ctypes.byref(W), FAKE, 0, None) == expect


def test_product_data_checks():
    W = qw()
    gemv = L.lib.harp_deq_gemv
    gemm = lambda W_, x, y, M: L.lib.harp_deq_gemm(W_, x, y, M, None, 0, None)
    for f in (lambda W_, x, y, M: gemv(W_, x, y, M, None), gemm):
        assert f(None, FAKE, FAKE, 1) == L.HARP_ERR_NULL
        assert f(ctypes.byref(W), 0, FAKE, 1) == L.HARP_ERR_NULL
        assert f(ctypes.byref(W), FAKE, 0, 3) == L.HARP_ERR_NULL
        assert f(ctypes.byref(W), FAKE, MISALIGNED, 3) == L.HARP_ERR_ALIGN
        assert f(ctypes.byref(W), FAKE, FAKE, -2) == L.HARP_ERR_SHAPE
        assert f(ctypes.byref(W), 0, 0, 0) == L.HARP_OK
    # split-K workspace: optional, but when given it must be aligned and big
    W4 = qw(N=4096, K=4096)
    need = L.harp_deq_gemm_workspace_bytes(512, 4096, 4096)
    assert need > 0
    g = L.lib.harp_deq_gemm
    assert g(ctypes.byref(W4), FAKE, FAKE, 512, FAKE + 16, need, None) == L.HARP_ERR_ALIGN
    assert g(ctypes.byref(W4), FAKE, FAKE, 512, FAKE, need - 1, None) == L.HARP_ERR_WORKSPACE
    assert g(ctypes.byref(W4), 0, FAKE, 512, FAKE, need, None) == L.HARP_ERR_NULL
    assert L.lib.harp_dequant(ctypes.byref(W), 0, 0, None) == L.HARP_ERR_NULL
    assert L.lib.harp_dequant(ctypes.byref(W), FAKE, 3, None) == L.HARP_ERR_DTYPE


def test_deq_gemv_ws_checks():
    """harp_deq_gemv_ws: harp_deq_gemv's checks, then (a workspace given)
    alignment and size; the size query is 0 where the FP4 product does not
    apply."""
    gw = L.lib.harp_deq_gemv_ws
    W = qw()
    assert gw(None, FAKE, FAKE, 1, None, 0, None) == L.HARP_ERR_NULL
    assert gw(ctypes.byref(W), 0, FAKE, 1, None, 0, None) == L.HARP_ERR_NULL
    assert gw(ctypes.byref(W), FAKE, MISALIGNED, 3, None, 0, None) == L.HARP_ERR_ALIGN
    assert gw(ctypes.byref(W), FAKE, FAKE, -2, None, 0, None) == L.HARP_ERR_SHAPE
    assert gw(ctypes.byref(W), 0, 0, 0, FAKE + 16, 0, None) == L.HARP_OK
    big = qw(N=28672, K=8192)
    need = L.harp_deq_gemv_workspace_bytes(1, 28672, 8192)
    assert need > 0
    assert gw(ctypes.byref(big), FAKE, FAKE, 1, FAKE + 16, need, None) == L.HARP_ERR_ALIGN
    assert gw(ctypes.byref(big), FAKE, FAKE, 1, FAKE, need - 1, None) == L.HARP_ERR_WORKSPACE
    assert gw(ctypes.byref(big), 0, FAKE, 1, FAKE, need, None) == L.HARP_ERR_NULL


def test_deq_gemv_workspace_bytes():
    """Counter area (2048 bytes), then planes (1 KB per 128 inputs), scale
    bytes (64 per 128 inputs), group sums (4 per 64 inputs, to a 256-byte
    boundary) and, with split K, slices x N float32 partials."""
    g = L.harp_deq_gemv_workspace_bytes
    C = 2048
    up = (8192 // 128) * 1088 + 8192 // 64 * 4          # 70144, already 256-aligned
    # 28672 x 8192: 1792 row tiles, one K slice (no partials)
    assert g(1, 28672, 8192) == C + up
    # 8192 x 28672: 512 tiles; 2048 waves want 4 slices (56 steps each <= 64)
    down = (28672 // 128) * 1088 + 28672 // 64 * 4
    assert g(1, 8192, 28672) == C + (down + 255) // 256 * 256 + 4 * 8192 * 4
    # 4096 x 34816: 256 tiles -> 8 slices of 17 step pairs
    k = 34816
    assert g(1, 4096, k) == C + ((k // 128) * 1088 + k // 64 * 4 + 255) // 256 * 256 \
        + 8 * 4096 * 4
    # below 2^27 weights, more than one row, ragged N or K: none
    assert g(1, 8192, 8192) == 0
    assert g(2, 28672, 8192) == 0
    assert g(1, 28680, 8192) == 0
    assert g(1, 28672, 8320) == 0
    assert g(0, 28672, 8192) == 0 and g(-1, 28672, 8192) == 0


def test_workspace_bytes():
    f = L.harp_linear_workspace_bytes
    g = L.harp_deq_gemm_workspace_bytes
    C = 2048   # the GEMM split-K counters, always first (fixed offset for every shape)
    # M < 64: float32 x~, then y'
    assert f(1, 4096, 4096) == C + 4096 * 4 + 4096 * 4
    assert f(15, 100, 64) == C + 3840 + 6144     # 15*100*4 = 6000 rounds up to 6144
    assert f(63, 100, 64) == C + 16128 + 25344   # 63*64*4; 25200 -> 25344
    # M = 64: bf16 x~, y', and the small-batch product needs no workspace
    assert g(64, 4096, 4096) == 0 and g(16, 4096, 4096) == 0
    assert f(64, 4096, 4096) == C + 64 * 4096 * 2 + 64 * 4096 * 4
    # M=65, 4096x4096: 32 tiles of 128x128 -> 4 K slices (8 groups each at
    # least): counters, then partials 4*32*128*128*4 bytes
    assert g(65, 4096, 4096) == C + 4 * 32 * 128 * 128 * 4
    assert f(65, 4096, 4096) == C + (65 * 4096 * 2 + 255) // 256 * 256 + 65 * 4096 * 4 \
        + 4 * 32 * 128 * 128 * 4
    # M=512, 4096x4096: 128 tiles -> 2 slices fill 256 CUs; 12288 outputs:
    # 384 tiles -> 2 slices fill three rounds of 256 (one slice: 1.5 rounds)
    assert g(512, 4096, 4096) == C + 2 * 128 * 128 * 128 * 4
    assert g(512, 12288, 4096) == C + 2 * 384 * 128 * 128 * 4
    # 1024 tiles fill four rounds unsplit
    assert g(1024, 16384, 4096) == 0
    # K of 64 (one group) cannot be split
    assert g(512, 256, 64) == 0
    assert f(0, 4096, 4096) == 0
    assert f(-1, 4096, 4096) == 0
    assert f(1, 0, 4096) == 0
    assert g(1, 4096, 32) == 0


def fused(V, W, U, x=FAKE, xdt=1, y=FAKE, ydt=0, M=1, ws=FAKE, wsb=1 << 30):
    b = lambda s: ctypes.byref(s) if s is not None else None
    return L.lib.harp_linear_fused(b(V), b(W), b(U), x, xdt, y, ydt, M, ws, wsb, None)


def test_fused_checks():
    V, U = rot(dim=256), rot(dim=512, block=256)
    W = qw(N=512, K=256)
    assert fused(None, W, U) == L.HARP_ERR_NULL
    assert fused(V, None, U) == L.HARP_ERR_NULL
    assert fused(V, W, None) == L.HARP_ERR_NULL
    assert fused(V, qw(N=512, K=512), U) == L.HARP_ERR_SHAPE          # V.dim != K
    assert fused(V, qw(N=256, K=256), U) == L.HARP_ERR_SHAPE          # U.dim != N
    assert fused(V, W, U, xdt=9) == L.HARP_ERR_DTYPE
    assert fused(V, W, U, ydt=9) == L.HARP_ERR_DTYPE
    assert fused(V, W, U, M=70000) == L.HARP_ERR_SHAPE
    assert fused(V, W, U, x=0) == L.HARP_ERR_NULL
    assert fused(V, W, U, ws=0) == L.HARP_ERR_WORKSPACE
    assert fused(V, W, U, ws=FAKE + 16) == L.HARP_ERR_ALIGN
    need = L.harp_linear_workspace_bytes(1, 512, 256)
    assert fused(V, W, U, wsb=need - 1) == L.HARP_ERR_WORKSPACE
    assert fused(V, W, U, x=0, y=0, ws=0, wsb=0, M=0) == L.HARP_OK
    assert fused(V, qw(N=512, K=256, bits=5), U) == L.HARP_ERR_UNSUPPORTED


def test_status_strings():
    for s in range(8):
        assert L.status_string(s).startswith("HARP_")
    assert "unknown" in L.status_string(42)
    assert L.harp_last_hip_error() == 0


def test_builder_loads_without_the_package():
    """build() must work on a tree with no library yet: loading the builder
    may not import the package (whose import loads the library)."""
    import subprocess
    import sys
    code = ("import sys, __graft_entry__ as g; m = g._builder(); "
            "assert callable(m.build); assert 'rotated_bit_amd' not in sys.modules")
    subprocess.run([sys.executable, "-c", code], check=True, cwd=ROOT)


def test_rotate_in_deq_gemv_checks():
    f = L.lib.harp_rotate_in_deq_gemv
    V, W = rot(), qw()

    def call(V=V, W=W, x=FAKE, xdt=0, yt=FAKE, M=1):
        return f(ctypes.byref(V) if V is not None else None,
                 ctypes.byref(W) if W is not None else None, x, xdt, yt, M, None)

    assert call(V=None) == L.HARP_ERR_NULL
    assert call(W=None) == L.HARP_ERR_NULL
    assert call(V=rot(dim=512, block=256)) == L.HARP_ERR_SHAPE      # V.dim != K
    assert call(xdt=3) == L.HARP_ERR_DTYPE
    assert call(M=-1) == L.HARP_ERR_SHAPE
    assert call(x=0) == L.HARP_ERR_NULL
    assert call(yt=MISALIGNED) == L.HARP_ERR_ALIGN
    assert call(x=0, yt=0, M=0) == L.HARP_OK
    # outside the single-launch shapes
    assert call(M=5) == L.HARP_ERR_UNSUPPORTED
    assert call(V=rot(dim=256, block=4)) == L.HARP_ERR_UNSUPPORTED
    assert call(V=rot(dim=8192, block=256), W=qw(K=8192)) == L.HARP_ERR_UNSUPPORTED


def test_rotate_weight_checks():
    f = L.lib.harp_rotate_weight
    V, U = rot(dim=256), rot(dim=512, block=256)
    need = L.harp_rotate_weight_workspace_bytes(512, 256)
    assert need == 512 * 256 * 4
    b = lambda s: ctypes.byref(s) if s is not None else None

    def call(V=V, U=U, W=FAKE, Wp=FAKE, N=512, K=256, ws=FAKE, wsb=need):
        return f(b(V), b(U), W, Wp, N, K, ws, wsb, None)

    assert call(V=None) == L.HARP_ERR_NULL
    assert call(U=None) == L.HARP_ERR_NULL
    assert call(K=512) == L.HARP_ERR_SHAPE                 # V.dim != K
    assert call(N=256) == L.HARP_ERR_SHAPE                 # U.dim != N
    assert call(N=0) == L.HARP_ERR_SHAPE
    assert call(W=0) == L.HARP_ERR_NULL
    assert call(ws=0) == L.HARP_ERR_NULL
    assert call(Wp=MISALIGNED) == L.HARP_ERR_ALIGN
    assert call(ws=FAKE + 16) == L.HARP_ERR_ALIGN
    assert call(wsb=need - 1) == L.HARP_ERR_WORKSPACE
    assert L.harp_rotate_weight_workspace_bytes(0, 256) == 0
    assert L.harp_rotate_weight_workspace_bytes(70000, 256) == 0


def test_quantize_pack_checks():
    f = L.lib.harp_quantize_pack

    def call(Wp=FAKE, N=4, K=128, bits=2, q=FAKE, s=FAKE, z=FAKE):
        return f(Wp, N, K, bits, q, s, z, None)

    assert call(bits=5) == L.HARP_ERR_UNSUPPORTED
    assert call(bits=1) == L.HARP_ERR_UNSUPPORTED
    assert call(K=100) == L.HARP_ERR_SHAPE
    assert call(K=0) == L.HARP_ERR_SHAPE
    assert call(N=0) == L.HARP_ERR_SHAPE
    assert call(Wp=0) == L.HARP_ERR_NULL
    assert call(z=0) == L.HARP_ERR_NULL
    assert call(q=MISALIGNED) == L.HARP_ERR_ALIGN


def mixed(dim=40, radices=(8, 5), blocks=FAKE, sb=FAKE, n=None):
    arr = (ctypes.c_int32 * L.HARP_MAX_STAGES)(*(list(radices) + [0] * (16 - len(radices))))
    return L.harp_mixed_rotation(dim, len(radices) if n is None else n, arr, blocks, sb)


@pytest.mark.parametrize("R,expect", [
    (mixed(blocks=0), L.HARP_ERR_NULL),
    (mixed(sb=0), L.HARP_ERR_NULL),
    (mixed(n=0), L.HARP_ERR_SHAPE),
    (mixed(n=17), L.HARP_ERR_SHAPE),
    (mixed(dim=40, radices=(8, 1, 5)), L.HARP_ERR_SHAPE),
    (mixed(dim=65 * 2, radices=(65, 2)), L.HARP_ERR_UNSUPPORTED),
    (mixed(dim=41), L.HARP_ERR_SHAPE),                       # product 40
    (mixed(dim=65536, radices=(64, 64, 16)), L.HARP_ERR_UNSUPPORTED),
    (mixed(blocks=MISALIGNED), L.HARP_ERR_ALIGN),
])
def test_mixed_rotation_checks(R, expect):
    assert L.lib.harp_rotate_in_mixed(ctypes.byref(R), FAKE, 0, FAKE, 0, 1, None, 0, None) == expect


def test_mixed_rotation_other_checks():
    R = mixed()
    f_in, f_out = L.lib.harp_rotate_in_mixed, L.lib.harp_rotate_out_mixed
    assert f_in(None, FAKE, 0, FAKE, 0, 1, None, 0, None) == L.HARP_ERR_NULL
    assert f_in(ctypes.byref(R), FAKE, 7, FAKE, 0, 1, None, 0, None) == L.HARP_ERR_DTYPE
    assert f_in(ctypes.byref(R), FAKE, 0, FAKE, 0, -2, None, 0, None) == L.HARP_ERR_SHAPE
    assert f_in(ctypes.byref(R), 0, 0, FAKE, 0, 1, None, 0, None) == L.HARP_ERR_NULL
    assert f_in(ctypes.byref(R), 0, 0, 0, 0, 0, None, 0, None) == L.HARP_OK
    assert f_out(ctypes.byref(R), FAKE, FAKE, 9, 1, None, 0, None) == L.HARP_ERR_DTYPE
    assert f_out(ctypes.byref(R), FAKE, MISALIGNED, 0, 1, None, 0, None) == L.HARP_ERR_ALIGN
    assert f_out(ctypes.byref(R), 0, 0, 0, 0, None, 0, None) == L.HARP_OK


def test_mixed_rotation_workspace():
    """bf16 outputs may bring a float32 workspace of M * dim floats; float32
    outputs need none (a given one is ignored)."""
    ws_bytes = L.lib.harp_rotate_mixed_workspace_bytes
    assert ws_bytes(40, 3, L.HARP_BF16) == 512            # 3 * 40 * 4 = 480, 256-aligned
    assert ws_bytes(5120, 512, L.HARP_BF16) == 5120 * 512 * 4
    assert ws_bytes(40, 3, L.HARP_F32) == 0
    assert ws_bytes(1, 3, L.HARP_BF16) == 0                # out of range: 0
    assert ws_bytes(40, -1, L.HARP_BF16) == 0
    assert ws_bytes(40, 0, L.HARP_BF16) == 0
    R = mixed()
    f_in, f_out = L.lib.harp_rotate_in_mixed, L.lib.harp_rotate_out_mixed
    bf = L.HARP_BF16
    assert f_in(ctypes.byref(R), FAKE, 0, FAKE, bf, 3, FAKE, 511, None) == L.HARP_ERR_WORKSPACE
    assert f_out(ctypes.byref(R), FAKE, FAKE, bf, 3, FAKE, 0, None) == L.HARP_ERR_WORKSPACE
    assert f_in(ctypes.byref(R), FAKE, 0, FAKE, bf, 3, MISALIGNED, 512, None) == L.HARP_ERR_ALIGN
    assert f_in(ctypes.byref(R), 0, 0, 0, bf, 0, FAKE, 0, None) == L.HARP_OK


def test_linear_mixed_workspace_bytes():
    f = L.lib.harp_linear_mixed_workspace_bytes
    C = 2048   # the GEMM split-K counters, always first
    # M = 1: float32 x~ (20480), y' (20480), bf16-output stage buffer (20480)
    assert f(1, 5120, 5120) == C + 3 * 20480
    # M = 16: float32 x~ (the operand, split into bf16 planes by the product),
    # y', output buffer
    assert f(16, 5120, 5120) == C + 327680 + 327680 + 327680
    # M = 100: float32 stage buffer and bf16 x~ of the input, y', output
    # buffer, then the GEMM's split-K partials (4 slices of 40 tiles)
    assert f(100, 5120, 5120) == C + 4 * 2048000 - 1024000 + 4 * 40 * 128 * 128 * 4
    assert f(1, 5120, 32) == 0            # K < 64
    assert f(-1, 5120, 5120) == 0
    assert f(1, 40000, 5120) == 0         # beyond the mixed-radix maximum


def test_linear_fused_mixed_checks():
    V, U = mixed(dim=320, radices=(8, 8, 5)), mixed(dim=40, radices=(8, 5))
    W = qw(N=40, K=320)
    b = ctypes.byref
    f = L.lib.harp_linear_fused_mixed
    need = L.lib.harp_linear_mixed_workspace_bytes(2, 40, 320)
    assert f(None, b(W), b(U), FAKE, 0, FAKE, 0, 2, FAKE, need, None) == L.HARP_ERR_NULL
    assert f(b(V), b(qw(N=40, K=256)), b(U), FAKE, 0, FAKE, 0, 2, FAKE, need, None) == \
        L.HARP_ERR_SHAPE                                   # V->dim != K
    assert f(b(V), b(W), b(V), FAKE, 0, FAKE, 0, 2, FAKE, need, None) == L.HARP_ERR_SHAPE
    assert f(b(V), b(W), b(U), FAKE, 5, FAKE, 0, 2, FAKE, need, None) == L.HARP_ERR_DTYPE
    assert f(b(V), b(W), b(U), FAKE, 0, FAKE, 0, 2, None, 0, None) == L.HARP_ERR_WORKSPACE
    assert f(b(V), b(W), b(U), FAKE, 0, FAKE, 0, 2, FAKE, need - 1, None) == \
        L.HARP_ERR_WORKSPACE
    assert f(b(V), b(W), b(U), FAKE, 0, FAKE, 0, 2, FAKE + 16, need, None) == L.HARP_ERR_ALIGN
    assert f(b(V), b(W), b(U), 0, 0, 0, 0, 0, None, 0, None) == L.HARP_OK
