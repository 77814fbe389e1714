"""ctypes binding of libharp.so (include/harp.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch is used for device memory and the current stream.  The
functions carry the C names; tensors are passed by ``data_ptr()`` on
``torch.cuda.current_stream()`` unless a stream handle is given.

If libharp.so is missing this module raises on import: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_char_p, c_float, c_int32, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libharp.so")

HARP_OK = 0
HARP_ERR_NULL = 1
HARP_ERR_SHAPE = 2
HARP_ERR_DTYPE = 3
HARP_ERR_ALIGN = 4
HARP_ERR_WORKSPACE = 5
HARP_ERR_UNSUPPORTED = 6
HARP_ERR_HIP = 7

HARP_F32 = 0
HARP_BF16 = 1

EXPORTED = (
    "harp_rotate_in", "harp_rotate_out", "harp_deq_gemv", "harp_deq_gemv_ws",
    "harp_deq_gemv_workspace_bytes", "harp_rotate_in_deq_gemv",
    "harp_deq_gemm",
    "harp_deq_gemm_workspace_bytes", "harp_linear_workspace_bytes", "harp_linear_fused",
    "harp_linear_fused_noalloc", "harp_linear_chain", "harp_linear_chain_workspace_bytes",
    "harp_dequant",
    "harp_rotate_weight", "harp_rotate_weight_workspace_bytes", "harp_quantize_pack",
    "harp_mixed_expand", "harp_rotate_in_mixed", "harp_rotate_out_mixed",
    "harp_rotate_mixed_workspace_bytes",
    "harp_linear_fused_mixed", "harp_linear_mixed_workspace_bytes",
    "harp_status_string", "harp_last_hip_error",
)


class HarpError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{where}: {status_string(status)}"
        if status == HARP_ERR_HIP:
            msg += f" (hipError_t {hip_error})"
        super().__init__(msg)


class harp_rotation(ctypes.Structure):
    _fields_ = [("dim", c_int32), ("block", c_int32),
                ("cs", c_void_p), ("sign_bits", c_void_p),
                ("phi_codes", c_void_p), ("phi_step", c_float)]


HARP_MAX_STAGES = 16


class harp_mixed_rotation(ctypes.Structure):
    _fields_ = [("dim", c_int32), ("n_stages", c_int32), ("radix", c_int32 * HARP_MAX_STAGES),
                ("blocks", c_void_p), ("sign_bits", c_void_p)]


class harp_qweight(ctypes.Structure):
    _fields_ = [("N", c_int32), ("K", c_int32), ("bits", c_int32),
                ("group", c_int32), ("qweight", c_void_p), ("scale", c_void_p),
                ("zero", c_void_p)]


class harp_chain_layer(ctypes.Structure):
    _fields_ = [("V", harp_rotation), ("W", harp_qweight), ("U", harp_rotation),
                ("y", c_void_p)]


def _load() -> ctypes.CDLL:
    # torch first: its bundled HIP runtime (soname libamdhip64.so.7) must be
    # the one loaded, so that torch's streams and allocations and this
    # library's kernels live in a single runtime.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python rotated_bit_amd/build.py` "
            "(or __graft_entry__.build()). There is no fallback path.")
    lib = ctypes.CDLL(LIB_PATH)
    R = ctypes.POINTER(harp_rotation)
    Q = ctypes.POINTER(harp_qweight)
    MR = ctypes.POINTER(harp_mixed_rotation)
    sig = {
        "harp_rotate_in": (c_int32, [R, c_void_p, c_int32, c_void_p, c_int32, c_int32, c_void_p]),
        "harp_rotate_out": (c_int32, [R, c_void_p, c_void_p, c_int32, c_int32, c_void_p]),
        "harp_deq_gemv": (c_int32, [Q, c_void_p, c_void_p, c_int32, c_void_p]),
        "harp_deq_gemv_ws": (c_int32, [Q, c_void_p, c_void_p, c_int32, c_void_p, c_size_t,
                                       c_void_p]),
        "harp_deq_gemv_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
        "harp_rotate_in_deq_gemv": (c_int32, [R, Q, c_void_p, c_int32, c_void_p, c_int32,
                                               c_void_p]),
        "harp_deq_gemm": (c_int32, [Q, c_void_p, c_void_p, c_int32, c_void_p, c_size_t,
                                    c_void_p]),
        "harp_deq_gemm_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
        "harp_linear_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
        "harp_linear_fused": (c_int32, [R, Q, R, c_void_p, c_int32, c_void_p, c_int32,
                                        c_int32, c_void_p, c_size_t, c_void_p]),
        "harp_linear_fused_noalloc": (c_int32, [R, Q, R, c_void_p, c_int32, c_void_p, c_int32,
                                                c_int32, c_void_p]),
        "harp_linear_chain": (c_int32, [ctypes.POINTER(harp_chain_layer), c_int32, c_void_p,
                                        c_int32, c_int32, c_int32, c_void_p, c_size_t,
                                        c_void_p]),
        "harp_linear_chain_workspace_bytes": (c_size_t, [c_int32]),
        "harp_dequant": (c_int32, [Q, c_void_p, c_int32, c_void_p]),
        "harp_rotate_weight": (c_int32, [R, R, c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                                          c_size_t, c_void_p]),
        "harp_rotate_weight_workspace_bytes": (c_size_t, [c_int32, c_int32]),
        "harp_mixed_expand": (c_int32, [c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
        "harp_rotate_in_mixed": (c_int32, [MR, c_void_p, c_int32, c_void_p, c_int32, c_int32,
                                            c_void_p, c_size_t, c_void_p]),
        "harp_rotate_out_mixed": (c_int32, [MR, c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                                             c_size_t, c_void_p]),
        "harp_rotate_mixed_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
        "harp_linear_fused_mixed": (c_int32, [MR, Q, MR, c_void_p, c_int32, c_void_p, c_int32,
                                              c_int32, c_void_p, c_size_t, c_void_p]),
        "harp_linear_mixed_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
        "harp_quantize_pack": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                          c_void_p, c_void_p]),
        "harp_status_string": (c_char_p, [c_int32]),
        "harp_last_hip_error": (c_int32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.harp_status_string(status).decode()


# ---------------------------------------------------------------------------
# torch-facing marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _dtype_of(dtype) -> int:
    torch = _torch()
    if dtype == torch.float32:
        return HARP_F32
    if dtype == torch.bfloat16:
        return HARP_BF16
    raise TypeError(f"unsupported dtype {dtype} (float32 or bfloat16)")


def _dtype_code(t) -> int:
    return _dtype_of(t.dtype)


def _stream(stream):
    if stream is None:
        return c_void_p(_torch().cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return c_void_p(stream)
    return c_void_p(stream.cuda_stream)


def _check(status: int, where: str):
    if status != HARP_OK:
        raise HarpError(status, where, lib.harp_last_hip_error())


class Rotation:
    """One side: sign_bits int32/uint32 [ceil(dim/32)] and the angles, either
    cs float32 [dim/b][log2 b][b/2][2] (cos t, sin t) or, with cs None,
    phi_codes int8 [dim/b][log2 b][b/2] and phi_step (t = pi/4 + code*step)."""

    def __init__(self, cs, sign_bits, dim: int, block: int, phi_codes=None,
                 phi_step: float = 0.0):
        self.cs, self.sign_bits, self.dim, self.block = cs, sign_bits, dim, block
        self.phi_codes, self.phi_step = phi_codes, phi_step
        self.c = harp_rotation(dim, block, None if cs is None else cs.data_ptr(),
                               sign_bits.data_ptr(),
                               None if phi_codes is None else phi_codes.data_ptr(),
                               float(phi_step))


class MixedRotation:
    """A mixed-radix side: blocks float32 (stages concatenated, stage t
    [dim/b_t][b_t][b_t] row-major), sign_bits int32/uint32 [ceil(dim/32)]."""

    def __init__(self, blocks, sign_bits, radices):
        radices = [int(b) for b in radices]
        if len(radices) > HARP_MAX_STAGES:
            raise ValueError("too many stages")
        self.blocks, self.sign_bits, self.radices = blocks, sign_bits, radices
        self.dim = 1
        for b in radices:
            self.dim *= b
        arr = (c_int32 * HARP_MAX_STAGES)(*(radices + [0] * (HARP_MAX_STAGES - len(radices))))
        self.c = harp_mixed_rotation(self.dim, len(radices), arr, blocks.data_ptr(),
                                     sign_bits.data_ptr())


class QWeight:
    """Packed weight: qweight int32 [N][K*bits/32], scale/zero int16 or fp16 [N][K/64]."""

    def __init__(self, qweight, scale, zero, N: int, K: int, bits: int, group: int = 64):
        self.qweight, self.scale, self.zero = qweight, scale, zero
        self.N, self.K, self.bits, self.group = N, K, bits, group
        self.c = harp_qweight(N, K, bits, group, qweight.data_ptr(),
                              scale.data_ptr(), zero.data_ptr())


def harp_rotate_in(V: Rotation, x, xt, M: int | None = None, stream=None) -> None:
    M = x.shape[0] if M is None else M
    _check(lib.harp_rotate_in(ctypes.byref(V.c), _ptr(x), _dtype_code(x), _ptr(xt),
                              _dtype_code(xt), M, _stream(stream)), "harp_rotate_in")


def harp_rotate_out(U: Rotation, yt, y, M: int | None = None, stream=None) -> None:
    M = yt.shape[0] if M is None else M
    _check(lib.harp_rotate_out(ctypes.byref(U.c), _ptr(yt), _ptr(y), _dtype_code(y), M,
                               _stream(stream)), "harp_rotate_out")


def harp_deq_gemv(W: QWeight, xt, yt, M: int | None = None, stream=None) -> None:
    M = xt.shape[0] if M is None else M
    _check(lib.harp_deq_gemv(ctypes.byref(W.c), _ptr(xt), _ptr(yt), M, _stream(stream)),
           "harp_deq_gemv")


def harp_deq_gemv_ws(W: QWeight, xt, yt, workspace=None, M: int | None = None,
                     stream=None) -> None:
    M = xt.shape[0] if M is None else M
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.harp_deq_gemv_ws(ctypes.byref(W.c), _ptr(xt), _ptr(yt), M, _ptr(workspace),
                                ws_bytes, _stream(stream)), "harp_deq_gemv_ws")


def harp_deq_gemv_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib.harp_deq_gemv_workspace_bytes(M, N, K))


def harp_rotate_in_deq_gemv(V: Rotation, W: QWeight, x, yt, M: int | None = None,
                            stream=None) -> None:
    M = x.shape[0] if M is None else M
    _check(lib.harp_rotate_in_deq_gemv(ctypes.byref(V.c), ctypes.byref(W.c), _ptr(x),
                                       _dtype_code(x), _ptr(yt), M, _stream(stream)),
           "harp_rotate_in_deq_gemv")


def harp_deq_gemm(W: QWeight, xt_bf16, yt, workspace=None, M: int | None = None,
                  stream=None) -> None:
    M = xt_bf16.shape[0] if M is None else M
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.harp_deq_gemm(ctypes.byref(W.c), _ptr(xt_bf16), _ptr(yt), M,
                             _ptr(workspace), ws_bytes, _stream(stream)), "harp_deq_gemm")


def harp_deq_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib.harp_deq_gemm_workspace_bytes(M, N, K))


def harp_linear_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib.harp_linear_workspace_bytes(M, N, K))


def harp_linear_fused(V: Rotation, W: QWeight, U: Rotation, x, y, workspace,
                      M: int | None = None, stream=None) -> None:
    M = x.shape[0] if M is None else M
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.harp_linear_fused(ctypes.byref(V.c), ctypes.byref(W.c), ctypes.byref(U.c),
                                 _ptr(x), _dtype_code(x), _ptr(y), _dtype_code(y), M,
                                 _ptr(workspace), ws_bytes, _stream(stream)),
           "harp_linear_fused")


def harp_linear_fused_noalloc(V: Rotation, W: QWeight, U: Rotation, x, y,
                              M: int | None = None, stream=None) -> None:
    M = x.shape[0] if M is None else M
    _check(lib.harp_linear_fused_noalloc(ctypes.byref(V.c), ctypes.byref(W.c), ctypes.byref(U.c),
                                         _ptr(x), _dtype_code(x), _ptr(y), _dtype_code(y), M,
                                         _stream(stream)),
           "harp_linear_fused_noalloc")


def harp_linear_chain_workspace_bytes(dim: int) -> int:
    return int(lib.harp_linear_chain_workspace_bytes(dim))


def harp_linear_chain(layers, x, workspace, M: int | None = None, stream=None) -> None:
    """layers: sequence of (V, W, U, y) with y the layer's output tensor
    [M][dim] (float32 or bfloat16, the same for every layer)."""
    layers = list(layers)
    M = x.shape[0] if M is None else M
    arr = (harp_chain_layer * max(1, len(layers)))()
    y_dt = HARP_F32
    for i, (V, W, U, y) in enumerate(layers):
        arr[i] = harp_chain_layer(V.c, W.c, U.c, y.data_ptr())
        y_dt = _dtype_code(y)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.harp_linear_chain(arr, len(layers), _ptr(x), _dtype_code(x), y_dt, M,
                                 _ptr(workspace), ws_bytes, _stream(stream)),
           "harp_linear_chain")


def harp_dequant(W: QWeight, out, stream=None) -> None:
    _check(lib.harp_dequant(ctypes.byref(W.c), _ptr(out), _dtype_code(out), _stream(stream)),
           "harp_dequant")


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def harp_rotate_mixed_workspace_bytes(dim: int, M: int, out_dtype) -> int:
    return int(lib.harp_rotate_mixed_workspace_bytes(dim, M, _dtype_of(out_dtype)))


def harp_mixed_expand(radices, params, gaussians=None):
    """Host expansion of a mixed-radix side (numpy in, numpy out).

    params: per stage an array of shape (dim / b_t, b_t (b_t - 1) / 2);
    gaussians: per stage a (b_t, b_t) array for radices that are not powers
    of two (None entries, or None, for powers of two).  Returns the float32
    blocks, stages concatenated, ready for MixedRotation.
    """
    import numpy as np
    radices = [int(b) for b in radices]
    dim = 1
    for b in radices:
        dim *= b
    rad = np.ascontiguousarray(radices, dtype=np.int32)
    p = np.ascontiguousarray(np.concatenate([np.asarray(a, dtype=np.float64).ravel()
                                             for a in params]))
    gl = [np.asarray(g, dtype=np.float64).ravel()
          for g, b in zip(gaussians or [None] * len(radices), radices)
          if b & (b - 1) and g is not None]
    g = np.ascontiguousarray(np.concatenate(gl)) if gl else None
    out = np.empty(dim * sum(radices), dtype=np.float32)
    _check(lib.harp_mixed_expand(len(radices), rad.ctypes.data, p.ctypes.data,
                                 None if g is None else g.ctypes.data, out.ctypes.data),
           "harp_mixed_expand")
    return out


def harp_rotate_in_mixed(R: MixedRotation, x, xt, workspace=None, M: int | None = None,
                         stream=None) -> None:
    M = x.shape[0] if M is None else M
    wp, wb = _ws(workspace)
    _check(lib.harp_rotate_in_mixed(ctypes.byref(R.c), _ptr(x), _dtype_code(x), _ptr(xt),
                                    _dtype_code(xt), M, wp, wb, _stream(stream)),
           "harp_rotate_in_mixed")


def harp_rotate_out_mixed(R: MixedRotation, yt, y, workspace=None, M: int | None = None,
                          stream=None) -> None:
    M = yt.shape[0] if M is None else M
    wp, wb = _ws(workspace)
    _check(lib.harp_rotate_out_mixed(ctypes.byref(R.c), _ptr(yt), _ptr(y), _dtype_code(y), M,
                                     wp, wb, _stream(stream)), "harp_rotate_out_mixed")


def harp_linear_mixed_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib.harp_linear_mixed_workspace_bytes(M, N, K))


def harp_linear_fused_mixed(V: MixedRotation, W: QWeight, U: MixedRotation, x, y, workspace,
                            M: int | None = None, stream=None) -> None:
    M = x.shape[0] if M is None else M
    wp, wb = _ws(workspace)
    _check(lib.harp_linear_fused_mixed(ctypes.byref(V.c), ctypes.byref(W.c), ctypes.byref(U.c),
                                       _ptr(x), _dtype_code(x), _ptr(y), _dtype_code(y), M,
                                       wp, wb, _stream(stream)), "harp_linear_fused_mixed")


def harp_rotate_weight_workspace_bytes(N: int, K: int) -> int:
    return int(lib.harp_rotate_weight_workspace_bytes(N, K))


def harp_rotate_weight(V: Rotation, U: Rotation, W, Wp, workspace, stream=None) -> None:
    """Wp = F_U W F_V^T for W, Wp float32 [N][K]."""
    N, K = W.shape
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.harp_rotate_weight(ctypes.byref(V.c), ctypes.byref(U.c), _ptr(W), _ptr(Wp), N, K,
                                  _ptr(workspace), ws_bytes, _stream(stream)),
           "harp_rotate_weight")


def harp_quantize_pack(Wp, bits: int, qweight, scale, zero, stream=None) -> None:
    """Quantize float32 Wp [N][K] into qweight [N][K*bits/32] and fp16-bit
    scale / zero [N][K/64] (int32 / int16 tensors)."""
    N, K = Wp.shape
    _check(lib.harp_quantize_pack(_ptr(Wp), N, K, bits, _ptr(qweight), _ptr(scale), _ptr(zero),
                                  _stream(stream)), "harp_quantize_pack")


def harp_last_hip_error() -> int:
    return int(lib.harp_last_hip_error())
