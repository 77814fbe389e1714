"""Move boundary-format numpy buffers to the GPU and wrap them for the binding.

Test-side plumbing only: no arithmetic of the method happens here.
"""
import numpy as np
import torch

import rotated_bit_amd as H
from oracle import harp_oracle as O


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def dev_rotation(rot) -> "H.Rotation":
    if rot.cs is None:
        return H.Rotation(None, dev(rot.sign_bits), rot.dim, rot.block,
                          phi_codes=dev(rot.phi_codes), phi_step=rot.phi_step)
    return H.Rotation(dev(rot.cs), dev(rot.sign_bits), rot.dim, rot.block)


def cs64(rot) -> np.ndarray:
    """The side's (cos t, sin t) pairs for the oracle: the stored float32
    pairs, or the oracle's float64 decode of int8-stored angles."""
    if rot.cs is None:
        return O.decode_angle_codes(rot.phi_codes, rot.phi_step)
    return rot.cs


def dev_qweight(w) -> "H.QWeight":
    return H.QWeight(dev(w.words), dev(w.scale), dev(w.zero), w.N, w.K, w.bits)


def dev_x(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return dev(x).view(torch.bfloat16)
    return dev(x.astype(np.float32))


def x_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """The values the device receives, decoded to float64."""
    if dtype == "bf16":
        return O.bf16_bits_to_f64(x)
    return x.astype(np.float64)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return O.bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


def scale_f16(w):
    return w.scale.view(np.float16)


def zero_f16(w):
    return w.zero.view(np.float16)


def workspace(M, N, K) -> torch.Tensor:
    """Fused-linear workspace, zero-filled (its GEMM counters start at 0)."""
    nbytes = H.harp_linear_workspace_bytes(M, N, K)
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device="cuda")


def gemm_workspace(M, N, K):
    """Split-K GEMM workspace (zero-filled), or None when one slice is used."""
    nbytes = H.harp_deq_gemm_workspace_bytes(M, N, K)
    return torch.zeros(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
