"""rotated_bit_amd: MI355X (gfx950) HIP implementation of the HARP rotated
low-bit linear, y = U deq(Wq) V^T x, behind the C ABI of include/harp.h.

The Python surface is the ctypes binding in _lib (argument marshalling only);
importing this package fails if libharp.so has not been built.
"""
from ._lib import (  # noqa: F401
    HARP_BF16, HARP_F32, HarpError, MixedRotation, QWeight, Rotation, harp_dequant,
    harp_deq_gemm, harp_deq_gemm_workspace_bytes, harp_deq_gemv, harp_deq_gemv_ws,
    harp_deq_gemv_workspace_bytes, harp_last_hip_error, harp_linear_fused,
    harp_linear_fused_noalloc, harp_linear_chain, harp_linear_chain_workspace_bytes,
    harp_linear_fused_mixed, harp_mixed_expand, harp_linear_mixed_workspace_bytes, harp_linear_workspace_bytes, harp_quantize_pack, harp_rotate_in, harp_rotate_in_deq_gemv,
    harp_rotate_in_mixed, harp_rotate_mixed_workspace_bytes, harp_rotate_out, harp_rotate_out_mixed, harp_rotate_weight,
    harp_rotate_weight_workspace_bytes, lib,
    status_string,
)
