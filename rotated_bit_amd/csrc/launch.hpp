// Internal kernel launchers (C++ linkage, not exported).  Arguments have
// already been validated by harp_api.cpp when these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/harp.h"

namespace harp {

// xt = F x (transpose == false) or y = F^T y' (transpose == true) for M rows.
hipError_t launch_rotate(const harp_rotation& R, const void* in, int in_dt,
                         void* out, int out_dt, int M, bool transpose,
                         hipStream_t stream);

// Mixed-radix side: xt = F x or y = F^T y' for M rows (one workgroup per row).
// x~ = F x into bf16 for M rows, with M x dim floats of scratch for the
// float32 intermediate of the two-launch form (b = 4096 / 8192, M <= 64);
// other shapes run launch_rotate.
hipError_t launch_rotate_in_scratch(const harp_rotation& R, const void* in, int in_dt,
                                    uint16_t* out, float* scratch, int M,
                                    hipStream_t stream);
hipError_t launch_rotate_mixed(const harp_mixed_rotation& R, const void* in, int in_dt,
                               void* out, int out_dt, int M, bool transpose,
                               float* workspace, hipStream_t stream);

// yt = w_hat xt on the vector ALUs, float32.
hipError_t launch_gemv(const harp_qweight& W, const float* xt, float* yt,
                       int M, hipStream_t stream);

// yt = w_hat (F_V x) in one launch: every workgroup rotates x itself.  For
// small batches and input sides only (gemv_rotated_supported).
constexpr int kDecodeRotMaxM = 4;
constexpr int kDecodeRotMaxK = 4096;
bool gemv_rotated_supported(const harp_rotation& V, const harp_qweight& W, int M);
hipError_t launch_gemv_rotated(const harp_rotation& V, const harp_qweight& W,
                               const void* x, int x_dt, float* yt, int M,
                               hipStream_t stream);

// yt = bf16(w_hat) xt_bf16 on the matrix cores, float32 accumulation, in
// `splits` K slices (splits > 1 needs the GEMM workspace, zero-filled
// before its first use and left zero-filled).
hipError_t launch_gemm(const harp_qweight& W, const uint16_t* xt, float* yt,
                       int M, int splits, void* workspace, hipStream_t stream);

// The same product for 1 <= M <= 64 with one workgroup per 16 output
// features (no workspace, no tiles).
hipError_t launch_gemm_skinny(const harp_qweight& W, const uint16_t* xt, float* yt,
                              int M, hipStream_t stream);

// Offline preparation: out [C][R] = in [R][C]^T (float32), and the packed
// uniform grid of a float32 weight [N][K] (qweight, scale, zero in the
// harp_qweight layout).
hipError_t launch_transpose(const float* in, float* out, int R, int C, hipStream_t stream);
hipError_t launch_quantize_pack(const float* wp, int N, int K, int bits, uint32_t* qw,
                                uint16_t* sc, uint16_t* zr, hipStream_t stream);

// Dense w_hat [N][K], float32 or bf16.
hipError_t launch_dequant(const harp_qweight& W, void* out, int out_dt,
                          hipStream_t stream);

}  // namespace harp
