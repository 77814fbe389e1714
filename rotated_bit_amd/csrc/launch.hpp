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

// One row of 2-bit codes on the FP4 x FP8 matrix cores (gemv_f4.hip): x~
// is turned into digit planes in the f4 region (f4_region_bytes in
// validate.hpp), then the product runs in `slices` K slices (f4_slices);
// slices > 1 needs zeroed `counters` (one uint32 per 16-row tile, left
// zero) and the partials that follow the planes in the region.
// planes_ready: the planes are already in the region (launch_rotate_in_f4)
// and x~ is not read.  U non-null (gemv_f4_fold_supported): the output
// rotation is applied in the same launch, y (y_dt) is written and yt holds
// y' only as an intermediate; needs zeroed counters (one per 256 outputs,
// left zero).
hipError_t launch_gemv_f4(const harp_qweight& W, const float* xt, float* yt, uint8_t* f4,
                          uint32_t* counters, int slices, bool planes_ready,
                          hipStream_t stream, const harp_rotation* U = nullptr,
                          void* y = nullptr, int y_dt = HARP_F32);
bool gemv_f4_fold_supported(const harp_rotation& U, const harp_qweight& W, int slices);

// One row of x~ = F x at b = 256 / 4096 / 8192 finished straight into that
// product's planes in the f4 region (b = 256: one launch; b = 4096 / 8192:
// the sub-blocks into the float32 scratch, then the last three stages and
// the planes); x~ itself is not written.
bool rotate_in_f4_supported(const harp_rotation& R, int M);
hipError_t launch_rotate_in_f4(const harp_rotation& R, const void* in, int in_dt,
                               float* scratch, uint8_t* f4r, hipStream_t stream);

// The same product on the bf16 matrix cores with x~ split into exact bf16
// planes (gemv_mc.hip): kGemvMcMinM <= M <= kGemvMcMaxM, 2 or 4 bits.
hipError_t launch_gemv_mc(const harp_qweight& W, const float* xt, float* yt,
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
// `splits` K slices.  splits > 1 needs `partials` (splits x tiles float32
// tiles, no initialisation) and `counters` (one uint32 per output tile,
// zero before the call and left zero by it).
hipError_t launch_gemm(const harp_qweight& W, const uint16_t* xt, float* yt,
                       int M, int splits, float* partials, uint32_t* counters,
                       hipStream_t stream);

// The same product for 1 <= M <= 64 with one workgroup per 16 output
// features (no workspace, no tiles); w_hat enters exactly.
hipError_t launch_gemm_skinny(const harp_qweight& W, const uint16_t* xt, float* yt,
                              int M, hipStream_t stream);
// The same kernel on a float32 xt, split into two bf16 planes hi + lo
// (|xt - hi - lo| <= 2^-16 |xt|), 1 <= M <= 64.
hipError_t launch_gemm_skinny_split(const harp_qweight& W, const float* xt, float* yt,
                                    int M, hipStream_t stream);

// The same products on strips of 16 fb features per wave
// (skinny_wide.hip, fb 2 or 4), which read x~ correspondingly fewer times,
// in `splits` K slices (see skinny_wide_split in validate.hpp; splits > 1
// needs `partials`, splits x M x N floats, and zeroed `counters`, one per
// strip and row tile, left zero).  The launchers above use it without
// split K where it applies; launch_gemm_skinny_split_k with split K, on a
// float32 x~ in the caller's workspace that it splits in place first.
// xin: 0 bf16 x~, 1 float32 x~, 2 float32 x~ split in place by
// launch_split_chunks.
hipError_t launch_skinny_wide(const harp_qweight& W, const void* xt, int xin, float* yt,
                              int M, int fb, int splits, float* partials, uint32_t* counters,
                              hipStream_t stream);
// In place over n float32 values (n a multiple of 8): each 8-value chunk
// becomes its 8 bf16 hi values then its 8 bf16 lo values.
hipError_t launch_split_chunks(float* xt, size_t n, hipStream_t stream);
hipError_t launch_gemm_skinny_split_k(const harp_qweight& W, const float* xt, float* yt,
                                      int M, float* partials, uint32_t* counters,
                                      hipStream_t stream);

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
