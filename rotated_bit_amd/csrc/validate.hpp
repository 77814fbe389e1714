// Argument checks of the C ABI.  Pure C++ with no HIP dependency, so the
// same translation unit is linked into libharp.so and into a host-only test
// built with sanitizers.  Every check runs before any HIP call.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/harp.h"

namespace harp {

harp_status check_rotation(const harp_rotation* R);
harp_status check_qweight(const harp_qweight* W);

harp_status validate_rotate_in(const harp_rotation* V, const void* x, int x_dt,
                               const void* xt, int xt_dt, int32_t M);
harp_status validate_rotate_out(const harp_rotation* U, const void* yt,
                                const void* y, int y_dt, int32_t M);
harp_status validate_gemv(const harp_qweight* W, const void* xt, const void* yt,
                          int32_t M);
harp_status validate_rotate_gemv(const harp_rotation* V, const harp_qweight* W,
                                const void* x, int x_dt, const void* yt, int32_t M);
harp_status validate_gemm(const harp_qweight* W, const void* xt, const void* yt,
                          int32_t M, const void* workspace, size_t ws_bytes);
harp_status validate_fused(const harp_rotation* V, const harp_qweight* W,
                           const harp_rotation* U, const void* x, int x_dt,
                           const void* y, int y_dt, int32_t M,
                           const void* workspace, size_t ws_bytes);
harp_status validate_dequant(const harp_qweight* W, const void* out, int out_dt);
size_t rotate_mixed_workspace_bytes(int32_t dim, int32_t M, int out_dt);
harp_status validate_rotate_mixed(const harp_mixed_rotation* R, const void* in, int in_dt,
                                  const void* out, int out_dt, int32_t M,
                                  const void* workspace, size_t ws_bytes);
harp_status validate_rotate_weight(const harp_rotation* V, const harp_rotation* U,
                                   const float* W, const float* Wp, int32_t N, int32_t K,
                                   const void* workspace, size_t ws_bytes);
harp_status validate_quantize_pack(const float* Wp, int32_t N, int32_t K, int32_t bits,
                                   const void* qweight, const void* scale, const void* zero);
size_t rotate_weight_workspace_bytes(int32_t N, int32_t K);

// Matrix-core GEMM tiling and its split over K: the number of K slices is
// chosen so that about one 128 x 128 output tile slice runs per CU (256 on
// MI355X), at most 4, each slice at least 8 quantization groups.  With
// slices > 1 the GEMM needs a workspace: per slice and tile a float32
// partial tile, then one uint32 arrival counter per tile.
constexpr int32_t kGemmTile = 128;
int32_t gemm_splits(int32_t M, int32_t N, int32_t K);
size_t gemm_workspace_bytes(int32_t M, int32_t N, int32_t K);

// Batch ranges of the products: harp_deq_gemm runs the small-batch
// matrix-core kernel (no workspace) up to kSkinnyMaxM rows and the tiled
// kernel above; the fused linear takes the float32 vector-ALU product below
// kMfmaMinM rows and the bf16 matrix-core product from there on.
constexpr int32_t kSkinnyMaxM = 64;
constexpr int32_t kMfmaMinM = 16;
// The fused linear folds the input rotation into the product launch up to
// this many rows and output features: every workgroup of the one-launch
// form rotates all rows itself, so it only pays off with few rows and at
// most one workgroup (16 features) per CU.  Beyond either limit the
// rotation runs once in its own launch (K = 4096, M = 1: N = 11008 takes
// 16.9 us in two launches against 22.3 us in one).
constexpr int32_t kFusedRotGemvMaxM = 2;
constexpr int32_t kFusedRotGemvMaxN = 4096;

// Workspace layout of the fused linear: x~, then y', then (M > kSkinnyMaxM)
// the tiled GEMM's workspace, each 256-byte aligned.  x~ is float32 below
// kMfmaMinM rows and bf16 from there on.
size_t workspace_bytes(int32_t M, int32_t N, int32_t K);
size_t workspace_yp_offset(int32_t M, int32_t K);
size_t mixed_ws_xb_offset(int32_t M, int32_t K);
size_t mixed_ws_yp_offset(int32_t M, int32_t K);
size_t mixed_ws_ys_offset(int32_t M, int32_t N, int32_t K);
size_t mixed_ws_gemm_offset(int32_t M, int32_t N, int32_t K);
size_t mixed_workspace_bytes(int32_t M, int32_t N, int32_t K);
harp_status validate_fused_mixed(const harp_mixed_rotation* V, const harp_qweight* W,
                                 const harp_mixed_rotation* U, const void* x, int x_dt,
                                 const void* y, int y_dt, int32_t M,
                                 const void* workspace, size_t ws_bytes);
size_t workspace_gemm_offset(int32_t M, int32_t N, int32_t K);

const char* status_string(harp_status s);

}  // namespace harp
