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
harp_status validate_gemv_ws(const harp_qweight* W, const void* xt, const void* yt,
                             int32_t M, const void* workspace, size_t ws_bytes);
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

// Matrix-core GEMM tiling and its split over K: the number of K slices
// (at most kGemmMaxSplits, each slice at least 8 quantization groups) is
// the one whose workgroups best fill their last round of kGemmSlots (one
// 128 x 128 tile slice per CU, 256 CUs on MI355X); tile counts above
// kGemmMaxSplitTiles run unsplit.  Split K needs a workspace: a fixed area
// of per-tile uint32 arrival counters at its front, then per slice and tile
// a float32 partial tile.  The counters sit at the same offset for every
// shape, so one zero-filled workspace serves any sequence of shapes that
// fit in it.
constexpr int32_t kGemmTile = 128;
constexpr int32_t kGemmSlots = 256;
constexpr int32_t kGemmMaxSplits = 4;
constexpr int32_t kGemmMaxSplitTiles = 512;
constexpr size_t kGemmCounterBytes = 2048;   // >= 4 * kGemmMaxSplitTiles, 256-aligned
int32_t gemm_splits(int32_t M, int32_t N, int32_t K);

// Small-batch product on wide strips (skinny_wide.hip): feature blocks of
// 16 per wave (2 or 4) and K slices.  Eligible when K is a multiple of 4096
// (every wave a whole number of eight-group blocks) and enough strips fill
// the chip.  With split K allowed (the fused linear's workspace) four blocks
// per wave read x~ half as often as two, and the K slices (each a multiple
// of 64 groups, at most 8) restore at least kGemmSlots workgroups; the
// slices' float32 partials follow y' in the workspace and use the GEMM's
// arrival counters.  fb == 0: the 16-feature kernel runs.
struct WideSplit {
  int32_t fb;
  int32_t splits;
};
WideSplit skinny_wide_split(int32_t M, int32_t N, int32_t K, bool allow_split);
size_t skinny_partial_bytes(int32_t M, int32_t N, int32_t K);
size_t gemm_workspace_bytes(int32_t M, int32_t N, int32_t K);
// harp_deq_gemv_ws's workspace: the counter area (kGemmCounterBytes), then
// the f4 region; 0 when the FP4 product does not apply to the shape.
size_t gemv_workspace_bytes(int32_t M, int32_t N, int32_t K);
size_t gemm_partial_bytes(int32_t M, int32_t N, int32_t K);

// Batch ranges of the products.  harp_deq_gemm runs the small-batch
// matrix-core kernel (no workspace) up to kSkinnyMaxM rows and the tiled
// kernel above.  The fused linears keep x~ in float32 below kBf16MinM rows:
// the vector-ALU / float32 matrix-core product below kSplitMinM, the
// small-batch matrix-core product on the two-plane bf16 split of x~ from
// kSplitMinM; from kBf16MinM rows on x~ is rounded to bf16 for the
// matrix-core products.
constexpr int32_t kSkinnyMaxM = 64;
constexpr int32_t kSplitMinM = 16;
// The float32-x~ product below kSplitMinM: the vector-ALU kernel, except for
// kGemvMcMinM .. kGemvMcMaxM rows at 2 and 4 bits, where the matrix cores
// on the exact bf16 planes of x~ are faster.
constexpr int32_t kGemvMcMinM = 3;
constexpr int32_t kGemvMcMaxM = 8;
constexpr int32_t kBf16MinM = 64;
// The fused linear folds the input rotation into the product launch up to
// this many rows and output features: every workgroup of the one-launch
// form rotates all rows itself, so it only pays off with few rows and at
// most one workgroup (16 features) per CU.  Beyond either limit the
// rotation runs once in its own launch (K = 4096, M = 1: N = 11008 takes
// 16.9 us in two launches against 22.3 us in one).
constexpr int32_t kFusedRotGemvMaxM = 2;
constexpr int32_t kFusedRotGemvMaxN = 4096;

// One-row decode product of 2-bit codes on the FP4 x FP8 matrix cores
// (gemv_f4.hip).  x~ is first turned into FP8 planes of 4-bit digits (one
// exponent per quantization group and plane) in the "f4 region" of the
// workspace; each workgroup holds one K slice of them in LDS, at most
// kF4MaxSliceSteps steps of kF4Step inputs (slices are whole pairs of
// steps).  Eligible: M == 1, 2-bit codes (FP4 operands) or 4-bit codes (FP8
// operands), N a multiple of 16, K a multiple
// of 2 kF4Step, at least kF4MinWeights weights (below that the vector-ALU
// kernel is faster).  f4_slices returns the number of K slices (0: not
// eligible).  With split K allowed it aims at kF4Waves one-tile waves (16
// rows each) and splits only up to kF4MaxSplitTiles tiles (the slices then
// meet on the arrival counters at the workspace's front, their float32
// partials in the f4 region); without it every K must fit one slice.
constexpr int32_t kF4Step = 128;
constexpr int32_t kF4MaxSliceSteps = 64;
constexpr int64_t kF4MinWeights = int64_t{1} << 27;
constexpr int32_t kF4Waves = 2048;
constexpr int32_t kF4MaxSplits = 8;
constexpr int32_t kF4MaxSplitTiles = 512;   // <= kGemmCounterBytes / 4
int32_t f4_slices(int32_t M, int32_t N, int32_t K, int32_t bits, bool allow_split);
// The f4 region: planes (K/128 steps x 64 lanes x 16 bytes), scale bytes
// (K/128 x 64 bytes), group sums of x~ (K/64 floats), then `slices` x N
// float32 partials when slices > 1; offsets within it.
size_t f4_region_bytes(int32_t N, int32_t K, int32_t slices);
size_t f4_psc_offset(int32_t K);
size_t f4_sx_offset(int32_t K);
size_t f4_partial_offset(int32_t K);
// Offset of the f4 region in the fused linear's workspace (after every
// other part).
size_t workspace_f4_offset(int32_t M, int32_t N, int32_t K);

// Workspace layout of the fused linear: the GEMM arrival counters
// (kGemmCounterBytes, always reserved), x~, y', then (M > kSkinnyMaxM) the
// GEMM's partial tiles, then (M == 1, shapes f4_slices admits) the f4
// region, each part 256-byte aligned.  x~ is float32 below
// kBf16MinM rows and bf16 from there on.
size_t workspace_bytes(int32_t M, int32_t N, int32_t K);
size_t workspace_xt_offset();
size_t workspace_yp_offset(int32_t M, int32_t K);
size_t mixed_ws_xf_offset();
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

// Decode chain: uniform square layers of dim 4096 / 8192, full-width sides,
// float32 pairs, one bit width; M up to 4 (4096) or 2 (8192).
size_t chain_ws_bytes(int32_t dim);
harp_status validate_chain(const harp_chain_layer* layers, int32_t n_layers, const void* x,
                           int x_dt, int y_dt, int32_t M, const void* workspace,
                           size_t ws_bytes);

const char* status_string(harp_status s);

}  // namespace harp
