// extern "C" entry points of libharp (declared in include/harp.h): check the
// arguments, pick the kernels, launch them on the caller's stream.
#include <hip/hip_runtime.h>

#include "../../include/harp.h"
#include "launch.hpp"
#include "validate.hpp"

namespace {

thread_local int32_t g_last_hip_error = 0;

harp_status from_hip(hipError_t e) {
  if (e == hipSuccess) return HARP_OK;
  g_last_hip_error = static_cast<int32_t>(e);
  return HARP_ERR_HIP;
}

hipStream_t as_stream(harp_stream s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

harp_status harp_rotate_in(const harp_rotation* V, const void* x,
                           harp_dtype x_dt, void* xt, harp_dtype xt_dt,
                           int32_t M, harp_stream stream) {
  const harp_status st = harp::validate_rotate_in(V, x, x_dt, xt, xt_dt, M);
  if (st != HARP_OK || M == 0) return st;
  return from_hip(harp::launch_rotate(*V, x, x_dt, xt, xt_dt, M, false,
                                      as_stream(stream)));
}

harp_status harp_rotate_out(const harp_rotation* U, const float* yt, void* y,
                            harp_dtype y_dt, int32_t M, harp_stream stream) {
  const harp_status st = harp::validate_rotate_out(U, yt, y, y_dt, M);
  if (st != HARP_OK || M == 0) return st;
  return from_hip(harp::launch_rotate(*U, yt, HARP_F32, y, y_dt, M, true,
                                      as_stream(stream)));
}

harp_status harp_rotate_in_mixed(const harp_mixed_rotation* R, const void* x,
                                 harp_dtype x_dt, void* xt, harp_dtype xt_dt, int32_t M,
                                 void* workspace, size_t ws_bytes, harp_stream stream) {
  const harp_status st =
      harp::validate_rotate_mixed(R, x, x_dt, xt, xt_dt, M, workspace, ws_bytes);
  if (st != HARP_OK || M == 0) return st;
  return from_hip(harp::launch_rotate_mixed(*R, x, x_dt, xt, xt_dt, M, false,
                                            static_cast<float*>(workspace), as_stream(stream)));
}

harp_status harp_rotate_out_mixed(const harp_mixed_rotation* R, const float* yt, void* y,
                                  harp_dtype y_dt, int32_t M, void* workspace, size_t ws_bytes,
                                  harp_stream stream) {
  const harp_status st =
      harp::validate_rotate_mixed(R, yt, HARP_F32, y, y_dt, M, workspace, ws_bytes);
  if (st != HARP_OK || M == 0) return st;
  return from_hip(harp::launch_rotate_mixed(*R, yt, HARP_F32, y, y_dt, M, true,
                                            static_cast<float*>(workspace), as_stream(stream)));
}

size_t harp_rotate_mixed_workspace_bytes(int32_t dim, int32_t M, harp_dtype out_dt) {
  return harp::rotate_mixed_workspace_bytes(dim, M, out_dt);
}

harp_status harp_deq_gemv(const harp_qweight* W, const float* xt, float* yt,
                          int32_t M, harp_stream stream) {
  const harp_status st = harp::validate_gemv(W, xt, yt, M);
  if (st != HARP_OK || M == 0) return st;
  return from_hip(harp::launch_gemv(*W, xt, yt, M, as_stream(stream)));
}

harp_status harp_rotate_in_deq_gemv(const harp_rotation* V, const harp_qweight* W,
                                    const void* x, harp_dtype x_dt, float* yt,
                                    int32_t M, harp_stream stream) {
  const harp_status st = harp::validate_rotate_gemv(V, W, x, x_dt, yt, M);
  if (st != HARP_OK || M == 0) return st;
  if (!harp::gemv_rotated_supported(*V, *W, M)) return HARP_ERR_UNSUPPORTED;
  return from_hip(harp::launch_gemv_rotated(*V, *W, x, x_dt, yt, M, as_stream(stream)));
}

harp_status harp_deq_gemm(const harp_qweight* W, const uint16_t* xt_bf16,
                          float* yt, int32_t M, void* workspace, size_t ws_bytes,
                          harp_stream stream) {
  const harp_status st = harp::validate_gemm(W, xt_bf16, yt, M, workspace, ws_bytes);
  if (st != HARP_OK || M == 0) return st;
  if (M <= harp::kSkinnyMaxM)
    return from_hip(harp::launch_gemm_skinny(*W, xt_bf16, yt, M, as_stream(stream)));
  const int splits = workspace ? harp::gemm_splits(M, W->N, W->K) : 1;
  return from_hip(harp::launch_gemm(*W, xt_bf16, yt, M, splits, workspace,
                                    as_stream(stream)));
}

size_t harp_deq_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (M < 0 || M > HARP_MAX_M || N < 1 || N > HARP_MAX_DIM || K < 64 ||
      K > HARP_MAX_DIM)
    return 0;
  return harp::gemm_workspace_bytes(M, N, K);
}

size_t harp_linear_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  return harp::workspace_bytes(M, N, K);
}

harp_status harp_linear_fused(const harp_rotation* V, const harp_qweight* W,
                              const harp_rotation* U, const void* x,
                              harp_dtype x_dt, void* y, harp_dtype y_dt,
                              int32_t M, void* workspace, size_t ws_bytes,
                              harp_stream stream) {
  const harp_status st = harp::validate_fused(V, W, U, x, x_dt, y, y_dt, M,
                                              workspace, ws_bytes);
  if (st != HARP_OK || M == 0) return st;
  const hipStream_t s = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  float* yp = reinterpret_cast<float*>(ws + harp::workspace_yp_offset(M, W->K));
  if (M <= harp::kFusedRotGemvMaxM && W->N <= harp::kFusedRotGemvMaxN &&
      harp::gemv_rotated_supported(*V, *W, M)) {
    const harp_status r = from_hip(harp::launch_gemv_rotated(*V, *W, x, x_dt, yp, M, s));
    if (r != HARP_OK) return r;
  } else if (M < harp::kMfmaMinM) {
    float* xt = reinterpret_cast<float*>(ws);
    harp_status r = from_hip(harp::launch_rotate(*V, x, x_dt, xt, HARP_F32, M, false, s));
    if (r != HARP_OK) return r;
    r = from_hip(harp::launch_gemv(*W, xt, yp, M, s));
    if (r != HARP_OK) return r;
  } else {
    uint16_t* xt = reinterpret_cast<uint16_t*>(ws);
    // y' is not yet written: when it is at least as large as x~ in float32
    // it holds the intermediate of the two-launch input rotation
    harp_status r = from_hip(
        W->N >= W->K ? harp::launch_rotate_in_scratch(*V, x, x_dt, xt, yp, M, s)
                     : harp::launch_rotate(*V, x, x_dt, xt, HARP_BF16, M, false, s));
    if (r != HARP_OK) return r;
    if (M <= harp::kSkinnyMaxM)
      r = from_hip(harp::launch_gemm_skinny(*W, xt, yp, M, s));
    else
      r = from_hip(harp::launch_gemm(*W, xt, yp, M, harp::gemm_splits(M, W->N, W->K),
                                     ws + harp::workspace_gemm_offset(M, W->N, W->K), s));
    if (r != HARP_OK) return r;
  }
  return from_hip(harp::launch_rotate(*U, yp, HARP_F32, y, y_dt, M, true, s));
}

size_t harp_linear_mixed_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  return harp::mixed_workspace_bytes(M, N, K);
}

harp_status harp_linear_fused_mixed(const harp_mixed_rotation* V, const harp_qweight* W,
                                    const harp_mixed_rotation* U, const void* x,
                                    harp_dtype x_dt, void* y, harp_dtype y_dt, int32_t M,
                                    void* workspace, size_t ws_bytes, harp_stream stream) {
  const harp_status st =
      harp::validate_fused_mixed(V, W, U, x, x_dt, y, y_dt, M, workspace, ws_bytes);
  if (st != HARP_OK || M == 0) return st;
  const hipStream_t s = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  const int32_t N = W->N, K = W->K;
  float* xf = reinterpret_cast<float*>(ws);
  float* yp = reinterpret_cast<float*>(ws + harp::mixed_ws_yp_offset(M, K));
  float* ys = reinterpret_cast<float*>(ws + harp::mixed_ws_ys_offset(M, N, K));
  harp_status r;
  if (M < harp::kMfmaMinM) {
    r = from_hip(harp::launch_rotate_mixed(*V, x, x_dt, xf, HARP_F32, M, false, nullptr, s));
    if (r != HARP_OK) return r;
    r = from_hip(harp::launch_gemv(*W, xf, yp, M, s));
  } else {
    uint16_t* xb = reinterpret_cast<uint16_t*>(ws + harp::mixed_ws_xb_offset(M, K));
    r = from_hip(harp::launch_rotate_mixed(*V, x, x_dt, xb, HARP_BF16, M, false, xf, s));
    if (r != HARP_OK) return r;
    if (M <= harp::kSkinnyMaxM)
      r = from_hip(harp::launch_gemm_skinny(*W, xb, yp, M, s));
    else
      r = from_hip(harp::launch_gemm(*W, xb, yp, M, harp::gemm_splits(M, N, K),
                                     ws + harp::mixed_ws_gemm_offset(M, N, K), s));
  }
  if (r != HARP_OK) return r;
  return from_hip(harp::launch_rotate_mixed(*U, yp, HARP_F32, y, y_dt, M, true, ys, s));
}

harp_status harp_dequant(const harp_qweight* W, void* out, harp_dtype out_dt,
                         harp_stream stream) {
  const harp_status st = harp::validate_dequant(W, out, out_dt);
  if (st != HARP_OK) return st;
  return from_hip(harp::launch_dequant(*W, out, out_dt, as_stream(stream)));
}

size_t harp_rotate_weight_workspace_bytes(int32_t N, int32_t K) {
  return harp::rotate_weight_workspace_bytes(N, K);
}

harp_status harp_rotate_weight(const harp_rotation* V, const harp_rotation* U,
                               const float* W, float* Wp, int32_t N, int32_t K,
                               void* workspace, size_t ws_bytes, harp_stream stream) {
  const harp_status st = harp::validate_rotate_weight(V, U, W, Wp, N, K, workspace, ws_bytes);
  if (st != HARP_OK) return st;
  const hipStream_t s = as_stream(stream);
  float* t = static_cast<float*>(workspace);
  // rows: W F_V^T (each row w_n -> F_V w_n), then columns: F_U (.) by
  // rotating the rows of the transpose
  harp_status r = from_hip(harp::launch_rotate(*V, W, HARP_F32, t, HARP_F32, N, false, s));
  if (r != HARP_OK) return r;
  r = from_hip(harp::launch_transpose(t, Wp, N, K, s));          // Wp holds [K][N]
  if (r != HARP_OK) return r;
  r = from_hip(harp::launch_rotate(*U, Wp, HARP_F32, t, HARP_F32, K, false, s));
  if (r != HARP_OK) return r;
  return from_hip(harp::launch_transpose(t, Wp, K, N, s));
}

harp_status harp_quantize_pack(const float* Wp, int32_t N, int32_t K, int32_t bits,
                               uint32_t* qweight, uint16_t* scale, uint16_t* zero,
                               harp_stream stream) {
  const harp_status st = harp::validate_quantize_pack(Wp, N, K, bits, qweight, scale, zero);
  if (st != HARP_OK) return st;
  return from_hip(harp::launch_quantize_pack(Wp, N, K, bits, qweight, scale, zero,
                                             as_stream(stream)));
}

const char* harp_status_string(harp_status status) {
  return harp::status_string(status);
}

int32_t harp_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
