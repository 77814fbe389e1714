// extern "C" entry points of libharp (declared in include/harp.h): check the
// arguments, pick the kernels, launch them on the caller's stream.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/harp.h"
#include "chain.hpp"
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

// The whole linear on a workspace laid out as harp_linear_workspace_bytes
// describes (arguments already checked).  split_k: the M > 64 GEMM and the
// one-row FP4 product may split K (needs the counters at the front of ws,
// zero, and the partials after y' or in the f4 region); without it they run
// one K slice and only the counter area, x~, y' and (one-row FP4 product)
// the f4 region's planes are used (the counter area is then not read).
harp_status fused_linear(const harp_rotation& V, const harp_qweight& W, const harp_rotation& U,
                         const void* x, harp_dtype x_dt, void* y, harp_dtype y_dt, int32_t M,
                         char* ws, bool split_k, hipStream_t s) {
  float* yp = reinterpret_cast<float*>(ws + harp::workspace_yp_offset(M, W.K));
  harp_status r;
  if (M <= harp::kFusedRotGemvMaxM && W.N <= harp::kFusedRotGemvMaxN &&
      harp::gemv_rotated_supported(V, W, M)) {
    r = from_hip(harp::launch_gemv_rotated(V, W, x, x_dt, yp, M, s));
  } else if (M < harp::kBf16MinM) {
    // float32 x~: the float32 product, or the matrix cores on its two-plane
    // bf16 split
    float* xt = reinterpret_cast<float*>(ws + harp::workspace_xt_offset());
    // one row on the FP4 product: with a b = 256 / 4096 / 8192 input side
    // the rotation's last launch writes the product's planes itself
    const int32_t f4_slices = harp::f4_slices(M, W.N, W.K, W.bits, split_k);
    uint8_t* f4r = reinterpret_cast<uint8_t*>(ws + harp::workspace_f4_offset(M, W.N, W.K));
    const bool fold = f4_slices > 0 && harp::rotate_in_f4_supported(V, M);
    r = from_hip(fold ? harp::launch_rotate_in_f4(V, x, x_dt, xt, f4r, s)
                      : harp::launch_rotate(V, x, x_dt, xt, HARP_F32, M, false, s));
    if (r != HARP_OK) return r;
    // and with a b = 256 output side (one K slice, a zeroed workspace) the
    // product's last workgroup of each 256-output block applies F_U^T
    if (f4_slices > 0 && split_k && harp::gemv_f4_fold_supported(U, W, f4_slices))
      return from_hip(harp::launch_gemv_f4(W, xt, yp, f4r, reinterpret_cast<uint32_t*>(ws),
                                           f4_slices, fold, s, &U, y, y_dt));
    if (f4_slices > 0)
      r = from_hip(harp::launch_gemv_f4(W, xt, yp, f4r, reinterpret_cast<uint32_t*>(ws),
                                        f4_slices, fold, s));
    else if (M < harp::kSplitMinM)
      r = from_hip(harp::launch_gemv(W, xt, yp, M, s));
    else if (split_k)
      r = from_hip(harp::launch_gemm_skinny_split_k(
          W, xt, yp, M, reinterpret_cast<float*>(ws + harp::workspace_gemm_offset(M, W.N, W.K)),
          reinterpret_cast<uint32_t*>(ws), s));
    else
      r = from_hip(harp::launch_gemm_skinny_split(W, xt, yp, M, s));
  } else {
    uint16_t* xt = reinterpret_cast<uint16_t*>(ws + harp::workspace_xt_offset());
    // y' is not yet written: when it is at least as large as x~ in float32
    // it holds the intermediate of the two-launch input rotation
    r = from_hip(W.N >= W.K ? harp::launch_rotate_in_scratch(V, x, x_dt, xt, yp, M, s)
                            : harp::launch_rotate(V, x, x_dt, xt, HARP_BF16, M, false, s));
    if (r != HARP_OK) return r;
    if (M <= harp::kSkinnyMaxM)
      r = from_hip(harp::launch_gemm_skinny(W, xt, yp, M, s));
    else
      r = from_hip(harp::launch_gemm(
          W, xt, yp, M, split_k ? harp::gemm_splits(M, W.N, W.K) : 1,
          reinterpret_cast<float*>(ws + harp::workspace_gemm_offset(M, W.N, W.K)),
          reinterpret_cast<uint32_t*>(ws), s));
  }
  if (r != HARP_OK) return r;
  return from_hip(harp::launch_rotate(U, yp, HARP_F32, y, y_dt, M, true, s));
}

// Device memory of harp_linear_fused_noalloc: a file-scope array that every
// GPU the library runs on holds until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: its device
// address is taken once per device with hipGetSymbolAddress (that device
// current) and kept in scratch_ptr; only that pointer reaches kernels.
constexpr size_t kScratchBytes = size_t{32} << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

harp_status device_scratch(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e);
  if (dev < 0 || dev >= kMaxDevices) return HARP_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return from_hip(e);
    if (p == nullptr) return HARP_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return HARP_OK;
}

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

harp_status harp_deq_gemv_ws(const harp_qweight* W, const float* xt, float* yt, int32_t M,
                             void* workspace, size_t ws_bytes, harp_stream stream) {
  const harp_status st = harp::validate_gemv_ws(W, xt, yt, M, workspace, ws_bytes);
  if (st != HARP_OK || M == 0) return st;
  const int32_t slices =
      workspace != nullptr && W->bits == 2 ? harp::f4_slices(M, W->N, W->K, W->bits, true) : 0;
  if (slices > 0) {
    char* ws = static_cast<char*>(workspace);
    return from_hip(harp::launch_gemv_f4(*W, xt, yt,
                                         reinterpret_cast<uint8_t*>(ws + harp::kGemmCounterBytes),
                                         reinterpret_cast<uint32_t*>(ws), slices, false,
                                         as_stream(stream)));
  }
  return from_hip(harp::launch_gemv(*W, xt, yt, M, as_stream(stream)));
}

size_t harp_deq_gemv_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (M < 0 || M > HARP_MAX_M || N < 1 || N > HARP_MAX_DIM || K < 64 ||
      K > HARP_MAX_DIM)
    return 0;
  return harp::gemv_workspace_bytes(M, N, K);
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
  char* ws = static_cast<char*>(workspace);
  return from_hip(harp::launch_gemm(
      *W, xt_bf16, yt, M, splits,
      splits > 1 ? reinterpret_cast<float*>(ws + harp::kGemmCounterBytes) : nullptr,
      reinterpret_cast<uint32_t*>(ws), as_stream(stream)));
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
  return fused_linear(*V, *W, *U, x, x_dt, y, y_dt, M, static_cast<char*>(workspace),
                      true, as_stream(stream));
}

size_t harp_linear_chain_workspace_bytes(int32_t dim) { return harp::chain_ws_bytes(dim); }

harp_status harp_linear_chain(const harp_chain_layer* layers, int32_t n_layers, const void* x,
                              harp_dtype x_dt, harp_dtype y_dt, int32_t M, void* workspace,
                              size_t ws_bytes, harp_stream stream) {
  const harp_status st =
      harp::validate_chain(layers, n_layers, x, x_dt, y_dt, M, workspace, ws_bytes);
  if (st != HARP_OK || n_layers == 0 || M == 0) return st;
  const int32_t dim = layers[0].V.dim;
  const hipStream_t s = as_stream(stream);
  // one launch per kChainMaxLayers layers; a later launch starts from the
  // previous one's last output
  for (int32_t l0 = 0; l0 < n_layers; l0 += harp::kChainMaxLayers) {
    harp::ChainArgs a{};
    a.n_layers = n_layers - l0 < harp::kChainMaxLayers ? n_layers - l0 : harp::kChainMaxLayers;
    a.M = M;
    a.x = l0 == 0 ? x : layers[l0 - 1].y;
    a.x_bf16 = (l0 == 0 ? x_dt : y_dt) == HARP_BF16;
    a.y_bf16 = y_dt == HARP_BF16;
    a.ws = static_cast<uint32_t*>(workspace);
    for (int32_t i = 0; i < a.n_layers; ++i) {
      const harp_chain_layer& c = layers[l0 + i];
      a.layer[i] = harp::ChainLayer{reinterpret_cast<const float2*>(c.V.cs), c.V.sign_bits,
                                    c.W.qweight, c.W.scale, c.W.zero,
                                    reinterpret_cast<const float2*>(c.U.cs), c.U.sign_bits, c.y};
    }
    const harp_status r = from_hip(harp::launch_chain(a, dim, layers[0].W.bits, s));
    if (r != HARP_OK) return r;
  }
  return HARP_OK;
}

harp_status harp_linear_fused_noalloc(const harp_rotation* V, const harp_qweight* W,
                                      const harp_rotation* U, const void* x,
                                      harp_dtype x_dt, void* y, harp_dtype y_dt,
                                      int32_t M, harp_stream stream) {
  // the argument checks of harp_linear_fused with a stand-in workspace (an
  // aligned non-null address and no size limit); then the size this call
  // needs in the scratch: counter area, x~ and y' (one K slice, no
  // partials), and the f4 region's planes when the one-row FP4 product runs
  harp_status st = harp::validate_fused(V, W, U, x, x_dt, y, y_dt, M,
                                        reinterpret_cast<void*>(uintptr_t{256}), SIZE_MAX);
  if (st != HARP_OK || M == 0) return st;
  static_assert(kScratchBytes % 256 == 0, "scratch size");
  const int32_t f4s = harp::f4_slices(M, W->N, W->K, W->bits, false);
  const size_t need = f4s > 0 ? harp::workspace_f4_offset(M, W->N, W->K) +
                                    harp::f4_region_bytes(W->N, W->K, f4s)
                              : harp::workspace_gemm_offset(M, W->N, W->K);
  if (need > kScratchBytes) return HARP_ERR_WORKSPACE;
  char* scratch_ptr = nullptr;
  st = device_scratch(&scratch_ptr);
  if (st != HARP_OK) return st;
  return fused_linear(*V, *W, *U, x, x_dt, y, y_dt, M, scratch_ptr, false, as_stream(stream));
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
  float* xf = reinterpret_cast<float*>(ws + harp::mixed_ws_xf_offset());
  float* yp = reinterpret_cast<float*>(ws + harp::mixed_ws_yp_offset(M, K));
  float* ys = reinterpret_cast<float*>(ws + harp::mixed_ws_ys_offset(M, N, K));
  harp_status r;
  if (M < harp::kBf16MinM) {
    r = from_hip(harp::launch_rotate_mixed(*V, x, x_dt, xf, HARP_F32, M, false, nullptr, s));
    if (r != HARP_OK) return r;
    r = from_hip(M < harp::kSplitMinM ? harp::launch_gemv(*W, xf, yp, M, s)
                                      : harp::launch_gemm_skinny_split(*W, xf, yp, M, s));
  } else {
    uint16_t* xb = reinterpret_cast<uint16_t*>(ws + harp::mixed_ws_xb_offset(M, K));
    r = from_hip(harp::launch_rotate_mixed(*V, x, x_dt, xb, HARP_BF16, M, false, xf, s));
    if (r != HARP_OK) return r;
    if (M <= harp::kSkinnyMaxM)
      r = from_hip(harp::launch_gemm_skinny(*W, xb, yp, M, s));
    else
      r = from_hip(harp::launch_gemm(
          *W, xb, yp, M, harp::gemm_splits(M, N, K),
          reinterpret_cast<float*>(ws + harp::mixed_ws_gemm_offset(M, N, K)),
          reinterpret_cast<uint32_t*>(ws), s));
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
