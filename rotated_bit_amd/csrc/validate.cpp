// Argument checks of the C ABI (see validate.hpp).  Order of checks, which
// fixes the status returned when several arguments are wrong: structure
// pointers and their fields (NULL), unsupported formats, shapes, dtypes,
// batch range, data pointers (NULL when M > 0), alignment, workspace.
#include "validate.hpp"

#include "chain_layout.hpp"

#include <algorithm>
#include <cmath>

namespace harp {
namespace {

bool pow2(int32_t v) { return v > 0 && (v & (v - 1)) == 0; }
bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}
bool bad_dtype(int dt) { return dt != HARP_F32 && dt != HARP_BF16; }
size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

harp_status check_m(int32_t M) {
  return (M < 0 || M > HARP_MAX_M) ? HARP_ERR_SHAPE : HARP_OK;
}

// A data buffer of a call with M rows: NULL allowed only when M == 0.
harp_status check_data(const void* p, int32_t M) {
  if (M == 0) return HARP_OK;
  if (p == nullptr) return HARP_ERR_NULL;
  return aligned(p, 16) ? HARP_OK : HARP_ERR_ALIGN;
}

#define HARP_TRY(expr)                      \
  do {                                      \
    const harp_status st_ = (expr);         \
    if (st_ != HARP_OK) return st_;         \
  } while (0)

}  // namespace

harp_status check_rotation(const harp_rotation* R) {
  if (R == nullptr || R->sign_bits == nullptr ||
      (R->cs == nullptr && R->phi_codes == nullptr))
    return HARP_ERR_NULL;
  if (R->cs != nullptr && R->phi_codes != nullptr) return HARP_ERR_SHAPE;
  if (pow2(R->block) && R->block > HARP_MAX_BLOCK) return HARP_ERR_UNSUPPORTED;
  if (!pow2(R->block) || R->block < 2) return HARP_ERR_SHAPE;
  if (R->dim < 1 || R->dim > HARP_MAX_DIM || R->dim % R->block != 0)
    return HARP_ERR_SHAPE;
  if (R->phi_codes != nullptr && !std::isfinite(R->phi_step)) return HARP_ERR_SHAPE;
  const void* angles = R->cs != nullptr ? static_cast<const void*>(R->cs)
                                        : static_cast<const void*>(R->phi_codes);
  if (!aligned(angles, 16) || !aligned(R->sign_bits, 16)) return HARP_ERR_ALIGN;
  return HARP_OK;
}

harp_status check_qweight(const harp_qweight* W) {
  if (W == nullptr || W->qweight == nullptr || W->scale == nullptr ||
      W->zero == nullptr)
    return HARP_ERR_NULL;
  if (W->bits != 2 && W->bits != 3 && W->bits != 4) return HARP_ERR_UNSUPPORTED;
  if (W->group != 64) return HARP_ERR_UNSUPPORTED;
  if (W->N < 1 || W->N > HARP_MAX_DIM || W->K < 64 || W->K > HARP_MAX_DIM ||
      W->K % 64 != 0)
    return HARP_ERR_SHAPE;
  if (!aligned(W->qweight, 16) || !aligned(W->scale, 16) || !aligned(W->zero, 16))
    return HARP_ERR_ALIGN;
  return HARP_OK;
}

harp_status validate_rotate_in(const harp_rotation* V, const void* x, int x_dt,
                               const void* xt, int xt_dt, int32_t M) {
  HARP_TRY(check_rotation(V));
  if (bad_dtype(x_dt) || bad_dtype(xt_dt)) return HARP_ERR_DTYPE;
  HARP_TRY(check_m(M));
  HARP_TRY(check_data(x, M));
  HARP_TRY(check_data(xt, M));
  return HARP_OK;
}

harp_status validate_rotate_out(const harp_rotation* U, const void* yt,
                                const void* y, int y_dt, int32_t M) {
  HARP_TRY(check_rotation(U));
  if (bad_dtype(y_dt)) return HARP_ERR_DTYPE;
  HARP_TRY(check_m(M));
  HARP_TRY(check_data(yt, M));
  HARP_TRY(check_data(y, M));
  return HARP_OK;
}

harp_status validate_gemv(const harp_qweight* W, const void* xt, const void* yt,
                          int32_t M) {
  HARP_TRY(check_qweight(W));
  HARP_TRY(check_m(M));
  HARP_TRY(check_data(xt, M));
  HARP_TRY(check_data(yt, M));
  return HARP_OK;
}

harp_status validate_rotate_gemv(const harp_rotation* V, const harp_qweight* W,
                                const void* x, int x_dt, const void* yt, int32_t M) {
  HARP_TRY(check_rotation(V));
  HARP_TRY(check_qweight(W));
  if (V->dim != W->K) return HARP_ERR_SHAPE;
  if (bad_dtype(x_dt)) return HARP_ERR_DTYPE;
  HARP_TRY(check_m(M));
  HARP_TRY(check_data(x, M));
  HARP_TRY(check_data(yt, M));
  return HARP_OK;
}

harp_status validate_gemv_ws(const harp_qweight* W, const void* xt, const void* yt,
                             int32_t M, const void* workspace, size_t ws_bytes) {
  HARP_TRY(validate_gemv(W, xt, yt, M));
  if (M == 0 || workspace == nullptr) return HARP_OK;   // no workspace: harp_deq_gemv
  if (!aligned(workspace, 256)) return HARP_ERR_ALIGN;
  if (ws_bytes < gemv_workspace_bytes(M, W->N, W->K)) return HARP_ERR_WORKSPACE;
  return HARP_OK;
}

harp_status validate_gemm(const harp_qweight* W, const void* xt, const void* yt,
                          int32_t M, const void* workspace, size_t ws_bytes) {
  HARP_TRY(validate_gemv(W, xt, yt, M));
  if (M == 0 || workspace == nullptr) return HARP_OK;   // no workspace: one K slice
  if (!aligned(workspace, 256)) return HARP_ERR_ALIGN;
  if (ws_bytes < gemm_workspace_bytes(M, W->N, W->K)) return HARP_ERR_WORKSPACE;
  return HARP_OK;
}

harp_status validate_fused(const harp_rotation* V, const harp_qweight* W,
                           const harp_rotation* U, const void* x, int x_dt,
                           const void* y, int y_dt, int32_t M,
                           const void* workspace, size_t ws_bytes) {
  HARP_TRY(check_rotation(V));
  HARP_TRY(check_qweight(W));
  HARP_TRY(check_rotation(U));
  if (V->dim != W->K || U->dim != W->N) return HARP_ERR_SHAPE;
  if (bad_dtype(x_dt) || bad_dtype(y_dt)) return HARP_ERR_DTYPE;
  HARP_TRY(check_m(M));
  HARP_TRY(check_data(x, M));
  HARP_TRY(check_data(y, M));
  if (M == 0) return HARP_OK;
  if (workspace == nullptr) return HARP_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return HARP_ERR_ALIGN;
  if (ws_bytes < workspace_bytes(M, W->N, W->K)) return HARP_ERR_WORKSPACE;
  return HARP_OK;
}

harp_status validate_rotate_weight(const harp_rotation* V, const harp_rotation* U,
                                   const float* W, const float* Wp, int32_t N, int32_t K,
                                   const void* workspace, size_t ws_bytes) {
  HARP_TRY(check_rotation(V));
  HARP_TRY(check_rotation(U));
  // weight rows (N) and columns (K) are the batches of the two rotations
  if (N < 1 || K < 1 || N > HARP_MAX_M || K > HARP_MAX_M) return HARP_ERR_SHAPE;
  if (V->dim != K || U->dim != N) return HARP_ERR_SHAPE;
  if (W == nullptr || Wp == nullptr || workspace == nullptr) return HARP_ERR_NULL;
  if (!aligned(W, 16) || !aligned(Wp, 16) || !aligned(workspace, 256)) return HARP_ERR_ALIGN;
  if (ws_bytes < rotate_weight_workspace_bytes(N, K)) return HARP_ERR_WORKSPACE;
  return HARP_OK;
}

harp_status validate_quantize_pack(const float* Wp, int32_t N, int32_t K, int32_t bits,
                                   const void* qweight, const void* scale, const void* zero) {
  if (bits != 2 && bits != 3 && bits != 4) return HARP_ERR_UNSUPPORTED;
  if (N < 1 || N > HARP_MAX_DIM || K < 64 || K > HARP_MAX_DIM || K % 64 != 0)
    return HARP_ERR_SHAPE;
  if (Wp == nullptr || qweight == nullptr || scale == nullptr || zero == nullptr)
    return HARP_ERR_NULL;
  if (!aligned(Wp, 16) || !aligned(qweight, 16) || !aligned(scale, 16) || !aligned(zero, 16))
    return HARP_ERR_ALIGN;
  return HARP_OK;
}

size_t rotate_weight_workspace_bytes(int32_t N, int32_t K) {
  if (N < 1 || K < 1 || N > HARP_MAX_M || K > HARP_MAX_M) return 0;
  return align256(static_cast<size_t>(N) * K * 4);
}

size_t rotate_mixed_workspace_bytes(int32_t dim, int32_t M, int out_dt) {
  if (dim < 2 || dim > HARP_MAX_MIXED_DIM || M < 0 || M > HARP_MAX_M) return 0;
  if (out_dt != HARP_BF16) return 0;
  return align256(static_cast<size_t>(M) * dim * 4);
}

static harp_status check_mixed(const harp_mixed_rotation* R) {
  if (R == nullptr || R->blocks == nullptr || R->sign_bits == nullptr) return HARP_ERR_NULL;
  if (R->n_stages < 1 || R->n_stages > HARP_MAX_STAGES) return HARP_ERR_SHAPE;
  int64_t prod = 1;                 // capped: 16 radices of 64 would overflow
  for (int t = 0; t < R->n_stages; ++t) {
    if (R->radix[t] > HARP_MAX_RADIX) return HARP_ERR_UNSUPPORTED;
    if (R->radix[t] < 2) return HARP_ERR_SHAPE;
    prod = std::min<int64_t>(prod * R->radix[t], int64_t{HARP_MAX_MIXED_DIM} + 1);
  }
  if (R->dim > HARP_MAX_MIXED_DIM) return HARP_ERR_UNSUPPORTED;
  if (R->dim < 2 || prod != R->dim) return HARP_ERR_SHAPE;
  if (!aligned(R->blocks, 16) || !aligned(R->sign_bits, 16)) return HARP_ERR_ALIGN;
  return HARP_OK;
}

harp_status validate_rotate_mixed(const harp_mixed_rotation* R, const void* in, int in_dt,
                                  const void* out, int out_dt, int32_t M,
                                  const void* workspace, size_t ws_bytes) {
  HARP_TRY(check_mixed(R));
  if (bad_dtype(in_dt) || bad_dtype(out_dt)) return HARP_ERR_DTYPE;
  HARP_TRY(check_m(M));
  HARP_TRY(check_data(in, M));
  HARP_TRY(check_data(out, M));
  if (workspace != nullptr && out_dt == HARP_BF16) {
    if (ws_bytes < rotate_mixed_workspace_bytes(R->dim, M, out_dt)) return HARP_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return HARP_ERR_ALIGN;
  }
  return HARP_OK;
}

// Workspace of the mixed-radix linear: the GEMM arrival counters (always
// reserved, fixed offset), x~ as float32 (below kBf16MinM rows: the operand;
// otherwise the stage buffer of the bf16 operand, which follows), y'
// float32, the stage buffer of a bf16 output, then (M > 64) the GEMM's
// partial tiles.
size_t mixed_ws_xf_offset() { return kGemmCounterBytes; }

size_t mixed_ws_xb_offset(int32_t M, int32_t K) {
  return mixed_ws_xf_offset() + align256(static_cast<size_t>(M) * K * 4);
}

size_t mixed_ws_yp_offset(int32_t M, int32_t K) {
  return mixed_ws_xb_offset(M, K) +
         (M >= kBf16MinM ? align256(static_cast<size_t>(M) * K * 2) : 0);
}

size_t mixed_ws_ys_offset(int32_t M, int32_t N, int32_t K) {
  return mixed_ws_yp_offset(M, K) + align256(static_cast<size_t>(M) * N * 4);
}

size_t mixed_ws_gemm_offset(int32_t M, int32_t N, int32_t K) {
  return mixed_ws_ys_offset(M, N, K) + align256(static_cast<size_t>(M) * N * 4);
}

size_t mixed_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (M < 0 || M > HARP_MAX_M || N < 2 || N > HARP_MAX_MIXED_DIM || K < 64 ||
      K > HARP_MAX_MIXED_DIM)
    return 0;
  if (M == 0) return 0;
  return mixed_ws_gemm_offset(M, N, K) + gemm_partial_bytes(M, N, K);
}

harp_status validate_fused_mixed(const harp_mixed_rotation* V, const harp_qweight* W,
                                 const harp_mixed_rotation* U, const void* x, int x_dt,
                                 const void* y, int y_dt, int32_t M,
                                 const void* workspace, size_t ws_bytes) {
  HARP_TRY(check_mixed(V));
  HARP_TRY(check_qweight(W));
  HARP_TRY(check_mixed(U));
  if (V->dim != W->K || U->dim != W->N) return HARP_ERR_SHAPE;
  if (bad_dtype(x_dt) || bad_dtype(y_dt)) return HARP_ERR_DTYPE;
  HARP_TRY(check_m(M));
  HARP_TRY(check_data(x, M));
  HARP_TRY(check_data(y, M));
  if (M == 0) return HARP_OK;
  if (workspace == nullptr) return HARP_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return HARP_ERR_ALIGN;
  if (ws_bytes < mixed_workspace_bytes(M, W->N, W->K)) return HARP_ERR_WORKSPACE;
  return HARP_OK;
}

harp_status validate_dequant(const harp_qweight* W, const void* out, int out_dt) {
  HARP_TRY(check_qweight(W));
  if (bad_dtype(out_dt)) return HARP_ERR_DTYPE;
  HARP_TRY(check_data(out, 1));
  return HARP_OK;
}

int32_t gemm_splits(int32_t M, int32_t N, int32_t K) {
  if (M <= kSkinnyMaxM || N < 1 || K < 64) return 1;
  const int64_t tiles = static_cast<int64_t>((M + kGemmTile - 1) / kGemmTile) *
                        ((N + kGemmTile - 1) / kGemmTile);
  if (tiles > kGemmMaxSplitTiles) return 1;   // many rounds: the split gains little
  // The slice count whose workgroups fill the last round of kGemmSlots
  // best (ties to fewer slices), each slice at least 8 groups.
  const int32_t groups = K / 64;
  int32_t best = 1;
  double best_fill = 0.0;
  for (int32_t s = 1; s <= kGemmMaxSplits && groups / s >= 8; ++s) {
    const int64_t wgs = tiles * s;
    const int64_t rounds = (wgs + kGemmSlots - 1) / kGemmSlots;
    const double fill = static_cast<double>(wgs) / static_cast<double>(rounds * kGemmSlots);
    if (fill > best_fill + 1e-9) {
      best = s;
      best_fill = fill;
    }
  }
  return best;
}

WideSplit skinny_wide_split(int32_t M, int32_t N, int32_t K, bool allow_split) {
  WideSplit r{0, 1};
  if (M < 1 || M > kSkinnyMaxM || N < 1 || K < 4096 || K % 4096 != 0) return r;
  const int32_t G = K / 64;
  const int64_t row_tiles = M <= 16 ? 1 : (M + 31) / 32;   // 16-row, else 32-row tiles
  const int64_t tiles4 = (N + 63) / 64;
  const int64_t tiles2 = (N + 31) / 32;
  if (tiles4 >= kGemmSlots) return WideSplit{4, 1};
  if (allow_split && tiles4 * row_tiles <= kGemmMaxSplitTiles) {
    for (int32_t s = 2; s <= 8; ++s)
      if (G % (64 * s) == 0 && tiles4 * s >= kGemmSlots) return WideSplit{4, s};
  }
  if (tiles2 >= kGemmSlots) return WideSplit{2, 1};
  return r;
}

size_t skinny_partial_bytes(int32_t M, int32_t N, int32_t K) {
  if (M < kSplitMinM || M >= kBf16MinM) return 0;   // the fused linear's split range
  const WideSplit w = skinny_wide_split(M, N, K, true);
  if (w.splits <= 1) return 0;
  return align256(static_cast<size_t>(w.splits) * M * N * 4);
}

size_t gemm_partial_bytes(int32_t M, int32_t N, int32_t K) {
  const int32_t s = gemm_splits(M, N, K);
  if (s <= 1) return 0;
  const size_t tiles = static_cast<size_t>((M + kGemmTile - 1) / kGemmTile) *
                       ((N + kGemmTile - 1) / kGemmTile);
  return align256(static_cast<size_t>(s) * tiles * kGemmTile * kGemmTile * 4);
}

// harp_deq_gemm's own workspace: counters, then partial tiles.
size_t gemm_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  const size_t p = gemm_partial_bytes(M, N, K);
  return p == 0 ? 0 : kGemmCounterBytes + p;
}

size_t workspace_xt_offset() { return kGemmCounterBytes; }

size_t workspace_yp_offset(int32_t M, int32_t K) {
  const size_t xt_elem = M < kBf16MinM ? 4 : 2;
  return workspace_xt_offset() + align256(static_cast<size_t>(M) * K * xt_elem);
}

size_t workspace_gemm_offset(int32_t M, int32_t N, int32_t K) {
  return workspace_yp_offset(M, K) + align256(static_cast<size_t>(M) * N * 4);
}

int32_t f4_slices(int32_t M, int32_t N, int32_t K, int32_t bits, bool allow_split) {
  if (M != 1 || (bits != 2 && bits != 4) || N < 16 || N % 16 != 0 || K < 2 * kF4Step || K % (2 * kF4Step) != 0 ||
      static_cast<int64_t>(N) * K < kF4MinWeights)
    return 0;
  // slices are whole step pairs; the largest of them must fit in LDS
  const int32_t pairs = K / (2 * kF4Step);
  const int32_t tiles = N / 16;
  const auto fits = [&](int32_t s) { return (pairs + s - 1) / s * 2 <= kF4MaxSliceSteps; };
  if (!allow_split || tiles > kF4MaxSplitTiles) return fits(1) ? 1 : 0;
  int32_t s = (kF4Waves + tiles - 1) / tiles;
  s = std::min(s, kF4MaxSplits);
  s = std::min(s, std::max(1, pairs / 2));   // at least 2 step pairs per slice
  while (!fits(s)) ++s;
  return s <= kF4MaxSplits ? s : 0;
}

size_t f4_psc_offset(int32_t K) { return static_cast<size_t>(K / kF4Step) * 1024; }
size_t f4_sx_offset(int32_t K) { return f4_psc_offset(K) + static_cast<size_t>(K / kF4Step) * 64; }
size_t f4_partial_offset(int32_t K) {
  return align256(f4_sx_offset(K) + static_cast<size_t>(K / 64) * 4);   // one float per group
}
size_t f4_region_bytes(int32_t N, int32_t K, int32_t slices) {
  if (slices <= 0) return 0;
  return f4_partial_offset(K) + (slices > 1 ? align256(static_cast<size_t>(slices) * N * 4) : 0);
}

size_t gemv_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  // the size query does not know the bit width: sized for 2-bit codes
  const int32_t s = f4_slices(M, N, K, 2, true);
  return s > 0 ? kGemmCounterBytes + f4_region_bytes(N, K, s) : 0;
}

size_t workspace_f4_offset(int32_t M, int32_t N, int32_t K) {
  return workspace_gemm_offset(M, N, K) + gemm_partial_bytes(M, N, K) +
         skinny_partial_bytes(M, N, K);
}

size_t workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (M < 0 || M > HARP_MAX_M || N < 1 || N > HARP_MAX_DIM || K < 1 ||
      K > HARP_MAX_DIM)
    return 0;
  if (M == 0) return 0;
  // the f4 region is reserved for every bit width (the size query does not
  // know it)
  return workspace_f4_offset(M, N, K) + f4_region_bytes(N, K, f4_slices(M, N, K, 2, true));
}

size_t chain_ws_bytes(int32_t dim) { return chain_workspace_bytes(dim); }

harp_status validate_chain(const harp_chain_layer* layers, int32_t n_layers, const void* x,
                           int x_dt, int y_dt, int32_t M, const void* workspace,
                           size_t ws_bytes) {
  if (n_layers < 0) return HARP_ERR_SHAPE;
  if (n_layers == 0) return HARP_OK;
  if (layers == nullptr) return HARP_ERR_NULL;
  if (bad_dtype(x_dt) || bad_dtype(y_dt)) return HARP_ERR_DTYPE;
  HARP_TRY(check_m(M));
  const int32_t dim = layers[0].V.dim;
  for (int32_t l = 0; l < n_layers; ++l) {
    const harp_chain_layer& c = layers[l];
    HARP_TRY(check_rotation(&c.V));
    HARP_TRY(check_qweight(&c.W));
    HARP_TRY(check_rotation(&c.U));
    if (c.V.dim != dim || c.W.K != dim || c.W.N != dim || c.U.dim != dim) return HARP_ERR_SHAPE;
    if (c.W.bits != layers[0].W.bits) return HARP_ERR_UNSUPPORTED;
    if (dim != 4096 && dim != 8192) return HARP_ERR_UNSUPPORTED;
    if (c.V.block != dim || c.U.block != dim) return HARP_ERR_UNSUPPORTED;
    if (c.V.cs == nullptr || c.U.cs == nullptr) return HARP_ERR_UNSUPPORTED;
    HARP_TRY(check_data(c.y, M));
  }
  if (M > (dim == 4096 ? 4 : 2)) return HARP_ERR_UNSUPPORTED;
  HARP_TRY(check_data(x, M));
  if (M == 0) return HARP_OK;
  if (workspace == nullptr) return HARP_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return HARP_ERR_ALIGN;
  if (ws_bytes < chain_ws_bytes(dim)) return HARP_ERR_WORKSPACE;
  return HARP_OK;
}

const char* status_string(harp_status s) {
  switch (s) {
    case HARP_OK: return "HARP_OK";
    case HARP_ERR_NULL: return "HARP_ERR_NULL: a required pointer is NULL";
    case HARP_ERR_SHAPE: return "HARP_ERR_SHAPE: inconsistent or out-of-range dimension";
    case HARP_ERR_DTYPE: return "HARP_ERR_DTYPE: unknown dtype";
    case HARP_ERR_ALIGN: return "HARP_ERR_ALIGN: pointer not aligned (16 B data, 256 B workspace)";
    case HARP_ERR_WORKSPACE: return "HARP_ERR_WORKSPACE: workspace missing or too small";
    case HARP_ERR_UNSUPPORTED: return "HARP_ERR_UNSUPPORTED: bits not in {2,3,4}, group != 64 or block > 8192";
    case HARP_ERR_HIP: return "HARP_ERR_HIP: a HIP launch failed";
  }
  return "unknown harp_status";
}

}  // namespace harp
