// Host-only driver of libharp's argument checks (rotated_bit_amd/csrc/
// validate.cpp), built with AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_validate_sanitized.py.  It walks every error path of every
// check (NULL structures and fields, unsupported formats, shapes, dtypes,
// batch range, data pointers, alignment, workspace size) and sweeps extreme
// integer arguments through the checks and the workspace-size functions.
// Pointers are stand-in addresses that are never dereferenced.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include <limits>

#include "../../rotated_bit_amd/csrc/validate.hpp"

using namespace harp;

static int g_fail = 0;

#define EXPECT(expr, want)                                                        \
  do {                                                                            \
    const int got_ = static_cast<int>(expr);                                      \
    if (got_ != static_cast<int>(want)) {                                         \
      std::fprintf(stderr, "%s:%d: %s = %d, want %d\n", __FILE__, __LINE__, #expr, \
                   got_, static_cast<int>(want));                                 \
      ++g_fail;                                                                   \
    }                                                                             \
  } while (0)

static const void* addr(uintptr_t a) { return reinterpret_cast<const void*>(a); }
static const void* const A = addr(0x10000);    // 256-byte aligned stand-in
static const void* const MIS = addr(0x10008);  // not 16-byte aligned

static harp_rotation rot(int32_t dim, int32_t block) {
  harp_rotation r{};
  r.dim = dim;
  r.block = block;
  r.cs = static_cast<const float*>(A);
  r.sign_bits = static_cast<const uint32_t*>(A);
  return r;
}

static harp_qweight qw(int32_t N, int32_t K, int32_t bits = 2) {
  harp_qweight w{};
  w.N = N;
  w.K = K;
  w.bits = bits;
  w.group = 64;
  w.qweight = static_cast<const uint32_t*>(A);
  w.scale = static_cast<const uint16_t*>(A);
  w.zero = static_cast<const uint16_t*>(A);
  return w;
}

static harp_mixed_rotation mixed(std::initializer_list<int> radices) {
  harp_mixed_rotation r{};
  int32_t d = 1;
  for (int b : radices) {
    r.radix[r.n_stages++] = b;
    d *= b;
  }
  r.dim = d;
  r.blocks = static_cast<const float*>(A);
  r.sign_bits = static_cast<const uint32_t*>(A);
  return r;
}

static void rotation_checks() {
  harp_rotation r = rot(4096, 4096);
  EXPECT(check_rotation(&r), HARP_OK);
  EXPECT(check_rotation(nullptr), HARP_ERR_NULL);
  r = rot(4096, 4096); r.sign_bits = nullptr; EXPECT(check_rotation(&r), HARP_ERR_NULL);
  r = rot(4096, 4096); r.cs = nullptr; EXPECT(check_rotation(&r), HARP_ERR_NULL);
  r = rot(4096, 4096); r.phi_codes = static_cast<const int8_t*>(A);
  EXPECT(check_rotation(&r), HARP_ERR_SHAPE);                       // both formats
  r = rot(4096, 4096); r.cs = nullptr; r.phi_codes = static_cast<const int8_t*>(A);
  r.phi_step = 0.01f; EXPECT(check_rotation(&r), HARP_OK);
  r.phi_step = std::numeric_limits<float>::quiet_NaN(); EXPECT(check_rotation(&r), HARP_ERR_SHAPE);
  r.phi_step = std::numeric_limits<float>::infinity(); EXPECT(check_rotation(&r), HARP_ERR_SHAPE);
  r = rot(16384, 16384); EXPECT(check_rotation(&r), HARP_ERR_UNSUPPORTED);
  r = rot(4096, 3); EXPECT(check_rotation(&r), HARP_ERR_SHAPE);
  r = rot(4096, 1); EXPECT(check_rotation(&r), HARP_ERR_SHAPE);
  r = rot(4096, 0); EXPECT(check_rotation(&r), HARP_ERR_SHAPE);
  r = rot(4096, -2); EXPECT(check_rotation(&r), HARP_ERR_SHAPE);
  r = rot(4100, 256); EXPECT(check_rotation(&r), HARP_ERR_SHAPE);
  r = rot(0, 2); EXPECT(check_rotation(&r), HARP_ERR_SHAPE);
  r = rot(HARP_MAX_DIM + 256, 256); EXPECT(check_rotation(&r), HARP_ERR_SHAPE);
  r = rot(4096, 4096); r.cs = static_cast<const float*>(MIS); EXPECT(check_rotation(&r), HARP_ERR_ALIGN);
  r = rot(4096, 4096); r.sign_bits = static_cast<const uint32_t*>(MIS);
  EXPECT(check_rotation(&r), HARP_ERR_ALIGN);
}

static void qweight_checks() {
  harp_qweight w = qw(4096, 4096);
  EXPECT(check_qweight(&w), HARP_OK);
  EXPECT(check_qweight(nullptr), HARP_ERR_NULL);
  w = qw(4096, 4096); w.qweight = nullptr; EXPECT(check_qweight(&w), HARP_ERR_NULL);
  w = qw(4096, 4096); w.scale = nullptr; EXPECT(check_qweight(&w), HARP_ERR_NULL);
  w = qw(4096, 4096); w.zero = nullptr; EXPECT(check_qweight(&w), HARP_ERR_NULL);
  for (int b : {0, 1, 5, 8, -3}) { w = qw(64, 64, b); EXPECT(check_qweight(&w), HARP_ERR_UNSUPPORTED); }
  w = qw(64, 64); w.group = 128; EXPECT(check_qweight(&w), HARP_ERR_UNSUPPORTED);
  w = qw(0, 64); EXPECT(check_qweight(&w), HARP_ERR_SHAPE);
  w = qw(64, 32); EXPECT(check_qweight(&w), HARP_ERR_SHAPE);
  w = qw(64, 96); EXPECT(check_qweight(&w), HARP_ERR_SHAPE);
  w = qw(HARP_MAX_DIM + 1, 64); EXPECT(check_qweight(&w), HARP_ERR_SHAPE);
  w = qw(64, 64); w.scale = static_cast<const uint16_t*>(MIS); EXPECT(check_qweight(&w), HARP_ERR_ALIGN);
}

static void call_checks() {
  const harp_rotation V = rot(4096, 4096), U = rot(1024, 256);
  const harp_qweight W = qw(1024, 4096);
  // rotate in / out
  EXPECT(validate_rotate_in(&V, A, HARP_BF16, A, HARP_F32, 1), HARP_OK);
  EXPECT(validate_rotate_in(&V, A, 7, A, HARP_F32, 1), HARP_ERR_DTYPE);
  EXPECT(validate_rotate_in(&V, A, HARP_F32, A, -1, 1), HARP_ERR_DTYPE);
  EXPECT(validate_rotate_in(&V, A, HARP_F32, A, HARP_F32, -1), HARP_ERR_SHAPE);
  EXPECT(validate_rotate_in(&V, A, HARP_F32, A, HARP_F32, HARP_MAX_M + 1), HARP_ERR_SHAPE);
  EXPECT(validate_rotate_in(&V, nullptr, HARP_F32, A, HARP_F32, 1), HARP_ERR_NULL);
  EXPECT(validate_rotate_in(&V, nullptr, HARP_F32, nullptr, HARP_F32, 0), HARP_OK);
  EXPECT(validate_rotate_in(&V, MIS, HARP_F32, A, HARP_F32, 1), HARP_ERR_ALIGN);
  EXPECT(validate_rotate_out(&U, A, A, HARP_BF16, 3), HARP_OK);
  EXPECT(validate_rotate_out(&U, A, nullptr, HARP_BF16, 3), HARP_ERR_NULL);
  EXPECT(validate_rotate_out(&U, A, A, 2, 3), HARP_ERR_DTYPE);
  // products
  EXPECT(validate_gemv(&W, A, A, 5), HARP_OK);
  EXPECT(validate_gemv(&W, A, MIS, 5), HARP_ERR_ALIGN);
  EXPECT(validate_rotate_gemv(&V, &W, A, HARP_BF16, A, 1), HARP_OK);
  const harp_rotation V2 = rot(2048, 2048);
  EXPECT(validate_rotate_gemv(&V2, &W, A, HARP_BF16, A, 1), HARP_ERR_SHAPE);
  EXPECT(validate_gemm(&W, A, A, 512, nullptr, 0), HARP_OK);
  const size_t g = gemm_workspace_bytes(512, 1024, 4096);
  EXPECT(validate_gemm(&W, A, A, 512, A, g), HARP_OK);
  if (g > 0) EXPECT(validate_gemm(&W, A, A, 512, A, g - 1), HARP_ERR_WORKSPACE);
  EXPECT(validate_gemm(&W, A, A, 512, addr(0x10010), g), HARP_ERR_ALIGN);
  // fused
  const size_t f = workspace_bytes(16, 1024, 4096);
  EXPECT(validate_fused(&V, &W, &U, A, HARP_BF16, A, HARP_F32, 16, A, f), HARP_OK);
  EXPECT(validate_fused(&V, &W, &U, A, HARP_BF16, A, HARP_F32, 16, A, f - 1), HARP_ERR_WORKSPACE);
  EXPECT(validate_fused(&V, &W, &U, A, HARP_BF16, A, HARP_F32, 16, nullptr, f), HARP_ERR_WORKSPACE);
  EXPECT(validate_fused(&V, &W, &U, A, HARP_BF16, A, HARP_F32, 16, addr(0x10040), f), HARP_ERR_ALIGN);
  EXPECT(validate_fused(&V, &W, &V, A, HARP_BF16, A, HARP_F32, 16, A, f), HARP_ERR_SHAPE);
  EXPECT(validate_fused(&V, &W, &U, A, HARP_BF16, A, 9, 16, A, f), HARP_ERR_DTYPE);
  EXPECT(validate_fused(&V, &W, &U, nullptr, HARP_BF16, nullptr, HARP_F32, 0, nullptr, 0), HARP_OK);
  EXPECT(validate_fused(nullptr, &W, &U, A, HARP_BF16, A, HARP_F32, 1, A, f), HARP_ERR_NULL);
  // dequant
  EXPECT(validate_dequant(&W, A, HARP_F32), HARP_OK);
  EXPECT(validate_dequant(&W, nullptr, HARP_F32), HARP_ERR_NULL);
  EXPECT(validate_dequant(&W, A, 4), HARP_ERR_DTYPE);
  // offline preparation
  const float* F = static_cast<const float*>(A);
  const size_t rw = rotate_weight_workspace_bytes(1024, 4096);
  EXPECT(validate_rotate_weight(&V, &U, F, F, 1024, 4096, A, rw), HARP_OK);
  EXPECT(validate_rotate_weight(&V, &U, F, F, 1024, 4096, A, rw - 1), HARP_ERR_WORKSPACE);
  EXPECT(validate_rotate_weight(&V, &U, nullptr, F, 1024, 4096, A, rw), HARP_ERR_NULL);
  EXPECT(validate_rotate_weight(&V, &U, F, F, 1024, 2048, A, rw), HARP_ERR_SHAPE);
  EXPECT(validate_rotate_weight(&V, &U, F, F, 0, 4096, A, rw), HARP_ERR_SHAPE);
  EXPECT(validate_quantize_pack(F, 1024, 4096, 2, A, A, A), HARP_OK);
  EXPECT(validate_quantize_pack(F, 1024, 4096, 5, A, A, A), HARP_ERR_UNSUPPORTED);
  EXPECT(validate_quantize_pack(F, 1024, 4000, 2, A, A, A), HARP_ERR_SHAPE);
  EXPECT(validate_quantize_pack(F, 1024, 4096, 2, nullptr, A, A), HARP_ERR_NULL);
  EXPECT(validate_quantize_pack(F, 1024, 4096, 2, A, MIS, A), HARP_ERR_ALIGN);
  // mixed radix
  const harp_mixed_rotation R = mixed({8, 8, 8, 5, 2}), R2 = mixed({8, 4});
  const harp_qweight W5 = qw(5120, 5120);
  EXPECT(validate_rotate_mixed(&R, A, HARP_BF16, A, HARP_F32, 4, nullptr, 0), HARP_OK);
  const size_t mw = rotate_mixed_workspace_bytes(5120, 4, HARP_BF16);
  EXPECT(validate_rotate_mixed(&R, A, HARP_BF16, A, HARP_BF16, 4, A, mw), HARP_OK);
  EXPECT(validate_rotate_mixed(&R, A, HARP_BF16, A, HARP_BF16, 4, A, mw - 1), HARP_ERR_WORKSPACE);
  harp_mixed_rotation bad = mixed({8, 8, 8, 5, 2}); bad.dim = 5121;
  EXPECT(validate_rotate_mixed(&bad, A, HARP_BF16, A, HARP_F32, 4, nullptr, 0), HARP_ERR_SHAPE);
  bad = mixed({65, 2}); EXPECT(validate_rotate_mixed(&bad, A, HARP_F32, A, HARP_F32, 1, nullptr, 0),
                               HARP_ERR_UNSUPPORTED);
  bad = mixed({8, 8}); bad.n_stages = 0;
  EXPECT(validate_rotate_mixed(&bad, A, HARP_F32, A, HARP_F32, 1, nullptr, 0), HARP_ERR_SHAPE);
  bad = mixed({8, 8}); bad.n_stages = HARP_MAX_STAGES + 1;
  EXPECT(validate_rotate_mixed(&bad, A, HARP_F32, A, HARP_F32, 1, nullptr, 0), HARP_ERR_SHAPE);
  bad = mixed({8, 8}); bad.radix[1] = 1;
  EXPECT(validate_rotate_mixed(&bad, A, HARP_F32, A, HARP_F32, 1, nullptr, 0), HARP_ERR_SHAPE);
  bad = mixed({8, 8}); bad.blocks = nullptr;
  EXPECT(validate_rotate_mixed(&bad, A, HARP_F32, A, HARP_F32, 1, nullptr, 0), HARP_ERR_NULL);
  const size_t lm = mixed_workspace_bytes(16, 5120, 5120);
  EXPECT(validate_fused_mixed(&R, &W5, &R, A, HARP_BF16, A, HARP_F32, 16, A, lm), HARP_OK);
  EXPECT(validate_fused_mixed(&R, &W5, &R, A, HARP_BF16, A, HARP_F32, 16, A, lm - 1),
         HARP_ERR_WORKSPACE);
  EXPECT(validate_fused_mixed(&R, &W5, &R2, A, HARP_BF16, A, HARP_F32, 16, A, lm), HARP_ERR_SHAPE);
  // status strings
  for (int s = 0; s <= 8; ++s) (void)status_string(static_cast<harp_status>(s));
}

// Extreme integers through every check and size function: only the
// sanitizers judge (no overflow, no out-of-bounds); statuses must stay in
// the enum and sizes must be 0 for out-of-range arguments.
static void sweep() {
  const int32_t vals[] = {std::numeric_limits<int32_t>::min(), -65536, -64, -1, 0, 1, 2, 63, 64,
                          65, 128, 4096, 8192, 65536, 65537, HARP_MAX_DIM, HARP_MAX_DIM + 64,
                          std::numeric_limits<int32_t>::max()};
  for (int32_t a : vals) {
    for (int32_t b : vals) {
      for (int32_t c : vals) {
        const size_t w = workspace_bytes(a, b, c);
        const size_t m = mixed_workspace_bytes(a, b, c);
        if (a < 0 || a > HARP_MAX_M) {
          EXPECT(w, 0u);
          EXPECT(m, 0u);
        }
      }
      (void)rotate_weight_workspace_bytes(a, b);
      (void)rotate_mixed_workspace_bytes(a, b, HARP_BF16);
      harp_rotation r = rot(a, b);
      const int s = check_rotation(&r);
      if (s < 0 || s > 7) ++g_fail;
      harp_qweight q = qw(a, b);
      const int t = check_qweight(&q);
      if (t < 0 || t > 7) ++g_fail;
      if (t == HARP_OK) {
        for (int32_t m : vals) {
          const int u = validate_gemm(&q, A, A, m, A, std::numeric_limits<size_t>::max());
          if (u < 0 || u > 7) ++g_fail;
        }
      }
    }
  }
}

int main() {
  rotation_checks();
  qweight_checks();
  call_checks();
  sweep();
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("validate: all checks passed\n");
  return 0;
}
