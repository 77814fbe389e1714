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
harp_status validate_gemm(const harp_qweight* W, const void* xt, const void* yt,
                          int32_t M);
harp_status validate_fused(const harp_rotation* V, const harp_qweight* W,
                           const harp_rotation* U, const void* x, int x_dt,
                           const void* y, int y_dt, int32_t M,
                           const void* workspace, size_t ws_bytes);
harp_status validate_dequant(const harp_qweight* W, const void* out, int out_dt);

// Workspace layout of the fused linear: x~ first, then y' (both 256-byte
// aligned).  x~ is float32 below kGemmMinM rows and bf16 from there on.
constexpr int32_t kGemmMinM = 64;
size_t workspace_bytes(int32_t M, int32_t N, int32_t K);
size_t workspace_yp_offset(int32_t M, int32_t K);

const char* status_string(harp_status s);

}  // namespace harp
