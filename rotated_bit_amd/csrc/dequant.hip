// Test hook: dense w_hat [N][K] through the same unpack and dequant code the
// products use, as float32 (exact) or bf16 (round to nearest even, the
// matrix-core operand).  Not on the hot path.
#include "launch.hpp"
#include "unpack.hpp"

namespace harp {
namespace {

template <int BITS>
__global__ __launch_bounds__(256) void dequant_kernel(
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint16_t* __restrict__ zr, void* __restrict__ out, int out_dt, int N,
    int K) {
  const int runs = K / 32;
  const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<size_t>(N) * runs) return;
  const int n = static_cast<int>(idx / runs);
  const int r = static_cast<int>(idx - static_cast<size_t>(n) * runs);
  const size_t WPR = static_cast<size_t>(K) * BITS / 32;
  const size_t gi = static_cast<size_t>(n) * (K / kGroup) + r / 2;
  uint32_t w[BITS];
  load_run32<BITS>(qw + static_cast<size_t>(n) * WPR, r * BITS, w);
  float f[32];
  dequant_run32<BITS>(w, f16_to_f32(sc[gi]), f16_to_f32(zr[gi]), f);
  const size_t o = static_cast<size_t>(n) * K + static_cast<size_t>(r) * 32;
  if (out_dt == HARP_F32) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + o);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      p[i] = make_float4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
  } else {
    uint4* p = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + o);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      p[i] = make_uint4(pack_bf16x2(f[8 * i], f[8 * i + 1]),
                        pack_bf16x2(f[8 * i + 2], f[8 * i + 3]),
                        pack_bf16x2(f[8 * i + 4], f[8 * i + 5]),
                        pack_bf16x2(f[8 * i + 6], f[8 * i + 7]));
  }
}

template <int BITS>
hipError_t launch_bits(const harp_qweight& W, void* out, int out_dt,
                       hipStream_t stream) {
  const size_t total = static_cast<size_t>(W.N) * (W.K / 32);
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
  hipLaunchKernelGGL((dequant_kernel<BITS>), grid, dim3(256), 0, stream,
                     W.qweight, W.scale, W.zero, out, out_dt, W.N, W.K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(const harp_qweight& W, void* out, int out_dt,
                          hipStream_t stream) {
  switch (W.bits) {
    case 2: return launch_bits<2>(W, out, out_dt, stream);
    case 3: return launch_bits<3>(W, out, out_dt, stream);
    case 4: return launch_bits<4>(W, out, out_dt, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace harp
