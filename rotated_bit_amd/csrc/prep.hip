// Offline preparation on the GPU (HARP technical summary §2.4: the rotated
// weight W' = F_U W F_V^T is what the quantization backend receives; §5: an
// exact change of basis before quantization).
//
//   * transpose_kernel: float32 [R][C] -> [C][R] through 64 x 64 LDS tiles
//     (padded rows, coalesced reads and writes), used to apply F_U along the
//     columns of W with the row rotation kernel.
//   * quantize_pack_kernel: the per-row, per-group uniform grid of the
//     packed weight format.  One wave per (row, group of 64): lane j holds
//     w_j; min and max are exact wave reductions; scale, zero and codes are
//     computed with one IEEE float32 operation per step, rounded to nearest
//     even, in this order:
//         lo = min(min w, 0), hi = max(max w, 0)  (-1, 1 when both are 0)
//         s  = fp16((hi - lo) / (2^B - 1)), at least 2^-14
//         z  = clamp(rint(-lo / s), 0, 2^B - 1) + 0   (+0 for a zero z)
//         q  = clamp(rint(w / s) + z, 0, 2^B - 1)
//     The codes are packed into the boundary words through the wave's LDS
//     bytes (2 and 4 bits: 32/B codes per word, least significant first;
//     3 bits: 32-code runs as 96-bit little-endian integers).
#include "launch.hpp"
#include "device_common.hpp"

namespace harp {
namespace {

constexpr int kTile = 64;
constexpr int kTransposeThreads = 256;

__global__ __launch_bounds__(kTransposeThreads) void transpose_kernel(
    const float* __restrict__ in, float* __restrict__ out, int R, int C) {
  __shared__ float tile[kTile][kTile + 1];
  const int c0 = blockIdx.x * kTile;
  const int r0 = blockIdx.y * kTile;
  const int tx = threadIdx.x & (kTile - 1);
  const int ty = threadIdx.x >> 6;              // 0..3
#pragma unroll
  for (int i = 0; i < kTile; i += kTransposeThreads / kTile) {
    const int r = r0 + ty + i;
    const int c = c0 + tx;
    if (r < R && c < C) tile[ty + i][tx] = in[static_cast<size_t>(r) * C + c];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kTile; i += kTransposeThreads / kTile) {
    const int c = c0 + ty + i;                  // output row
    const int r = r0 + tx;                      // output column
    if (c < C && r < R) out[static_cast<size_t>(c) * R + r] = tile[tx][ty + i];
  }
}

constexpr int kQuantWaves = 4;
constexpr int kGroupCodes = 64;            // quantization group along K

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

template <int BITS>
__global__ __launch_bounds__(kQuantWaves * kWave) void quantize_pack_kernel(
    const float* __restrict__ wp, uint32_t* __restrict__ qw, uint16_t* __restrict__ sc,
    uint16_t* __restrict__ zr, int N, int K) {
  __shared__ uint8_t codes[kQuantWaves][kGroupCodes];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int G = K / kGroupCodes;
  const long long gid = static_cast<long long>(blockIdx.x) * kQuantWaves + wave;
  if (gid >= static_cast<long long>(N) * G) return;   // whole wave
  const int row = static_cast<int>(gid / G);
  const int g = static_cast<int>(gid - static_cast<long long>(row) * G);
  constexpr float qmax = static_cast<float>((1 << BITS) - 1);

  const float w = wp[static_cast<size_t>(row) * K + static_cast<size_t>(g) * kGroupCodes + lane];
  float lo = fminf(wave_min(w), 0.0f);
  float hi = fmaxf(wave_max(w), 0.0f);
  if (hi == lo) {
    lo = -1.0f;
    hi = 1.0f;
  }
  const float range = hi - lo;
  _Float16 s16 = static_cast<_Float16>(range / qmax);
  if (static_cast<float>(s16) < 6.103515625e-05f) s16 = static_cast<_Float16>(6.103515625e-05f);
  const float s = static_cast<float>(s16);
  const float neg_lo = -lo;
  const float z = fminf(fmaxf(rintf(neg_lo / s), 0.0f), qmax) + 0.0f;
  const float q = fminf(fmaxf(rintf(w / s) + z, 0.0f), qmax);

  codes[wave][lane] = static_cast<uint8_t>(q);
  if (lane == 0) {
    sc[static_cast<size_t>(row) * G + g] = __builtin_bit_cast(uint16_t, s16);
    zr[static_cast<size_t>(row) * G + g] =
        __builtin_bit_cast(uint16_t, static_cast<_Float16>(z));
  }
  // The wave's 64 code bytes are in LDS (one wave: program order suffices);
  // lanes 0 .. 2*BITS-1 each assemble one word of the group.
  constexpr int NW = 2 * BITS;
  if (lane < NW) {
    uint32_t word = 0;
    if constexpr (BITS == 2 || BITS == 4) {
      constexpr int PER = 32 / BITS;
#pragma unroll
      for (int j = 0; j < PER; ++j)
        word |= static_cast<uint32_t>(codes[wave][lane * PER + j]) << (BITS * j);
    } else {
      // word lane of the group: run lane / 3, word lane % 3 of that run's
      // 96 bits; code j of the run occupies bits 3j .. 3j + 2
      const int run = lane / 3;
      const int wi = lane - 3 * run;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint32_t c = codes[wave][32 * run + j];
        const int pos = 3 * j - 32 * wi;        // bit position inside this word
        if (pos >= 0 && pos < 32) word |= c << pos;
        else if (pos < 0 && pos > -3) word |= c >> (-pos);
      }
    }
    qw[static_cast<size_t>(row) * (static_cast<size_t>(K) * BITS / 32) +
       static_cast<size_t>(g) * NW + lane] = word;
  }
}

}  // namespace

hipError_t launch_transpose(const float* in, float* out, int R, int C, hipStream_t stream) {
  const dim3 grid((C + kTile - 1) / kTile, (R + kTile - 1) / kTile);
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(kTransposeThreads), 0, stream, in, out, R, C);
  return hipGetLastError();
}

hipError_t launch_quantize_pack(const float* wp, int N, int K, int bits, uint32_t* qw,
                                uint16_t* sc, uint16_t* zr, hipStream_t stream) {
  const long long groups = static_cast<long long>(N) * (K / kGroupCodes);
  const dim3 grid(static_cast<unsigned>((groups + kQuantWaves - 1) / kQuantWaves));
  const dim3 block(kQuantWaves * kWave);
  switch (bits) {
    case 2:
      hipLaunchKernelGGL(quantize_pack_kernel<2>, grid, block, 0, stream, wp, qw, sc, zr, N, K);
      break;
    case 3:
      hipLaunchKernelGGL(quantize_pack_kernel<3>, grid, block, 0, stream, wp, qw, sc, zr, N, K);
      break;
    case 4:
      hipLaunchKernelGGL(quantize_pack_kernel<4>, grid, block, 0, stream, wp, qw, sc, zr, N, K);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace harp
