// Dequant GEMM for prefill batches on the bf16 matrix cores:
//     y'[m][n] = sum_k bf16(w_hat[n][k]) * x~_bf16[m][k],  float32 accumulate.
//
// gfx950 mapping.  A workgroup of four waves computes a 128 (rows of x~) x
// 128 (output features) tile; each wave owns a 64 x 64 quarter as 2 x 2
// v_mfma_f32_32x32x16_bf16 accumulators.  K advances one quantization group
// (64) per step: the x~ tile is copied to LDS, and the packed weight tile is
// unpacked, dequantized to float32 (exact), rounded to bf16 and written to
// LDS, so each weight is dequantized once per tile.  LDS rows are padded to
// 144 bytes to spread the 16-byte fragment reads over the banks.  Global
// loads for the next step are issued before the barrier that retires the
// current step's matrix-core reads.
#include "launch.hpp"
#include "unpack.hpp"

namespace harp {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = kGroup;
constexpr int LDK = BK + 8;   // bf16 elements per padded LDS row

template <int BITS>
__global__ __launch_bounds__(256) void gemm_kernel(
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint16_t* __restrict__ zr, const uint16_t* __restrict__ xt,
    float* __restrict__ yt, int N, int K, int M) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[BN * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int wm = (wave >> 1) * 64;
  const int wn = (wave & 1) * 64;
  const size_t WPR = static_cast<size_t>(K) * BITS / 32;
  const int G = K / kGroup;

  // loader role: row lr of both tiles, half lh (32 of the 64 k values)
  const int lr = tid >> 1;
  const int lh = tid & 1;
  const int am = m0 + lr;
  const bool a_ok = am < M;
  const int bn = n0 + lr;
  const bool b_ok = bn < N;
  const uint16_t* arow = xt + static_cast<size_t>(a_ok ? am : 0) * K + lh * 32;
  const uint32_t* brow = qw + static_cast<size_t>(b_ok ? bn : 0) * WPR;
  const size_t sz_row = static_cast<size_t>(b_ok ? bn : 0) * G;

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int frag_row = lane & 31;
  const int frag_k = 8 * (lane >> 5);

  for (int kt = 0; kt < G; ++kt) {
    uint4 av[4];
    if (a_ok) {
      const uint4* p = reinterpret_cast<const uint4*>(arow + static_cast<size_t>(kt) * BK);
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = p[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = make_uint4(0, 0, 0, 0);
    }
    uint32_t w[BITS];
    float s = 0.0f, z = 0.0f;
    if (b_ok) {
      load_run32<BITS>(brow, (2 * kt + lh) * BITS, w);
      s = f16_to_f32(sc[sz_row + kt]);
      z = f16_to_f32(zr[sz_row + kt]);
    } else {
#pragma unroll
      for (int i = 0; i < BITS; ++i) w[i] = 0u;
    }
    float f[32];
    dequant_run32<BITS>(w, s, z, f);
    uint4 bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bv[i].x = pack_bf16x2(f[8 * i + 0], f[8 * i + 1]);
      bv[i].y = pack_bf16x2(f[8 * i + 2], f[8 * i + 3]);
      bv[i].z = pack_bf16x2(f[8 * i + 4], f[8 * i + 5]);
      bv[i].w = pack_bf16x2(f[8 * i + 6], f[8 * i + 7]);
    }
    __syncthreads();   // the previous step's fragment reads are done
    uint4* da = reinterpret_cast<uint4*>(sA + lr * LDK + lh * 32);
    uint4* db = reinterpret_cast<uint4*>(sB + lr * LDK + lh * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      da[i] = av[i];
      db[i] = bv[i];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(
            sA + (wm + 32 * i + frag_row) * LDK + kk * 16 + frag_k);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(
            sB + (wn + 32 * j + frag_row) * LDK + kk * 16 + frag_k);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // 32x32 accumulator layout: column = lane % 32,
  // row = 8 * (v / 4) + 4 * (lane / 32) + v % 4.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn + 32 * j + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < M && n < N) yt[static_cast<size_t>(m) * N + n] = acc[i][j][v];
      }
    }
  }
}

template <int BITS>
hipError_t launch_bits(const harp_qweight& W, const uint16_t* xt, float* yt,
                       int M, hipStream_t stream) {
  const dim3 grid((W.N + BN - 1) / BN, (M + BM - 1) / BM);
  hipLaunchKernelGGL((gemm_kernel<BITS>), grid, dim3(256), 0, stream, W.qweight,
                     W.scale, W.zero, xt, yt, W.N, W.K, M);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const harp_qweight& W, const uint16_t* xt, float* yt,
                       int M, hipStream_t stream) {
  switch (W.bits) {
    case 2: return launch_bits<2>(W, xt, yt, M, stream);
    case 3: return launch_bits<3>(W, xt, yt, M, stream);
    case 4: return launch_bits<4>(W, xt, yt, M, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace harp
