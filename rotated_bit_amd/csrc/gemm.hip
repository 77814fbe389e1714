// Dequant GEMM for prefill batches on the bf16 matrix cores:
//     y'[m][n] = sum_k bf16(w_hat[n][k]) * x~_bf16[m][k],  float32 accumulate.
//
// gfx950 mapping.  A workgroup of four waves computes a 128 (rows of x~) x
// 128 (output features) tile; each wave owns a 64 x 64 quarter as 2 x 2
// v_mfma_f32_32x32x16_bf16 accumulators.  K advances one quantization group
// (64) per step: the x~ tile is copied to LDS, and the packed weight tile is
// unpacked, dequantized to float32 (exact), rounded to bf16 and written to
// LDS, so each weight is dequantized once per tile.  LDS rows are padded to
// 144 bytes to spread the 16-byte fragment reads over the banks.  The
// K loop is software-pipelined: the global loads of step k+1 are issued
// right after step k is in LDS and complete while the matrix cores work on
// step k; LDS is double-buffered, so one barrier per step suffices.
#include "launch.hpp"
#include "unpack.hpp"

namespace harp {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = kGroup;
constexpr int LDK = BK + 8;   // bf16 elements per padded LDS row

// Global operands of one K step, held in registers between the load and
// the LDS store (the software-pipelined prefetch).
template <int BITS>
struct StepRegs {
  uint4 a[4];        // 32 bf16 of x~ (row lr, half lh)
  uint32_t w[BITS];  // 32 codes of weight row lr, half lh
  uint16_t s, z;
};

template <int BITS>
__device__ __forceinline__ void load_step(StepRegs<BITS>& r, int kt,
                                          const uint16_t* arow, bool a_ok,
                                          const uint32_t* brow, bool b_ok,
                                          const uint16_t* __restrict__ sc,
                                          const uint16_t* __restrict__ zr,
                                          size_t sz_row, int lh) {
  if (a_ok) {
    const uint4* p = reinterpret_cast<const uint4*>(arow + static_cast<size_t>(kt) * BK);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.a[i] = p[i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.a[i] = make_uint4(0, 0, 0, 0);
  }
  if (b_ok) {
    load_run32<BITS>(brow, (2 * kt + lh) * BITS, r.w);
    r.s = sc[sz_row + kt];
    r.z = zr[sz_row + kt];
  } else {
#pragma unroll
    for (int i = 0; i < BITS; ++i) r.w[i] = 0u;
    r.s = 0;   // scale 0: the padded rows dequantize to 0
    r.z = 0;
  }
}

template <int BITS>
__device__ __forceinline__ void store_step(const StepRegs<BITS>& r, uint16_t* sA,
                                           uint16_t* sB, int lr, int lh) {
  float f[32];
  dequant_run32<BITS>(r.w, f16_to_f32(r.s), f16_to_f32(r.z), f);
  uint4* da = reinterpret_cast<uint4*>(sA + lr * LDK + lh * 32);
  uint4* db = reinterpret_cast<uint4*>(sB + lr * LDK + lh * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    da[i] = r.a[i];
    db[i] = make_uint4(pack_bf16x2(f[8 * i + 0], f[8 * i + 1]),
                       pack_bf16x2(f[8 * i + 2], f[8 * i + 3]),
                       pack_bf16x2(f[8 * i + 4], f[8 * i + 5]),
                       pack_bf16x2(f[8 * i + 6], f[8 * i + 7]));
  }
}

template <int BITS>
__global__ __launch_bounds__(256) void gemm_kernel(
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint16_t* __restrict__ zr, const uint16_t* __restrict__ xt,
    float* __restrict__ yt, int N, int K, int M) {
  // two LDS stages: step kt is read from stage kt & 1 while step kt + 1 is
  // written to the other
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * LDK];

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

  StepRegs<BITS> regs;
  load_step<BITS>(regs, 0, arow, a_ok, brow, b_ok, sc, zr, sz_row, lh);
  for (int kt = 0; kt < G; ++kt) {
    const int st = kt & 1;
    store_step<BITS>(regs, sA[st], sB[st], lr, lh);
    __syncthreads();   // stage st complete; stage st^1 no longer read
    if (kt + 1 < G)
      load_step<BITS>(regs, kt + 1, arow, a_ok, brow, b_ok, sc, zr, sz_row, lh);
    const uint16_t* pa = sA[st];
    const uint16_t* pb = sB[st];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(
            pa + (wm + 32 * i + frag_row) * LDK + kk * 16 + frag_k);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(
            pb + (wn + 32 * j + frag_row) * LDK + kk * 16 + frag_k);
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
