// Dequant GEMM for small batches (M <= 64) on the bf16 matrix cores:
//     y'[m][n] = sum_k w_hat[n][k] * x~_bf16[m][k],  float32 accumulate,
// with w_hat = (q - z) s applied exactly: per quantization group g of 64
// inputs the matrix cores form T = sum_k (128 + q_k) x~_k (the codes enter
// as the exact bf16 values 128 + q) and S = sum_k x~_k (against a constant
// all-ones operand), and the group adds s (T - (128 + z) S) in float32.
// Only x~ is rounded (to bf16, by the caller); the large-batch GEMM instead
// rounds w_hat to bf16.
//
// gfx950 mapping.  A workgroup of eight waves owns a strip of 16 output
// features; wave w takes the w-th eighth of the quantization groups along
// K.  Per group (two k-slices of v_mfma_f32_16x16x32_bf16) lane l supplies
// feature n = l % 16 and inputs 8c .. 8c+7 of each slice, c = l / 16: it
// loads that feature's group of codes (16/24/32 bytes, shared with the three
// other lanes of the feature through the L1) and turns its 16 codes into the
// B operand with one AND-OR per two codes.  x~ is read with coalesced loads
// and passed through a per-wave LDS block into operand order.  Each code is fetched once; there
// are no LDS operand tiles and no barriers in the K loop, and the loads of
// the next groups are in flight while a group is multiplied.  The
// eight waves' partial sums are combined through LDS in wave order 0..7, so
// the result is bitwise reproducible.
#include "launch.hpp"
#include "unpack.hpp"

namespace harp {
namespace {

constexpr int kWavesS = 8;
constexpr int kThreadsS = kWavesS * kWave;   // 512
constexpr int kStrip = 16;                   // output features per workgroup

typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kXsRow = kGroup + 8;        // bf16 per padded LDS row of x~

// Operands of one quantization group for one lane.  x~ is loaded coalesced
// (eight lanes per 128-byte row segment: lane l holds row 8i + l/8, inputs
// 8 (l % 8) .. +7 of the group, i = 0, 1) and re-laid out through LDS into
// the matrix-core operand order, where neighbouring lanes read different
// rows.
template <int BITS, int MB>
struct GroupRegs {
  uint32_t w[2 * BITS];      // the feature's 64 codes
  uint16_t s16, z16;         // its fp16 scale and zero
  u32x4 a[MB][2];            // x~ rows 16 mb + 8 i + l/8, inputs 8 (l % 8) .. +7
};

template <int BITS, int MB>
__device__ __forceinline__ void load_group_regs(GroupRegs<BITS, MB>& r, int g,
                                                const uint32_t* __restrict__ wrow,
                                                const uint16_t* __restrict__ srow,
                                                const uint16_t* __restrict__ zrow,
                                                const uint16_t* const (&arow)[MB][2], int lane) {
  load_group<BITS>(wrow + static_cast<size_t>(g) * 2 * BITS, r.w);
  r.s16 = srow[g];
  r.z16 = zrow[g];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 2; ++i)
      r.a[mb][i] = *reinterpret_cast<const u32x4*>(arow[mb][i] + g * kGroup + 8 * (lane & 7));
}

template <int BITS, int MB>
__device__ __forceinline__ void mma_group(const GroupRegs<BITS, MB>& r, int lane,
                                          uint16_t (*xs)[16][kXsRow],
                                          floatx4_t (&acc)[MB]) {
  const int c = lane >> 4;
  // This wave's x~ block of the group into its own LDS rows (no other wave
  // touches them, so program order within the wave is the only ordering).
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4*>(&xs[mb][8 * i + (lane >> 3)][8 * (lane & 7)]) = r.a[mb][i];
  constexpr uint32_t kOnes = 0x3f803f80u;    // two bf16 1.0
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{kOnes, kOnes, kOnes, kOnes});
  floatx4_t t[MB], sx[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    t[mb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    sx[mb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, chunk8_bf16_offset<BITS>(chunk8<BITS>(r.w, h, c)));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&xs[mb][lane & 15][32 * h + 8 * c]);
      t[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, t[mb], 0, 0, 0);
      sx[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ones, sx[mb], 0, 0, 0);
    }
  }
  // Accumulator layout of a 16x16 block: lane l holds column (feature)
  // l % 16, so one scale and zero per lane.
  const float s = f16_to_f32(r.s16);
  const float zo = f16_to_f32(r.z16) + 128.0f;   // exact
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[mb][v] = fmaf(s, fmaf(-zo, sx[mb][v], t[mb][v]), acc[mb][v]);
}

template <int BITS, int MB>
__global__ __launch_bounds__(kThreadsS) void skinny_kernel(
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint16_t* __restrict__ zr, const uint16_t* __restrict__ xt,
    float* __restrict__ yt, int N, int K, int M) {
  __shared__ floatx4_t red[kWavesS][MB][kWave];
  __shared__ __attribute__((aligned(16))) uint16_t xsw[kWavesS][MB][16][kXsRow];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int G = K / kGroup;
  const size_t WPR = static_cast<size_t>(K) * BITS / 32;
  const int fl = lane & 15;          // feature within the strip (B column)
  const int n = min(blockIdx.x * kStrip + fl, N - 1);   // rows past N: never stored
  const uint32_t* wrow = qw + static_cast<size_t>(n) * WPR;
  const uint16_t* srow = sc + static_cast<size_t>(n) * G;
  const uint16_t* zrow = zr + static_cast<size_t>(n) * G;
  const uint16_t* arow[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)   // rows past M: read, never stored
#pragma unroll
    for (int i = 0; i < 2; ++i)
      arow[mb][i] = xt + static_cast<size_t>(min(16 * mb + 8 * i + (lane >> 3), M - 1)) * K;
  uint16_t (*xs)[16][kXsRow] = xsw[wave];

  floatx4_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // This wave's groups [gb, ge) through a ring of register sets (four, or
  // two for the widest batch block, whose x~ fragments fill the registers):
  // the loads of the next groups are in flight while a group is multiplied
  // (memory latency, not bandwidth, bounds a wave's progress here).  Loads
  // past ge re-read group ge-1 (valid memory, never multiplied).  Named sets,
  // not an array, keep the ring in registers.
  const int gb = wave * G / kWavesS;
  const int ge = (wave + 1) * G / kWavesS;
  if (gb < ge) {
    auto load = [&](GroupRegs<BITS, MB>& r, int g) {
      load_group_regs<BITS, MB>(r, min(g, ge - 1), wrow, srow, zrow, arow, lane);
    };
    if constexpr (MB <= 3) {
      GroupRegs<BITS, MB> r0, r1, r2, r3;
      load(r0, gb);
      load(r1, gb + 1);
      load(r2, gb + 2);
      load(r3, gb + 3);
      int g = gb;
      for (; g + 4 <= ge; g += 4) {
        mma_group<BITS, MB>(r0, lane, xs, acc);
        load(r0, g + 4);
        mma_group<BITS, MB>(r1, lane, xs, acc);
        load(r1, g + 5);
        mma_group<BITS, MB>(r2, lane, xs, acc);
        load(r2, g + 6);
        mma_group<BITS, MB>(r3, lane, xs, acc);
        load(r3, g + 7);
      }
      if (g < ge) mma_group<BITS, MB>(r0, lane, xs, acc);
      if (g + 1 < ge) mma_group<BITS, MB>(r1, lane, xs, acc);
      if (g + 2 < ge) mma_group<BITS, MB>(r2, lane, xs, acc);
    } else {
      GroupRegs<BITS, MB> r0, r1;
      load(r0, gb);
      load(r1, gb + 1);
      int g = gb;
      for (; g + 2 <= ge; g += 2) {
        mma_group<BITS, MB>(r0, lane, xs, acc);
        load(r0, g + 2);
        mma_group<BITS, MB>(r1, lane, xs, acc);
        load(r1, g + 3);
      }
      if (g < ge) mma_group<BITS, MB>(r0, lane, xs, acc);
    }
  }

  // Combine the eight K ranges in wave order.  Accumulator layout of the
  // 16x16 block: lane l holds column l % 16 and rows 4 * (l / 16) + v.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
  __syncthreads();
  for (int slot = tid; slot < MB * kWave * 4; slot += kThreadsS) {
    const int mb = slot / (kWave * 4);
    const int rem = slot - mb * kWave * 4;
    const int l = rem >> 2;
    const int v = rem & 3;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWavesS; ++w) sum += red[w][mb][l][v];
    const int m = 16 * mb + 4 * (l >> 4) + v;
    const int nn = blockIdx.x * kStrip + (l & 15);
    if (m < M && nn < N) yt[static_cast<size_t>(m) * N + nn] = sum;
  }
}

template <int BITS, int MB>
hipError_t launch_mb(const harp_qweight& W, const uint16_t* xt, float* yt, int M,
                     hipStream_t stream) {
  const dim3 grid((W.N + kStrip - 1) / kStrip);
  hipLaunchKernelGGL((skinny_kernel<BITS, MB>), grid, dim3(kThreadsS), 0, stream,
                     W.qweight, W.scale, W.zero, xt, yt, W.N, W.K, M);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const harp_qweight& W, const uint16_t* xt, float* yt, int M,
                       hipStream_t stream) {
  switch ((M + 15) / 16) {
    case 1: return launch_mb<BITS, 1>(W, xt, yt, M, stream);
    case 2: return launch_mb<BITS, 2>(W, xt, yt, M, stream);
    case 3: return launch_mb<BITS, 3>(W, xt, yt, M, stream);
    case 4: return launch_mb<BITS, 4>(W, xt, yt, M, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm_skinny(const harp_qweight& W, const uint16_t* xt, float* yt,
                              int M, hipStream_t stream) {
  switch (W.bits) {
    case 2: return launch_bits<2>(W, xt, yt, M, stream);
    case 3: return launch_bits<3>(W, xt, yt, M, stream);
    case 4: return launch_bits<4>(W, xt, yt, M, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace harp
