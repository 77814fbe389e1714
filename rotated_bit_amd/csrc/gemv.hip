// Dequant GEMV for decode batches: y'[m][n] = sum_k w_hat[n][k] x~[m][k],
// float32 throughout (w_hat is exact in float32, x~ is not rounded).
//
// gfx950 mapping.  A workgroup of eight waves owns 16 output rows, two per
// wave, and MT rows of x~.  K is walked in chunks of 4096 inputs (64
// quantization groups):
//   * the chunk of x~ is staged once in LDS with coalesced loads, padded to
//     68 floats per group so that each lane's 16-byte reads of its own
//     group are bank-conflict free; the sum of x~ over each group is formed
//     while staging (16 lanes per group, fixed butterfly order);
//   * lane l of every wave takes group l of the chunk: one contiguous
//     16/24/32-byte load of packed codes per row and one fp16 scale and zero
//     per row, all issued before the staging so they are in flight together.
// Per group the product is factored as
//     sum_k (q_k - z) s x~_k = s (sum_k q_k x~_k - z sum_k x~_k),
// which leaves one convert and MT fused multiply-adds per code.  A wave
// needs no other wave's data: its RW*MT partial sums are combined with a
// transposing reduction over its 64 lanes in a fixed order, so the result
// is bitwise reproducible.
#include "launch.hpp"
#include "unpack.hpp"

namespace harp {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;   // 512
constexpr int RW = 2;                      // output rows per wave
constexpr int kRowsPerWg = kWaves * RW;    // 16
constexpr int KC = 4096;                   // inputs per staged chunk
constexpr int GC = KC / kGroup;            // groups per chunk: one per lane
constexpr int kGStride = kGroup + 4;       // LDS floats per staged group

// One group (64 codes) of one row occupies 2*BITS words.
template <int BITS>
__device__ __forceinline__ void load_group(const uint32_t* __restrict__ p,
                                           uint32_t (&w)[2 * BITS]) {
  if constexpr (BITS == 2) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if constexpr (BITS == 4) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p);
    const u32x4 b = *reinterpret_cast<const u32x4*>(p + 4);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
    w[4] = b[0]; w[5] = b[1]; w[6] = b[2]; w[7] = b[3];
  } else {
    // 24 bytes per group: 8-byte aligned (the row stride is 24*G bytes).
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const uint2 v = *reinterpret_cast<const uint2*>(p + 2 * i);
      w[2 * i] = v.x;
      w[2 * i + 1] = v.y;
    }
  }
}

// Codes per segment of the inner loop: one word for 2- and 4-bit codes,
// 8 codes (24 bits) for 3-bit codes.
template <int BITS> struct Seg { static constexpr int CODES = BITS == 2 ? 16 : 8; };

// Codes of segment i of a group as floats, q[j] = code (i*CODES + j).
template <int BITS>
__device__ __forceinline__ void seg_codes(const uint32_t (&w)[2 * BITS], int i,
                                          float (&q)[Seg<BITS>::CODES]) {
  if constexpr (BITS == 2) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t m = opaque((w[i] >> (2 * t)) & 0x03030303u);  // codes t, t+4, t+8, t+12
#pragma unroll
      for (int b = 0; b < 4; ++b) q[t + 4 * b] = static_cast<float>((m >> (8 * b)) & 0xffu);
    }
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t m = opaque((w[i] >> (4 * t)) & 0x0f0f0f0fu);  // codes t, t+2, t+4, t+6
#pragma unroll
      for (int b = 0; b < 4; ++b) q[t + 2 * b] = static_cast<float>((m >> (8 * b)) & 0xffu);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = static_cast<float>(code_at<3, 6>(w, 8 * i + j));
  }
}

template <int BITS, int MT>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint16_t* __restrict__ zr, const float* __restrict__ xt,
    float* __restrict__ yt, int N, int K, int M) {
  constexpr int NWG = 2 * BITS;                 // words per group
  constexpr int SEG = Seg<BITS>::CODES;
  constexpr int V = RW * MT;
  __shared__ __attribute__((aligned(16))) float xs[MT][GC * kGStride];
  __shared__ float sxs[MT][GC];

  const int G = K / kGroup;
  const size_t WPR = static_cast<size_t>(K) * BITS / 32;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int rbase = blockIdx.x * kRowsPerWg + wave * RW;
  const int m0 = blockIdx.y * MT;

  const uint32_t* wrow[RW];
  const uint16_t* srow[RW];
  const uint16_t* zrow[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int n = min(rbase + r, N - 1);        // rows past N: loaded, never stored
    wrow[r] = qw + static_cast<size_t>(n) * WPR;
    srow[r] = sc + static_cast<size_t>(n) * G;
    zrow[r] = zr + static_cast<size_t>(n) * G;
  }

  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.0f;

  for (int g0 = 0; g0 < G; g0 += GC) {
    const int ng = min(GC, G - g0);
    const int g = g0 + lane;
    const bool active = lane < ng;

    // This lane's group of every row: in flight during the staging below.
    uint32_t w[RW][NWG];
    uint16_t s16[RW], z16[RW];
    if (active) {
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        load_group<BITS>(wrow[r] + static_cast<size_t>(g) * NWG, w[r]);
        s16[r] = srow[r][g];
        z16[r] = zrow[r][g];
      }
    }

    // Stage x~[m][64*g0 .. 64*(g0+ng)) and its per-group sums.
    __syncthreads();   // the previous chunk is no longer read
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int mm = min(m0 + m, M - 1);   // rows past M: staged, never stored
      const float4* src = reinterpret_cast<const float4*>(
          xt + static_cast<size_t>(mm) * K + static_cast<size_t>(g0) * kGroup);
#pragma unroll
      for (int h = 0; h < GC * 16 / kThreads; ++h) {
        const int f = tid + h * kThreads;   // float4 index; 16 per group
        const int gi = f >> 4;
        float part = 0.0f;
        if (gi < ng) {
          const float4 v = src[f];
          *reinterpret_cast<float4*>(&xs[m][gi * kGStride + (f & 15) * 4]) = v;
          part = (v.x + v.y) + (v.z + v.w);
        }
        // 16 consecutive lanes hold one group (f is 16-aligned per group).
        part += shfl_xor(part, 8);
        part += shfl_xor(part, 4);
        part += shfl_xor(part, 2);
        part += shfl_xor(part, 1);
        if ((f & 15) == 0 && gi < ng) sxs[m][gi] = part;
      }
    }
    __syncthreads();

    if (active) {
      float dot[RW][MT];
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) dot[r][m] = 0.0f;
#pragma unroll
      for (int i = 0; i < kGroup / SEG; ++i) {
        // Codes of both rows once; then x~ one batch row at a time.
        float q[RW][SEG];
#pragma unroll
        for (int r = 0; r < RW; ++r) seg_codes<BITS>(w[r], i, q[r]);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float xv[SEG];
#pragma unroll
          for (int c = 0; c < SEG / 4; ++c) {
            const float4 v = *reinterpret_cast<const float4*>(
                &xs[m][lane * kGStride + i * SEG + 4 * c]);
            xv[4 * c + 0] = v.x;
            xv[4 * c + 1] = v.y;
            xv[4 * c + 2] = v.z;
            xv[4 * c + 3] = v.w;
          }
#pragma unroll
          for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int j = 0; j < SEG; ++j) dot[r][m] = fmaf(q[r][j], xv[j], dot[r][m]);
        }
      }
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const float s = f16_to_f32(s16[r]);
        const float z = f16_to_f32(z16[r]);
#pragma unroll
        for (int m = 0; m < MT; ++m)
          acc[r * MT + m] = fmaf(s, fmaf(-z, sxs[m][lane], dot[r][m]), acc[r * MT + m]);
      }
    }
  }

  wave_transpose_reduce<V>(acc, lane);
  // Lane lane_of_value(t) holds value t = r * MT + m.
#pragma unroll
  for (int t = 0; t < V; ++t) {
    if (lane == lane_of_value<V>(t)) {
      const int r = t / MT;
      const int m = t - r * MT;
      const int n = rbase + r;
      if (n < N && m0 + m < M) yt[static_cast<size_t>(m0 + m) * N + n] = acc[0];
    }
  }
}

template <int BITS, int MT>
hipError_t launch_cfg(const harp_qweight& W, const float* xt, float* yt, int M,
                      hipStream_t stream) {
  const dim3 grid((W.N + kRowsPerWg - 1) / kRowsPerWg, (M + MT - 1) / MT);
  hipLaunchKernelGGL((gemv_kernel<BITS, MT>), grid, dim3(kThreads), 0, stream,
                     W.qweight, W.scale, W.zero, xt, yt, W.N, W.K, M);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const harp_qweight& W, const float* xt, float* yt, int M,
                       hipStream_t stream) {
  // MT rows of x~ per pass (grid.y passes over the weights).
  if (M == 1) return launch_cfg<BITS, 1>(W, xt, yt, M, stream);
  if (M == 2) return launch_cfg<BITS, 2>(W, xt, yt, M, stream);
  return launch_cfg<BITS, 4>(W, xt, yt, M, stream);
}

}  // namespace

hipError_t launch_gemv(const harp_qweight& W, const float* xt, float* yt, int M,
                       hipStream_t stream) {
  switch (W.bits) {
    case 2: return launch_bits<2>(W, xt, yt, M, stream);
    case 3: return launch_bits<3>(W, xt, yt, M, stream);
    case 4: return launch_bits<4>(W, xt, yt, M, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace harp
