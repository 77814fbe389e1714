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
//     per row, issued one chunk ahead (right after the chunk's x~ loads), so
//     that they stream in while the current chunk is staged and multiplied.
// Per group the product is factored as
//     sum_k (q_k - z) s x~_k = s (sum_k q_k x~_k - z sum_k x~_k),
// which leaves MT fused multiply-adds per code and one convert per two
// codes (2 and 4 bits: FP8 decodes of the masked codes).  A wave
// needs no other wave's data: its RW*MT partial sums are combined with a
// transposing reduction over its 64 lanes in a fixed order, so the result
// is bitwise reproducible.
#include "launch.hpp"
#include "unpack.hpp"
#include "validate.hpp"

namespace harp {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;   // 512
constexpr int RW = 2;                      // output rows per wave
constexpr int kRowsPerWg = kWaves * RW;    // 16
constexpr int KC = 4096;                   // inputs per staged chunk
constexpr int GC = KC / kGroup;            // groups per chunk: one per lane
constexpr int kGStride = kGroup + 4;       // LDS floats per staged group
constexpr int kPersistBlocks = 512;        // workgroups of a persistent grid

// Codes per segment of the inner loop: one word for 2- and 4-bit codes,
// 8 codes (24 bits) for 3-bit codes.
template <int BITS> struct Seg { static constexpr int CODES = BITS == 2 ? 16 : 8; };

// Codes of segment i of a group as floats, q[j] = code (i*CODES + j) /
// SegScale<BITS>::SCALE: 2- and 4-bit codes are masked four at a time into
// byte lanes and decoded two per instruction as FP8 (q 2^-9, exact), 3-bit
// codes are extracted and converted one at a time.
template <int BITS> struct SegScale {
  static constexpr float SCALE = BITS == 3 ? 1.0f : kFp8CodeScale;
};
template <int BITS>
__device__ __forceinline__ void seg_codes(const uint32_t (&w)[2 * BITS], int i,
                                          float (&q)[Seg<BITS>::CODES]) {
  if constexpr (BITS == 2) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t m = (w[i] >> (2 * t)) & 0x03030303u;  // codes t, t+4, t+8, t+12
      fp8_codes4(m, q[t], q[t + 4], q[t + 8], q[t + 12]);
    }
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t m = (w[i] >> (4 * t)) & 0x0f0f0f0fu;  // codes t, t+2, t+4, t+6
      fp8_codes4(m, q[t], q[t + 2], q[t + 4], q[t + 6]);
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
  const int m0 = blockIdx.y * MT;
  // Work items (row block, chunk): this workgroup takes row blocks
  // blockIdx.x, blockIdx.x + gridDim.x, ... (one each when the grid covers
  // every block; a smaller grid keeps the code prefetch running across its
  // blocks), every chunk of each.
  const int nrb = (N + kRowsPerWg - 1) / kRowsPerWg;
  const int nch = (G + GC - 1) / GC;
  const int nit = (nrb - static_cast<int>(blockIdx.x) + static_cast<int>(gridDim.x) - 1) /
                  static_cast<int>(gridDim.x) * nch;
  auto item_rbase = [&](int it) {
    return (static_cast<int>(blockIdx.x) + it / nch * static_cast<int>(gridDim.x)) * kRowsPerWg +
           wave * RW;
  };

  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.0f;

  // This lane's group of every row for one chunk.  The loads are never
  // conditional (lanes past the chunk's end and the prefetch after the last
  // chunk re-read a valid group), so the compiler's waits stay partial.
  struct ChunkRegs {
    uint32_t w[RW][NWG];
    uint16_t s16[RW], z16[RW];
  };
  auto load_item = [&](int it, ChunkRegs& R) {
    const int g = min((it % nch) * GC + lane, G - 1);
    const int rbase = item_rbase(it);
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int n = min(rbase + r, N - 1);      // rows past N: loaded, never stored
      load_group<BITS>(qw + static_cast<size_t>(n) * WPR + static_cast<size_t>(g) * NWG, R.w[r]);
      R.s16[r] = sc[static_cast<size_t>(n) * G + g];
      R.z16[r] = zr[static_cast<size_t>(n) * G + g];
    }
  };
  // One item: its x~ loads first, then the next item's codes (in flight
  // during this item's staging and product), then x~ staged in LDS with its
  // per-group sums, then the product on the codes loaded one item ago; the
  // last chunk of a row block stores the block's rows.
  auto chunk = [&](int it, const ChunkRegs& cur, ChunkRegs& nxt) {
    const int g0 = (it % nch) * GC;
    const int ng = min(GC, G - g0);
    const bool active = lane < ng;
    constexpr int H = GC * 16 / kThreads;          // float4 per thread per row
    float4 xv4[MT][H];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int mm = min(m0 + m, M - 1);   // rows past M: staged, never stored
      const float4* src = reinterpret_cast<const float4*>(
          xt + static_cast<size_t>(mm) * K + static_cast<size_t>(g0) * kGroup);
#pragma unroll
      for (int h = 0; h < H; ++h) {
        const int f = tid + h * kThreads;   // float4 index; 16 per group
        xv4[m][h] = src[min(f, ng * 16 - 1)];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_item(min(it + 1, nit - 1), nxt);
    // x~ arrives here, with the prefetch still in flight; the empty asm pins
    // each value so that no load is re-issued behind the prefetch
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int h = 0; h < H; ++h)
        asm volatile("" : "+v"(xv4[m][h].x), "+v"(xv4[m][h].y), "+v"(xv4[m][h].z),
                     "+v"(xv4[m][h].w));
    __syncthreads();   // the previous chunk is no longer read
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int h = 0; h < H; ++h) {
        const int f = tid + h * kThreads;
        const int gi = f >> 4;
        const float4 v = xv4[m][h];
        float part = 0.0f;
        if (gi < ng) {
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
        for (int r = 0; r < RW; ++r) seg_codes<BITS>(cur.w[r], i, q[r]);
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
        const float s = f16_to_f32(cur.s16[r]);
        const float z = f16_to_f32(cur.z16[r]);
#pragma unroll
        for (int m = 0; m < MT; ++m)
          acc[r * MT + m] = fmaf(s, fmaf(-z, sxs[m][lane], dot[r][m] * SegScale<BITS>::SCALE),
                               acc[r * MT + m]);
      }
    }
    if (g0 + GC >= G) {
      float out[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        out[i] = acc[i];
        acc[i] = 0.0f;
      }
      wave_transpose_reduce<V>(out, lane);
      // Lane lane_of_value(t) holds value t = r * MT + m.
      const int rbase = item_rbase(it);
#pragma unroll
      for (int t = 0; t < V; ++t) {
        if (lane == lane_of_value<V>(t)) {
          const int r = t / MT;
          const int m = t - r * MT;
          const int n = rbase + r;
          if (n < N && m0 + m < M) yt[static_cast<size_t>(m0 + m) * N + n] = out[0];
        }
      }
    }
  };
  ChunkRegs ra, rb;
  load_item(0, ra);
  for (int it = 0; it < nit; it += 2) {
    chunk(it, ra, rb);
    if (it + 1 < nit) chunk(it + 1, rb, ra);
  }
}

template <int BITS, int MT>
hipError_t launch_cfg(const harp_qweight& W, const float* xt, float* yt, int M,
                      hipStream_t stream) {
  // Row blocks beyond kPersistBlocks per launch are taken in turn by a grid
  // of kPersistBlocks workgroups (two per CU), so that short rows (one or
  // two chunks) do not expose each workgroup's first code load.
  const int nrb = (W.N + kRowsPerWg - 1) / kRowsPerWg;
  const int gx = (M <= MT && nrb > 2 * kPersistBlocks) ? kPersistBlocks : nrb;
  const dim3 grid(gx, (M + MT - 1) / MT);
  hipLaunchKernelGGL((gemv_kernel<BITS, MT>), grid, dim3(kThreads), 0, stream,
                     W.qweight, W.scale, W.zero, xt, yt, W.N, W.K, M);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Batches of nine or more rows on the float32 matrix cores
// (v_mfma_f32_16x16x4_f32): the same float32 product, w_hat exact and x~
// not rounded, but the multiply-adds of a 16-row tile of x~ run on the
// matrix cores instead of one vector FMA per code and row (which also had to
// re-read x~ from LDS for every pair of output rows).  A workgroup of eight
// waves owns 16 output features and one 16-row tile of x~ (grid.y tiles);
// wave w takes a contiguous eighth of the quantization groups.  In a group,
// lane l = c + 16 h (c < 16, h < 4) holds x~[c][16h .. 16h+15] of its tile
// row c and the 16 codes 16h .. 16h+15 of feature c, dequantized exactly in
// float32.  Instruction t of the group's sixteen multiplies the inputs
// {t, 16+t, 32+t, 48+t} (lane quarter h supplies input 16h + t to both
// operands), so every product of the group is formed once.  Even and odd t
// accumulate separately; the eight waves' 16 x 16 partials are then added
// in wave order through LDS.
// ---------------------------------------------------------------------------
constexpr int kMfRows = 16;            // rows of x~ per tile (matrix-core M)
constexpr int kMfMinM = 9;             // batches from this size use the matrix cores
constexpr int kMfFeatures = 16;        // output features per workgroup

// One lane's raw operands of one group: x~[c][16h .. 16h+15], the code
// words holding codes 16h .. 16h+15 of feature c, its scale and zero.
template <int BITS>
struct MfRegs {
  float4 x[4];
  uint32_t w[BITS == 2 ? 1 : 2];
  uint32_t sz;      // fp16 scale | fp16 zero << 16
};

template <int BITS>
__device__ __forceinline__ void mf_load(MfRegs<BITS>& r, int g,
                                        const float* __restrict__ xrow_p,
                                        const uint32_t* __restrict__ crow,
                                        const uint16_t* __restrict__ srow,
                                        const uint16_t* __restrict__ zrow, int h) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r.x[i] = *reinterpret_cast<const float4*>(xrow_p + g * kGroup + 16 * h + 4 * i);
  if constexpr (BITS == 2) {
    r.w[0] = crow[g * 4 + h];
  } else if constexpr (BITS == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(crow + g * 8 + 2 * h);
    r.w[0] = v.x;
    r.w[1] = v.y;
  } else {
    // a group is 192 bits (two 96-bit runs); codes 16h .. start at bit 48h
    const uint32_t* p = crow + g * 6 + ((48 * h) >> 5);
    r.w[0] = p[0];
    r.w[1] = p[1];
  }
  r.sz = static_cast<uint32_t>(srow[g]) | (static_cast<uint32_t>(zrow[g]) << 16);
}

// Codes 16h .. 16h+15 of the group as floats.
template <int BITS>
__device__ __forceinline__ void mf_codes(const MfRegs<BITS>& r, int h, float (&q)[16]) {
  if constexpr (BITS == 2) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t m = opaque((r.w[0] >> (2 * t)) & 0x03030303u);  // codes t, t+4, t+8, t+12
#pragma unroll
      for (int b = 0; b < 4; ++b) q[t + 4 * b] = static_cast<float>((m >> (8 * b)) & 0xffu);
    }
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t m = opaque((r.w[i] >> (4 * t)) & 0x0f0f0f0fu);  // codes t, t+2, t+4, t+6
#pragma unroll
        for (int b = 0; b < 4; ++b) q[8 * i + t + 2 * b] = static_cast<float>((m >> (8 * b)) & 0xffu);
      }
    }
  } else {
    const uint64_t v = static_cast<uint64_t>(r.w[0]) | (static_cast<uint64_t>(r.w[1]) << 32);
    const int off = (48 * h) & 31;
#pragma unroll
    for (int t = 0; t < 16; ++t) q[t] = static_cast<float>((v >> (off + 3 * t)) & 7u);
  }
}

template <int BITS>
__device__ __forceinline__ void mf_group(const MfRegs<BITS>& r, int h, floatx4& acc0,
                                         floatx4& acc1) {
  float q[16];
  mf_codes<BITS>(r, h, q);
  const float s = f16_to_f32(static_cast<uint16_t>(r.sz & 0xffffu));
  const float nzs = -f16_to_f32(static_cast<uint16_t>(r.sz >> 16)) * s;
  const float xs[16] = {r.x[0].x, r.x[0].y, r.x[0].z, r.x[0].w, r.x[1].x, r.x[1].y,
                        r.x[1].z, r.x[1].w, r.x[2].x, r.x[2].y, r.x[2].z, r.x[2].w,
                        r.x[3].x, r.x[3].y, r.x[3].z, r.x[3].w};
  // all sixteen weights first, so the matrix-core instructions issue back
  // to back instead of each waiting for the vector ALU
  float wv[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) wv[t] = fmaf(q[t], s, nzs);
#pragma unroll
  for (int t = 0; t < 16; t += 2) {
    acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(xs[t], wv[t], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(xs[t + 1], wv[t + 1], acc1, 0, 0, 0);
  }
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void gemv_mfma_kernel(
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint16_t* __restrict__ zr, const float* __restrict__ xt, float* __restrict__ yt,
    int N, int K, int M) {
  __shared__ floatx4 red[kWaves][kWave];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // the wave index as a scalar: the group range and the loop are uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15;
  const int h = lane >> 4;
  const int n0 = blockIdx.x * kMfFeatures;
  const int m0 = blockIdx.y * kMfRows;
  const int G = K / kGroup;
  const size_t WPR = static_cast<size_t>(K) * BITS / 32;
  const int feat = min(n0 + c, N - 1);
  const uint32_t* crow = qw + static_cast<size_t>(feat) * WPR;
  const uint16_t* srow = sc + static_cast<size_t>(feat) * G;
  const uint16_t* zrow = zr + static_cast<size_t>(feat) * G;
  // tile rows past M read row M - 1: matrix row c only feeds output row c,
  // which is then not stored, so no load needs a guard
  const float* xrow_p = xt + static_cast<size_t>(min(m0 + c, M - 1)) * K;
  const int gb = wave * G / kWaves;
  const int ge = (wave + 1) * G / kWaves;

  floatx4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f};
  floatx4 acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
  if (gb < ge) {
    // three register sets: the loads of the next two groups are in flight
    // while a group is multiplied; a load past the range re-loads the last
    // group (valid memory, unused)
    MfRegs<BITS> ra, rb, rc;
    const int gl = ge - 1;
    mf_load<BITS>(ra, gb, xrow_p, crow, srow, zrow, h);
    mf_load<BITS>(rb, min(gb + 1, gl), xrow_p, crow, srow, zrow, h);
    int g = gb;
    for (; g + 3 <= ge; g += 3) {
      mf_load<BITS>(rc, min(g + 2, gl), xrow_p, crow, srow, zrow, h);
      mf_group<BITS>(ra, h, acc0, acc1);
      mf_load<BITS>(ra, min(g + 3, gl), xrow_p, crow, srow, zrow, h);
      mf_group<BITS>(rb, h, acc0, acc1);
      mf_load<BITS>(rb, min(g + 4, gl), xrow_p, crow, srow, zrow, h);
      mf_group<BITS>(rc, h, acc0, acc1);
    }
    if (g < ge) mf_group<BITS>(ra, h, acc0, acc1);
    if (g + 1 < ge) mf_group<BITS>(rb, h, acc0, acc1);
  }
  red[wave][lane] = acc0 + acc1;
  __syncthreads();
  if (wave == 0) {
    floatx4 sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += red[w][lane];
    // 16 x 16 accumulator layout: lane l holds rows 4 (l / 16) + r of
    // column l % 16, i.e. x~ rows m0 + 4h + r of feature n0 + c
    const int n = n0 + c;
    if (n < N) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 4 * h + r;
        if (m < M) yt[static_cast<size_t>(m) * N + n] = sum[r];
      }
    }
  }
}

template <int BITS>
hipError_t launch_mfma(const harp_qweight& W, const float* xt, float* yt, int M,
                       hipStream_t stream) {
  const dim3 grid((W.N + kMfFeatures - 1) / kMfFeatures, (M + kMfRows - 1) / kMfRows);
  hipLaunchKernelGGL((gemv_mfma_kernel<BITS>), grid, dim3(kThreads), 0, stream, W.qweight,
                     W.scale, W.zero, xt, yt, W.N, W.K, M);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const harp_qweight& W, const float* xt, float* yt, int M,
                       hipStream_t stream) {
  // Up to eight rows the vector-ALU kernel (at most two passes over the
  // weights) is faster; from nine rows on, 16-row tiles on the matrix cores
  // (4096x4096 2-bit: 13.0 vs 12.3 us at M = 8, 14.5 vs 18.3 at M = 12,
  // 52.0 vs 70.3 at M = 64).
  if (M == 1) return launch_cfg<BITS, 1>(W, xt, yt, M, stream);
  if (M == 2) return launch_cfg<BITS, 2>(W, xt, yt, M, stream);
  if (M <= kMfMinM - 1) return launch_cfg<BITS, 4>(W, xt, yt, M, stream);
  return launch_mfma<BITS>(W, xt, yt, M, stream);
}

// ---------------------------------------------------------------------------
// Decode batches with the input rotation in the prologue:
//   y'[m][n] = sum_k w_hat[n][k] (F_V x_m)[k]
// for M <= 4 and K <= 4096.  Every workgroup computes the whole x~ = F_V x in
// LDS (HARP technical summary §2.1-2.2: sign flip, then stages 0..L-1), which
// costs it a few microseconds of VALU and LDS time that overlap the fetch of
// its own weights, and saves the separate rotation launch.
//
// Rotation layout.  Task tid (one per thread, K/8 of them) owns 8 elements of
// one block of b = 2^L inputs in each round; round r covers stages 3r ..
// 3r+2 (fewer in the last round), exactly as the stand-alone rotation kernel
// does with 8 elements per thread.  The rotated rows live in LDS in the
// padded group layout of the product phase, so the product phase reads them
// where the rotation left them.
// ---------------------------------------------------------------------------

constexpr int kRotMaxRounds = 4;            // b <= 4096: L <= 12 stages

// Index inside a block of local element jj (0..7) of task t in a round over
// stages s0 .. s0+R-1 (R <= 3): the low R bits of jj walk those strides, the
// rest of the task index and of jj fill the other bits in order.
__device__ __forceinline__ int round_elem(int t, int jj, int s0, int R) {
  const int rest = (t << (3 - R)) + (jj >> R);
  const int jl = jj & ((1 << R) - 1);
  const int lo = rest & ((1 << s0) - 1);
  const int hi = rest >> s0;
  return (hi << (s0 + R)) | (jl << s0) | lo;
}

__device__ __forceinline__ int pair_of(int i, int s) {   // i with bit s deleted
  return ((i >> (s + 1)) << s) | (i & ((1 << s) - 1));
}

__host__ __device__ constexpr int with_zero_bit(int p, int k) {
  return ((p >> k) << (k + 1)) | (p & ((1 << k) - 1));
}

__device__ __forceinline__ int padded(int i) { return (i >> 6) * kGStride + (i & 63); }

// LOGB_: log2 of the input-side block size when fixed at compile time (the
// index arithmetic of the rounds then folds to constants), 0 to take it from
// logb at run time.
template <int BITS, int MT, bool Q8, int LOGB_>
__global__ __launch_bounds__(kThreads) void gemv_rot_kernel(
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint16_t* __restrict__ zr, const void* __restrict__ xin, int x_bf16,
    const float2* __restrict__ cs, const int8_t* __restrict__ codes, float step,
    const uint32_t* __restrict__ sign, int logb, float* __restrict__ yt, int N,
    int K, int M) {
  constexpr int NWG = 2 * BITS;
  constexpr int SEG = Seg<BITS>::CODES;
  constexpr int V = RW * MT;
  __shared__ __attribute__((aligned(16))) float xs[MT][GC * kGStride];
  __shared__ float sxs[MT][GC];
  __shared__ float2 table[Q8 ? 256 : 1];

  const int G = K / kGroup;                 // <= 64: one group per lane
  const size_t WPR = static_cast<size_t>(K) * BITS / 32;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int rbase = blockIdx.x * kRowsPerWg + wave * RW;

  // 1. This lane's group of each of the wave's rows: in flight during the
  //    rotation below.
  const bool gact = lane < G;
  uint32_t w[RW][NWG];
  uint16_t s16[RW], z16[RW];
  if (gact) {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int n = min(rbase + r, N - 1);   // rows past N: loaded, never stored
      load_group<BITS>(qw + static_cast<size_t>(n) * WPR + static_cast<size_t>(lane) * NWG, w[r]);
      s16[r] = sc[static_cast<size_t>(n) * G + lane];
      z16[r] = zr[static_cast<size_t>(n) * G + lane];
    }
  }

  // 2. Rotation coefficients of this thread's task, every round.
  const int L = LOGB_ ? LOGB_ : logb;
  const int B = 1 << L;
  const int NR = (L + 2) / 3;
  const bool tact = tid < (K >> 3);
  const int tl = L - 3;                      // log2 tasks per block
  const int blk = tid >> tl;
  const int t = tid & ((1 << tl) - 1);
  const size_t blk_off = static_cast<size_t>(blk) * L * (B / 2);
  float2 cf[kRotMaxRounds][3][4];
  int qc[Q8 ? kRotMaxRounds : 1][3][4];
  auto for_task = [&](auto&& f) {
#pragma unroll
    for (int r = 0; r < kRotMaxRounds; ++r) {
      if (r < NR) {
        const int s0 = 3 * r;
        const int R = min(3, L - s0);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          if (k < R) {
            const int s = s0 + k;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const int i = round_elem(t, with_zero_bit(p, k), s0, R);
              f(r, k, p, blk_off + static_cast<size_t>(s) * (B / 2) + pair_of(i, s));
            }
          }
        }
      }
    }
  };
  if (tact) {
    if constexpr (Q8) {
      for_task([&](int r, int k, int p, size_t c) { qc[r][k][p] = codes[c]; });
    } else {
      for_task([&](int r, int k, int p, size_t c) { cf[r][k][p] = cs[c]; });
    }
  }

  // 3. Eight consecutive inputs per task and row, raw, and their sign bits.
  u32x4 raw[MT][2];
  if (tact) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < M) {
        if (x_bf16) {
          raw[m][0] = reinterpret_cast<const u32x4*>(
              static_cast<const uint16_t*>(xin) + static_cast<size_t>(m) * K)[tid];
        } else {
          const u32x4* src = reinterpret_cast<const u32x4*>(
              static_cast<const float*>(xin) + static_cast<size_t>(m) * K);
          raw[m][0] = src[2 * tid];
          raw[m][1] = src[2 * tid + 1];
        }
      }
    }
  }
  const uint32_t sbits = tact ? (sign[tid >> 2] >> ((tid & 3) * 8)) : 0u;

  if constexpr (Q8) {
    for (int i = tid; i < 256; i += kThreads) {
      float sn, cn;
      sincosf(fmaf(static_cast<float>(i - 128), step, 0.785398163397448310f), &sn, &cn);
      table[i] = make_float2(cn, sn);
    }
  }
  // 4. D x into LDS (8 consecutive inputs stay inside one 64-group).
  if (tact) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v[8];
      if (m >= M) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.0f;
      } else if (x_bf16) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          v[j] = bf16_to_f32(static_cast<uint16_t>(raw[m][0][j >> 1] >> (16 * (j & 1))));
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(raw[m][j >> 2][j & 3]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = flip_sign(v[j], (sbits >> j) & 1u);
      float* d = &xs[m][padded(tid * 8)];
      *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(d + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
  __syncthreads();

  // 5. Stages in place, three per round, one barrier per round.
#pragma unroll
  for (int r = 0; r < kRotMaxRounds; ++r) {
    if (r < NR) {
      const int s0 = 3 * r;
      const int R = min(3, L - s0);
      if (tact) {
        if constexpr (Q8) {
#pragma unroll
          for (int k = 0; k < 3; ++k)
#pragma unroll
            for (int p = 0; p < 4; ++p)
              if (k < R) cf[r][k][p] = table[qc[r][k][p] + 128];
        }
        int pos[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pos[j] = padded(blk * B + round_elem(t, j, s0, R));
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = xs[m][pos[j]];
#pragma unroll
          for (int k = 0; k < 3; ++k) {
            if (k < R) {
#pragma unroll
              for (int p = 0; p < 4; ++p) {
                const int j1 = with_zero_bit(p, k);
                const int j2 = j1 | (1 << k);
                const float a = v[j1];
                const float b = v[j2];
                const float c = cf[r][k][p].x;
                const float sn = cf[r][k][p].y;
                v[j1] = fmaf(c, a, sn * b);
                v[j2] = fmaf(sn, a, -(c * b));
              }
            }
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) xs[m][pos[j]] = v[j];
        }
      }
      __syncthreads();
    }
  }

  // 6. Per-group sums of x~ (16 lanes per group, fixed order).
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int h = 0; h < GC * 16 / kThreads; ++h) {
      const int f = tid + h * kThreads;
      const int gi = f >> 4;
      float part = 0.0f;
      if (gi < G) {
        const float4 v = *reinterpret_cast<const float4*>(&xs[m][gi * kGStride + (f & 15) * 4]);
        part = (v.x + v.y) + (v.z + v.w);
      }
      part += shfl_xor(part, 8);
      part += shfl_xor(part, 4);
      part += shfl_xor(part, 2);
      part += shfl_xor(part, 1);
      if ((f & 15) == 0 && gi < G) sxs[m][gi] = part;
    }
  }
  __syncthreads();

  // 7. The product, as in gemv_kernel.
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.0f;
  if (gact) {
    float dot[RW][MT];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) dot[r][m] = 0.0f;
#pragma unroll
    for (int i = 0; i < kGroup / SEG; ++i) {
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
        acc[r * MT + m] = fmaf(s, fmaf(-z, sxs[m][lane], dot[r][m] * SegScale<BITS>::SCALE),
                               acc[r * MT + m]);
    }
  }
  wave_transpose_reduce<V>(acc, lane);
#pragma unroll
  for (int tv = 0; tv < V; ++tv) {
    if (lane == lane_of_value<V>(tv)) {
      const int r = tv / MT;
      const int m = tv - r * MT;
      const int n = rbase + r;
      if (n < N && m < M) yt[static_cast<size_t>(m) * N + n] = acc[0];
    }
  }
}

template <int BITS, int MT, bool Q8, int LOGB_>
hipError_t launch_rot_logb(const harp_rotation& Vr, const harp_qweight& W,
                           const void* x, int x_dt, float* yt, int M,
                           hipStream_t stream) {
  const dim3 grid((W.N + kRowsPerWg - 1) / kRowsPerWg);
  hipLaunchKernelGGL((gemv_rot_kernel<BITS, MT, Q8, LOGB_>), grid, dim3(kThreads), 0, stream,
                     W.qweight, W.scale, W.zero, x, x_dt == HARP_BF16 ? 1 : 0,
                     reinterpret_cast<const float2*>(Vr.cs), Vr.phi_codes, Vr.phi_step,
                     Vr.sign_bits, __builtin_ctz(static_cast<unsigned>(Vr.block)), yt,
                     W.N, W.K, M);
  return hipGetLastError();
}

template <int BITS, int MT, bool Q8>
hipError_t launch_rot_cfg(const harp_rotation& Vr, const harp_qweight& W,
                          const void* x, int x_dt, float* yt, int M,
                          hipStream_t stream) {
  if (Vr.block == 4096)
    return launch_rot_logb<BITS, MT, Q8, 12>(Vr, W, x, x_dt, yt, M, stream);
  return launch_rot_logb<BITS, MT, Q8, 0>(Vr, W, x, x_dt, yt, M, stream);
}

template <int BITS, bool Q8>
hipError_t launch_rot_bits(const harp_rotation& Vr, const harp_qweight& W,
                           const void* x, int x_dt, float* yt, int M,
                           hipStream_t stream) {
  if (M == 1) return launch_rot_cfg<BITS, 1, Q8>(Vr, W, x, x_dt, yt, M, stream);
  if (M == 2) return launch_rot_cfg<BITS, 2, Q8>(Vr, W, x, x_dt, yt, M, stream);
  return launch_rot_cfg<BITS, 4, Q8>(Vr, W, x, x_dt, yt, M, stream);
}

template <bool Q8>
hipError_t launch_rot_q(const harp_rotation& Vr, const harp_qweight& W,
                        const void* x, int x_dt, float* yt, int M,
                        hipStream_t stream) {
  switch (W.bits) {
    case 2: return launch_rot_bits<2, Q8>(Vr, W, x, x_dt, yt, M, stream);
    case 3: return launch_rot_bits<3, Q8>(Vr, W, x, x_dt, yt, M, stream);
    case 4: return launch_rot_bits<4, Q8>(Vr, W, x, x_dt, yt, M, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool gemv_rotated_supported(const harp_rotation& V, const harp_qweight& W, int M) {
  return M >= 1 && M <= kDecodeRotMaxM && W.K <= kDecodeRotMaxK && V.block >= 8 &&
         V.dim == W.K;
}

hipError_t launch_gemv_rotated(const harp_rotation& V, const harp_qweight& W,
                               const void* x, int x_dt, float* yt, int M,
                               hipStream_t stream) {
  if (!gemv_rotated_supported(V, W, M)) return hipErrorInvalidValue;
  if (V.phi_codes != nullptr) return launch_rot_q<true>(V, W, x, x_dt, yt, M, stream);
  return launch_rot_q<false>(V, W, x, x_dt, yt, M, stream);
}

hipError_t launch_gemv(const harp_qweight& W, const float* xt, float* yt, int M,
                       hipStream_t stream) {
  if (M >= kGemvMcMinM && M <= kGemvMcMaxM && W.bits != 3)
    return launch_gemv_mc(W, xt, yt, M, stream);
  switch (W.bits) {
    case 2: return launch_bits<2>(W, xt, yt, M, stream);
    case 3: return launch_bits<3>(W, xt, yt, M, stream);
    case 4: return launch_bits<4>(W, xt, yt, M, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace harp
