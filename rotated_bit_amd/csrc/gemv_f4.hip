// One-row decode product of 2-bit codes on the FP4 x FP8 matrix cores (and
// of 4-bit codes as FP8 values, transpose4 below):
//     y'[n] = sum_g s[n][g] (sum_{k in g} q[n][k] x~[k] - z[n][g] sum_{k in g} x~[k]).
//
// gfx950 has a block-scaled matrix-core instruction whose operands are
// FP8 / FP6 / FP4 values (v_mfma_scale_f32_16x16x128_f8f6f4: a 16 x 128
// times 128 x 16 product, float32 accumulation, one power-of-two scale per
// row or column and 32 inputs).  Both factors of q x~ map onto it exactly:
//   * a 2-bit code q is the FP4 (e2m1) value q / 2 when its two bits sit at
//     the bottom of a nibble: a code word masked with 0x33333333 and its
//     copy shifted right by two give sixteen FP4 values with two
//     instructions each, and the column scale 2^1 restores q;
//   * x~ (float32, not rounded) is carried as eight FP8 (e4m3) planes of
//     signed base-16 digits, one exponent per quantization group and plane,
//     which reproduce x~ to 2^-28 of the group maximum (see build_step).
// A small kernel builds the planes once per call; each product workgroup
// copies its K slice of them into LDS and streams the codes of its rows.
//
// Operand roles of one matrix-core step (128 inputs, two quantization
// groups): the planes are the 16 x 128 operand, one row per (plane p,
// group half h) so that row p + 8h carries plane p of the step's group h and
// zeros over the other group; the codes are the 128 x 16 operand, one
// column per output row.  Lane l then holds the four planes
// 4(l/16 % 2) .. +3 of group half (l/16) / 2 for output row l % 16: all four
// share that row's scale and zero, so the epilogue is one sum, one
// multiply-add for the zero point and one for the scale per step and lane.
//
// Lane layouts (checked on the device): FP4 operand lane l holds row or
// column l % 16 and inputs 32 (l/16) .. +31 in nibble order; FP8 operand
// lane l holds row or column l % 16 and inputs 16 (l/16) .. +15 (bytes
// 0..15) and 64 + 16 (l/16) .. +15 (bytes 16..31); the scale of row/column
// r and input block b comes from lane r + 16 b; result lane l holds column
// l % 16, rows 4 (l/16) .. +3.
//
// Inputs in operand order.  Steps come in pairs (2t, 2t + 1) over the 256
// inputs of groups 4t .. 4t+3: step 2t + e takes group 4t + e in its first
// group half and group 4t + 2 + e in its second, so block b of the step (a
// half group) is inputs 256 t + 128 (b/2) + 64 e + 32 (b%2) .. +31.  Within
// a block, operand offset o = 8 v + j (nibble j of code register v) is
// input pi(o) = 16 (v/2) + 2 j + (v % 2), because register v holds the even
// (v even) or odd codes of one code word.  Each lane loads one whole group
// (16 bytes) per pair, lanes 16 apart exchange half groups
// (v_permlane16_swap), and every row's 128-byte line of codes is read by
// four lanes of one load.
#include "f4_planes.hpp"
#include "fold256.hpp"
#include "launch.hpp"
#include "unpack.hpp"
#include "validate.hpp"

namespace harp {
namespace {

using namespace f4;

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kF4WgWaves = 8;                      // one 16-row tile per wave
constexpr int kF4Threads = kF4WgWaves * kWave;     // 512

// One wave per step: the step's planes, scale bytes and group sums built
// into LDS by build_step, then written to the f4 region by emit_step.
__global__ __launch_bounds__(256) void f4_planes_kernel(const float* __restrict__ xt, int K,
                                                        u32x4* __restrict__ pl,
                                                        uint32_t* __restrict__ psc,
                                                        float* __restrict__ sx) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[4][kStepLds + kWave];
  __shared__ float ssx[4][4];
  const int s = (blockIdx.x * 256 + threadIdx.x) >> 6;
  if (s >= K / kF4Step) return;   // whole waves
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  build_step(xt + 256 * (s >> 1) + 64 * (s & 1), stage[w], stage[w] + kStepLds, ssx[w], lane);
  emit_step(stage[w], ssx[w], s, pl, psc, sx, lane);
}

// ---- product ---------------------------------------------------------------
// Grid (ceil(tiles / 8), slices): wave w of workgroup (x, y) owns rows
// 16 (8x + w) .. +15 over the K slice y (step pairs [pa, pb)).  The first
// chunk's codes are requested before the slice's planes, scale bytes and
// group sums (from f4_planes_kernel) and the workgroup's scales and zeros
// (row-contiguous reads) are copied into LDS.  The codes then stream in
// chunks of kPairs step pairs through two register sets (the next chunk is
// requested before the current one is used); the steps of a chunk are
// issued 2 kBatchPairs matrix instructions at a time before their
// epilogues, with no branch inside (steps past the slice's end repeat its
// last step with the scale zeroed).
//
// LDS keeps each step's 1024 plane bytes followed by 16 zero bytes, so a
// lane forms its operand (plane bytes in one half, zeros in the other) from
// two reads at the same immediate offset and no selects.
constexpr int kPairs = 2;                 // step pairs per chunk
constexpr int kSzStride = kF4MaxSliceSteps + 1;   // LDS dwords per row of scales / zeros
constexpr int kBatchPairs = 2;            // step pairs per batch of matrix instructions

// Output side folded into the product (FOLD 1: float32 y, 2: bf16 y): a
// block-diagonal F_U with 256-output blocks, one K slice (fold256.hpp).

// 4-bit codes as FP8 (e4m3) values: a code q in the low nibble of a byte
// is q 2^-9 exactly (subnormal below 8, the first binade from 8), restored
// by the column scale 2^9.  The FP8 operand layout gives lane l (g = l/16)
// the inputs 16g .. 16g+15 of the step's two groups, in the order the planes
// use (even inputs in bytes 0..7, odd ones in bytes 8..15 of each half).
// Each lane loads one whole group (32 bytes) of its row per step pair; the
// four lanes of a row then exchange 16-input runs (a 4 x 4 transpose over
// lanes 16 apart: lanes 32 apart swap the runs whose upper index bit differs
// from theirs, then lanes 16 apart the rest), so that lane g holds run g of
// groups 4t .. 4t+3.
struct T4 {
  uint2 p[4];
};
__device__ __forceinline__ T4 transpose4(const u32x4 (&c)[2]) {
  // runs 0..3 of the lane's own group: (c0.x, c0.y), (c0.z, c0.w), ...
  const auto a0 = __builtin_amdgcn_permlane32_swap(c[0].x, c[1].x, false, false);
  const auto a1 = __builtin_amdgcn_permlane32_swap(c[0].y, c[1].y, false, false);
  const auto a2 = __builtin_amdgcn_permlane32_swap(c[0].z, c[1].z, false, false);
  const auto a3 = __builtin_amdgcn_permlane32_swap(c[0].w, c[1].w, false, false);
  // with g = 2 g1 + g0: now (a0[0], a1[0]) / (a0[1], a1[1]) hold run 2 g1
  // of groups 4t + g0 / 4t + 2 + g0, and (a2, a3) the same for run 2 g1 + 1
  const auto b0 = __builtin_amdgcn_permlane16_swap(a0[0], a2[0], false, false);
  const auto b1 = __builtin_amdgcn_permlane16_swap(a1[0], a3[0], false, false);
  const auto b2 = __builtin_amdgcn_permlane16_swap(a0[1], a2[1], false, false);
  const auto b3 = __builtin_amdgcn_permlane16_swap(a1[1], a3[1], false, false);
  T4 t;
  t.p[0] = make_uint2(b0[0], b1[0]);
  t.p[1] = make_uint2(b0[1], b1[1]);
  t.p[2] = make_uint2(b2[0], b3[0]);
  t.p[3] = make_uint2(b2[1], b3[1]);
  return t;
}

template <int BITS, int FOLD, bool Q8U>
__global__ __launch_bounds__(kF4Threads, 1) void gemv_f4_kernel(
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint16_t* __restrict__ zr, const u32x4* __restrict__ gpl,
    const uint32_t* __restrict__ gps, const float* __restrict__ gsx, float* __restrict__ yt,
    float* __restrict__ partials, uint32_t* __restrict__ counters, int N, int K, int slices,
    Fold256Out out) {
  __shared__ __attribute__((aligned(16))) uint8_t lpl[kF4MaxSliceSteps * kStepLds];
  __shared__ uint8_t lpsc[kF4MaxSliceSteps * kWave];
  __shared__ float lsx[2 * kF4MaxSliceSteps];
  // scales and zeros of the workgroup's rows over the slice: per row one
  // dword per (step pair, group half), rows kSzStride dwords apart (odd, so
  // that the 16 rows of a wave read distinct banks)
  __shared__ uint32_t lsc[kF4WgWaves * 16 * kSzStride];
  __shared__ uint32_t lzr[kF4WgWaves * 16 * kSzStride];

  const int pairs = K / (2 * kF4Step);
  const int pa = static_cast<int>(blockIdx.y) * pairs / slices;
  const int pb = (static_cast<int>(blockIdx.y) + 1) * pairs / slices;
  const int np = pb - pa;                 // step pairs of this slice
  const int ns = 2 * np;                  // steps
  const int sa = 2 * pa;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int tiles = N / 16;
  const int tile = static_cast<int>(blockIdx.x) * kF4WgWaves + wave;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int h = g >> 1;                    // group half of this lane's results
  const bool zlane = (g & 1) == 0;         // planes 0..3: carries the zero-point term
  const int row = min(tile, tiles - 1) * 16 + n;   // waves past the last tile load it, then leave
  // 2 bits: 16 bytes per group; 4 bits: 32 bytes per group (two vectors)
  constexpr int kVec = BITS / 2;
  const u32x4* qrow =
      reinterpret_cast<const u32x4*>(qw + static_cast<size_t>(row) * (K * BITS / 32)) + kVec * g;

  // one register set: per step pair this lane's group of codes (16 bytes,
  // group 4t + g); pairs past the slice re-read its last pair (one cached
  // line per lane)
  struct Chunk {
    u32x4 c[kPairs][kVec];
  };
  auto load = [&](int c, Chunk& ch) {
#pragma unroll
    for (int i = 0; i < kPairs; ++i)
#pragma unroll
      for (int v = 0; v < kVec; ++v)
        ch.c[i][v] = qrow[4 * kVec * (pa + min(c * kPairs + i, np - 1)) + v];
  };
  const int nch = (np + kPairs - 1) / kPairs;
  Chunk A, B;
  load(0, A);
  {
    // planes: at most 8 16-byte vectors per thread; scale bytes: ns * 16
    // <= 2 * kF4Threads dwords; group sums: 2 ns <= kF4Threads floats
    constexpr int kPer = kF4MaxSliceSteps * kWave / kF4Threads;
    constexpr int kPsPer = kF4MaxSliceSteps * 16 / kF4Threads;
    static_assert(kPsPer * kF4Threads == kF4MaxSliceSteps * 16 &&
                  2 * kF4MaxSliceSteps <= kF4Threads, "LDS fill shares");
    const u32x4* ppl = gpl + static_cast<size_t>(sa) * kWave;
    const int nv = ns * kWave;
    u32x4 v[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) v[q] = ppl[min(tid + q * kF4Threads, nv - 1)];
    uint32_t ps[kPsPer];
#pragma unroll
    for (int q = 0; q < kPsPer; ++q) ps[q] = gps[sa * 16 + min(tid + q * kF4Threads, ns * 16 - 1)];
    const float sxv = gsx[2 * sa + min(tid, 2 * ns - 1)];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int i = tid + q * kF4Threads;
      if (i < nv)
        *reinterpret_cast<u32x4*>(lpl + (i >> 6) * kStepLds + (i & 63) * 16) = v[q];
    }
    if (tid < ns)
      *reinterpret_cast<u32x4*>(lpl + tid * kStepLds + 1024) = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < kPsPer; ++q)
      if (tid + q * kF4Threads < ns * 16)
        reinterpret_cast<uint32_t*>(lpsc)[tid + q * kF4Threads] = ps[q];
    if (tid < 2 * ns) lsx[tid] = sxv;
    // scales and zeros: np 8-byte words (four groups) per row, consecutive
    // threads along a row, every load issued before the first LDS write;
    // rows past N re-read the last row
    constexpr int kSzPer = kF4WgWaves * 16 * (kF4MaxSliceSteps / 2) / kF4Threads;
    const int row0 = static_cast<int>(blockIdx.x) * kF4WgWaves * 16;
    const int nw = kF4WgWaves * 16 * np;
    uint2 sv[kSzPer], zv[kSzPer];
#pragma unroll
    for (int q = 0; q < kSzPer; ++q) {
      const int i = min(tid + q * kF4Threads, nw - 1);
      const int r = i / np;
      const size_t gi =
          static_cast<size_t>(min(row0 + r, N - 1)) * (K / (4 * kGroup)) + pa + (i - r * np);
      sv[q] = reinterpret_cast<const uint2*>(sc)[gi];
      zv[q] = reinterpret_cast<const uint2*>(zr)[gi];
    }
#pragma unroll
    for (int q = 0; q < kSzPer; ++q) {
      const int i = tid + q * kF4Threads;
      if (i < nw) {
        const int r = i / np;
        const int o = r * kSzStride + 2 * (i - r * np);
        lsc[o] = sv[q].x;
        lsc[o + 1] = sv[q].y;
        lzr[o] = zv[q].x;
        lzr[o + 1] = zv[q].y;
      }
    }
  }
  __syncthreads();
  if (tile >= tiles) return;

  // operand halves: rows p + 8h with h = 1 carry their planes in bytes
  // 16..31, the others in bytes 0..15; the other half reads the zeros
  const bool upper = (lane & 8) != 0;
  const uint8_t* lo_base = lpl + (upper ? 1024 : lane * 16);
  const uint8_t* hi_base = lpl + (upper ? lane * 16 : 1024);
  const float* sx_base = lsx + 2 * h;
  const uint32_t* sc_base = lsc + (wave * 16 + n) * kSzStride + h;
  const uint32_t* zr_base = lzr + (wave * 16 + n) * kSzStride + h;
  const float zmask = zlane ? 1.0f : 0.0f;

  float acc = 0.0f;
  auto process = [&](const Chunk& ch, int c) {
#pragma unroll
    for (int half = 0; half < kPairs / kBatchPairs; ++half) {
      floatx4 Dv[2 * kBatchPairs];
#pragma unroll
      for (int i = 0; i < 2 * kBatchPairs; ++i) {
        const int pi = half * kBatchPairs + i / 2;    // pair within the chunk
        const int e = i & 1;                           // step within the pair
        const int ls = min(2 * (c * kPairs + pi) + e, ns - 1);
        const u32x4 lo = *reinterpret_cast<const u32x4*>(lo_base + ls * kStepLds);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(hi_base + ls * kStepLds);
        const i32x8 Aop = {static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z),
                           static_cast<int>(lo.w), static_cast<int>(hi.x), static_cast<int>(hi.y),
                           static_cast<int>(hi.z), static_cast<int>(hi.w)};
        if constexpr (BITS == 2) {
          // half groups exchanged between lanes 16 apart: afterwards words
          // 0-1 belong to step 2t and words 2-3 to step 2t + 1 in every lane
          u32x4 w = ch.c[pi][0];
          {
            const auto s0 = __builtin_amdgcn_permlane16_swap(w.x, w.z, false, false);
            const auto s1 = __builtin_amdgcn_permlane16_swap(w.y, w.w, false, false);
            w.x = s0[0];
            w.z = s0[1];
            w.y = s1[0];
            w.w = s1[1];
          }
          const uint32_t w0 = e ? w.z : w.x;
          const uint32_t w1 = e ? w.w : w.y;
          const i32x8 Bop = {static_cast<int>(w0 & 0x33333333u),
                             static_cast<int>((w0 >> 2) & 0x33333333u),
                             static_cast<int>(w1 & 0x33333333u),
                             static_cast<int>((w1 >> 2) & 0x33333333u), 0, 0, 0, 0};
          Dv[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              Aop, Bop, floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 4, 0,
              static_cast<int>(lpsc[ls * kWave + lane]), 0, 128);
        } else {
          const T4 t = transpose4(ch.c[pi]);
          // bytes 0..15: the even, then the odd inputs of the lane's run of
          // group 4t + e; bytes 16..31: the same run of group 4t + 2 + e
          const uint2 ra = e ? t.p[1] : t.p[0];
          const uint2 rb = e ? t.p[3] : t.p[2];
          const i32x8 Bop = {static_cast<int>(ra.x & 0x0f0f0f0fu),
                             static_cast<int>(ra.y & 0x0f0f0f0fu),
                             static_cast<int>((ra.x >> 4) & 0x0f0f0f0fu),
                             static_cast<int>((ra.y >> 4) & 0x0f0f0f0fu),
                             static_cast<int>(rb.x & 0x0f0f0f0fu),
                             static_cast<int>(rb.y & 0x0f0f0f0fu),
                             static_cast<int>((rb.x >> 4) & 0x0f0f0f0fu),
                             static_cast<int>((rb.y >> 4) & 0x0f0f0f0fu)};
          Dv[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              Aop, Bop, floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0,
              static_cast<int>(lpsc[ls * kWave + lane]), 0, 127 + 9);
        }
      }
#pragma unroll
      for (int i = 0; i < 2 * kBatchPairs; ++i) {
        const int pi = half * kBatchPairs + i / 2;
        const int e = i & 1;
        const int ls = 2 * (c * kPairs + pi) + e;
        const float live = ls < ns ? 1.0f : 0.0f;
        const float dsum = (Dv[i][0] + Dv[i][1]) + (Dv[i][2] + Dv[i][3]);
        // the row's scale and zero of group 4t + 2h + e
        const int lp = min(c * kPairs + pi, np - 1);
        const float sf = live * f16_to_f32(static_cast<uint16_t>(sc_base[2 * lp] >> (16 * e)));
        const float zf = f16_to_f32(static_cast<uint16_t>(zr_base[2 * lp] >> (16 * e)));
        // group sum of group 4t + 2h + e (local group 2 ls + 2h - e), on
        // the lanes that carry the zero-point term
        const float sxg = zmask * sx_base[2 * min(ls, ns - 1) - e];
        acc = fmaf(sf, fmaf(-zf, sxg, dsum), acc);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // chunk c: request chunk c + 1 into the other register set, then use
  // chunk c (pairs past the slice all re-read its last pair).  One small
  // chunk ahead measured faster than two, or than larger chunks.  The second
  // half is unconditional (past the last chunk every step is zeroed): under
  // a branch its loads would be sunk behind the first half's use
  auto chunk = [&](int c, const Chunk& cur, Chunk& nxt) {
    load(c + 1, nxt);
    process(cur, c);
  };
  for (int c = 0; c < nch; c += 2) {
    chunk(c, A, B);
    chunk(c + 1, B, A);
  }
  // the four lanes of row n: (g0 + g1) + (g2 + g3), the same bits in each
  acc += shfl_xor(acc, 16);
  acc += shfl_xor(acc, 32);

  if constexpr (FOLD != 0) {
    // The output rotation of this workgroup's 256-output block (two
    // workgroups of 128 rows), the second to arrive applying it.
    __shared__ uint32_t last;
    const int ob = static_cast<int>(blockIdx.x) >> 1;
    Fold256Regs fr;
    fold256_prefetch<Q8U>(out, ob, tid, fr);
    if (g == 0)
      __hip_atomic_store(&yt[row], acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the planes are no longer read once every wave has arrived
    fold256_finish<FOLD, Q8U>(out, ob, tid, fr, yt, counters, 2u, reinterpret_cast<float*>(lpl),
                              reinterpret_cast<float2*>(lpl + 256 * sizeof(float)), &last);
    return;
  }
  if (slices == 1) {
    if (g == 0) yt[row] = acc;
    return;
  }
  // Split K: each slice stores its partial (device-coherent stores,
  // acknowledged before the arrival is counted); the last slice to arrive
  // adds the partials in slice order, so the result does not depend on the
  // arrival order, and resets the tile's counter.
  if (g == 0)
    __hip_atomic_store(&partials[static_cast<size_t>(blockIdx.y) * N + row], acc,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  uint32_t prev = 0;
  if (lane == 0)
    prev = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0, kWave);
  if (prev != static_cast<uint32_t>(slices - 1)) return;
  if (g == 0) {
    float t = 0.0f;
    for (int j = 0; j < slices; ++j) {
      const float part = __hip_atomic_load(&partials[static_cast<size_t>(j) * N + row],
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      t = j == 0 ? part : t + part;
    }
    yt[row] = t;
  }
  if (lane == 0)
    __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_gemv_f4(const harp_qweight& W, const float* xt, float* yt, uint8_t* f4,
                          uint32_t* counters, int slices, bool planes_ready,
                          hipStream_t stream, const harp_rotation* U, void* y, int y_dt) {
  const int steps = W.K / kF4Step;
  const int pairs = steps / 2;
  if ((W.bits != 2 && W.bits != 4) || W.N % 16 != 0 || W.K % (2 * kF4Step) != 0 || slices < 1 ||
      slices > kF4MaxSplits || (pairs + slices - 1) / slices * 2 > kF4MaxSliceSteps ||
      f4 == nullptr || (slices > 1 && (counters == nullptr || W.N / 16 > kF4MaxSplitTiles)) ||
      (U != nullptr && !gemv_f4_fold_supported(*U, W, slices)) ||
      (U != nullptr && (counters == nullptr || y == nullptr)))
    return hipErrorInvalidValue;
  u32x4* pl = reinterpret_cast<u32x4*>(f4);
  uint32_t* psc = reinterpret_cast<uint32_t*>(f4 + f4_psc_offset(W.K));
  float* sx = reinterpret_cast<float*>(f4 + f4_sx_offset(W.K));
  if (!planes_ready) {
    hipLaunchKernelGGL(f4_planes_kernel, dim3((steps + 3) / 4), dim3(256), 0, stream, xt, W.K,
                       pl, psc, sx);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int tiles = W.N / 16;
  const dim3 grid((tiles + kF4WgWaves - 1) / kF4WgWaves, slices);
  float* part = reinterpret_cast<float*>(f4 + f4_partial_offset(W.K));
  Fold256Out out{};
  if (U != nullptr)
    out = Fold256Out{reinterpret_cast<const float2*>(U->cs), U->phi_codes, U->phi_step, U->sign_bits,
                y};
#define HARP_F4(B, FO, Q)                                                                     \
  hipLaunchKernelGGL((gemv_f4_kernel<B, FO, Q>), grid, dim3(kF4Threads), 0, stream, W.qweight, \
                     W.scale, W.zero, pl, psc, sx, yt, part, counters, W.N, W.K, slices, out)
#define HARP_F4_BITS(B)                           \
  if (U == nullptr) HARP_F4(B, 0, false);         \
  else if (U->phi_codes != nullptr) {             \
    if (y_dt == HARP_BF16) HARP_F4(B, 2, true);   \
    else HARP_F4(B, 1, true);                     \
  } else if (y_dt == HARP_BF16) HARP_F4(B, 2, false); \
  else HARP_F4(B, 1, false);
  if (W.bits == 2) {
    HARP_F4_BITS(2)
  } else {
    HARP_F4_BITS(4)
  }
#undef HARP_F4_BITS
#undef HARP_F4
  return hipGetLastError();
}

bool gemv_f4_fold_supported(const harp_rotation& U, const harp_qweight& W, int slices) {
  return slices == 1 && U.block == 256 && U.dim == W.N && W.N % 256 == 0 &&
         W.N / 256 <= kF4MaxSplitTiles;
}

}  // namespace harp
