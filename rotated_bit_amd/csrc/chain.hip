// Decode chain: a stack of dependent rotated linears in one launch,
//     y_l = F_{U,l}^T deq(W_l) F_{V,l} y_{l-1},   y_{-1} = x,
// for M <= 4 rows (decode) of D = 4096 or 8192 features with full-width
// butterflies on both sides (b = D).  HARP technical summary §2.1-2.2 (the
// stride stages of each side), §2.4 (the rotated quantized linear, stages
// applied in place without materialising a permutation).
//
// Why one launch.  At D = 4096 and M = 1 a layer moves 5.7 MB, 0.7 us at the
// HBM peak, while a launch costs ~1.6 us and every full-width butterfly needs
// all of its input.  Here the weights of layer l + 1 stream in while layer l
// is still rotating, and the two unavoidable all-to-all steps of a layer are
// workgroup-to-workgroup handoffs (~0.5 us per flag) instead of launches.
//
// Work per layer l (roles by position in the 1-D grid):
//   product (D / 16 workgroups): 16 output features each, the eight
//        features q + j D/8 (j = 0..7) of two residues q, which are exactly
//        the ones that F_U^T's widest three stages mix.  Before waiting,
//        load the features' packed weights and the (cos, sin) pairs of the
//        last three input stages and the first three output stages.  Then
//        wait for z_l (the input after its sign flip and first log2(D) - 3
//        stages), apply the last three stages (strides D/8, D/4, D/2; each
//        thread owns one residue q < D/8 and its eight elements q + j D/8)
//        into LDS, form the float32 product y'_l for its features as the
//        decode GEMV does (lane = quantization group, s (sum q x~ - z sum x~)
//        per group), and apply F_U^T's widest three stages to its 16 values
//        across lanes: the value at q + j D/8 goes to sub-block j.
//   rotation (8 roles per row): sub-block w = 0..7 of D/8 features.  Wait
//        for the sub-block's D/8 values, apply F_U^T's other stages (they
//        never leave a sub-block) and the sign flip: y_l[w-th eighth],
//        stored as the layer's output.  Then, on the same eighth, the next
//        layer's input sign flip and first log2(D) - 3 stages: z_{l+1}.
// The first 8 M product workgroups of layer l + 1 run layer l's rotation
// roles before their own product (their weights are already in flight);
// separate rotation workgroups exist only for x -> z_0 and for the last
// layer's output.  Grid order: those first rotation workgroups, the product
// workgroups of layers 0 .. L-1, the last rotation workgroups.  Each
// workgroup takes more than half of a CU's LDS, so each CU runs one: two
// product workgroups of one layer sharing a CU's vector ALUs finished up to
// twice as late as the rest, and the next layer's workgroup still starts
// (and loads its weights) as soon as the CU's current one ends.
//
// Synchronisation.  A workgroup waits only for workgroups earlier in the
// grid, which the dispatcher has started before it, so the chain makes
// progress whatever number of workgroups fits on the chip at once (no
// co-residency is assumed).  Data crossing workgroups travels through
// device-coherent (sc1, write-through) stores and loads.  z: each rotation
// role waits for the acknowledgement of its stores (vmcnt(0)), then stores
// its flag in 16 copies; the product workgroups poll one copy, then load.
// y' (after F_U^T's widest three stages): every value leaves as a (value,
// epoch) pair in one 8-byte store, and each rotation role polls its D/8
// values themselves, one pair per residue (no acknowledgement wait and no
// flag on that side).  Flags and tags hold the launch's epoch (workspace
// word 0, plus one), so nothing needs resetting: the last workgroup to end
// advances the epoch for the next launch.  Every wait is bounded: a wait that
// runs out records an error in workspace word 1 and ends its workgroup, so
// the grid always drains.
#include "chain.hpp"

#include "device_common.hpp"
#include "unpack.hpp"

namespace harp {
namespace {

constexpr int kThreadsC = 512;
constexpr int kWavesC = kThreadsC / kWave;
constexpr int kRowsC = 16;                 // output features per product workgroup
constexpr int kGS = kGroup + 4;            // padded LDS floats per quantization group
constexpr int kSpinLimit = 1 << 20;        // polls before a wait gives up (~0.5 s)

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int LOGD>
struct ChainPlan {
  static constexpr int D = 1 << LOGD;
  static constexpr int BB = D / 8;         // sub-block of the rotation workgroups
  static constexpr int LB = LOGD - 3;      // stages inside a sub-block
  static constexpr int NRB = (LB + 2) / 3; // register rounds over a sub-block
  static constexpr int TB = BB / 8;        // threads of a sub-block round (8 elements each)
  static constexpr int QPT = BB / kThreadsC;   // residues per thread
  static constexpr int NG = D / kRowsC;    // product workgroups per layer
  static constexpr int GPL = D / 64 / kWave;   // quantization groups per lane
};

__device__ __forceinline__ int elem_index8(int t, int j, int s0, int R) {
  const int rest = (t << (3 - R)) + (j >> R);
  const int jl = j & ((1 << R) - 1);
  const int lo = rest & ((1 << s0) - 1);
  const int hi = rest >> s0;
  return (hi << (s0 + R)) | (jl << s0) | lo;
}
__device__ __forceinline__ int zero_bit(int p, int k) {
  return ((p >> k) << (k + 1)) | (p & ((1 << k) - 1));
}
__device__ __forceinline__ int del_bit(int i, int s) {
  return ((i >> (s + 1)) << s) | (i & ((1 << s) - 1));
}
__device__ __forceinline__ int round_w(int r, int L) { return (L - 3 * r) < 3 ? (L - 3 * r) : 3; }
__device__ __forceinline__ int padg(int i) { return (i >> 6) * kGS + (i & 63); }

__device__ __forceinline__ void bfly(float& a, float& b, float2 cs) {
  const float x = a, y = b;
  a = fmaf(cs.x, x, cs.y * y);
  b = fmaf(cs.y, x, -(cs.x * y));
}

// One output of a butterfly whose two inputs sit in lanes `bit` apart: the
// lane with `bit` clear holds the first input and keeps the first output (the
// same arithmetic as bfly).
__device__ __forceinline__ float bfly_lane(float v, int bit, bool high, float2 cs) {
  const float w = shfl_xor(v, bit);
  return high ? fmaf(cs.y, w, -(cs.x * v)) : fmaf(cs.x, v, cs.y * w);
}

// ---- device-coherent memory operations ------------------------------------

__device__ __forceinline__ uint32_t ld_flag(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sc1x4(float* p, floatx4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Eight sc1 loads p[0], p[s], ..., p[7 s], waited for inside the asm block.
__device__ __forceinline__ void ld8_sc1(const float* p, int s, float (&v)[8]) {
  float r0, r1, r2, r3, r4, r5, r6, r7;
  asm volatile(
      "global_load_dword %0, %8, off sc1\n\t"
      "global_load_dword %1, %9, off sc1\n\t"
      "global_load_dword %2, %10, off sc1\n\t"
      "global_load_dword %3, %11, off sc1\n\t"
      "global_load_dword %4, %12, off sc1\n\t"
      "global_load_dword %5, %13, off sc1\n\t"
      "global_load_dword %6, %14, off sc1\n\t"
      "global_load_dword %7, %15, off sc1\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(p), "v"(p + s), "v"(p + 2 * s), "v"(p + 3 * s), "v"(p + 4 * s), "v"(p + 5 * s),
        "v"(p + 6 * s), "v"(p + 7 * s)
      : "memory");
  v[0] = r0; v[1] = r1; v[2] = r2; v[3] = r3; v[4] = r4; v[5] = r5; v[6] = r6; v[7] = r7;
}
// A (value, tag) pair with one 8-byte store: a reader sees both or neither.
__device__ __forceinline__ void st_pair_sc1(u32x2 *p, float v, uint32_t tag) {
  u32x2 d;
  d[0] = __float_as_uint(v);
  d[1] = tag;
  asm volatile("global_store_dwordx2 %0, %1, off sc1" ::"v"(p), "v"(d) : "memory");
}
// N (1 or 2) device-coherent pair loads p[0], p[s], waited for inside the
// asm block.
template <int N>
__device__ __forceinline__ void ld_pairs_sc1(const u32x2* p, int s, u32x2 (&v)[N]) {
  static_assert(N == 1 || N == 2, "one or two pairs");
  if constexpr (N == 1) {
    u32x2 r0;
    asm volatile("global_load_dwordx2 %0, %1, off sc1\n\ts_waitcnt vmcnt(0)"
                 : "=&v"(r0) : "v"(p) : "memory");
    v[0] = r0;
  } else {
    u32x2 r0, r1;
    asm volatile(
        "global_load_dwordx2 %0, %2, off sc1\n\t"
        "global_load_dwordx2 %1, %3, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(r0), "=&v"(r1) : "v"(p), "v"(p + s) : "memory");
    v[0] = r0;
    v[1] = r1;
  }
}
// Polls p[0], p[s] (N of them) until every tag of the wave's loads holds
// `tag`; the values in v.  False if the wait ran out.
template <int N>
__device__ __forceinline__ bool poll_pairs(const u32x2* p, int s, uint32_t tag, float (&v)[N]) {
  int spins = 0;
  while (true) {
    u32x2 r[N];
    ld_pairs_sc1<N>(p, s, r);
    bool mine = true;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      mine = mine && r[j][1] == tag;
      v[j] = __uint_as_float(r[j][0]);
    }
    if (__all(mine)) return true;
    if (++spins > kSpinLimit) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Wait until every flag of f[0..n) holds `epoch`; n a multiple of 4, at
// most 256 (16-byte aligned f).  One wave polls, four flags per lane with one
// load; the others wait at the barrier.  False if the wait ran out (recorded
// in ctrl[1]).
__device__ __forceinline__ bool wait_flags(const uint32_t* f, int n, uint32_t epoch,
                                           uint32_t* ctrl, int* ok) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const bool has = 4 * lane < n;
    const uint32_t* p = f + 4 * (has ? lane : 0);
    int spins = 0;
    bool done = false;
    while (!done) {
      u32x4 v;
      asm volatile("global_load_dwordx4 %0, %1, off sc1\n\ts_waitcnt vmcnt(0)"
                   : "=&v"(v) : "v"(p) : "memory");
      done = __all(!has || (v[0] == epoch && v[1] == epoch && v[2] == epoch && v[3] == epoch));
      if (!done) {
        if (++spins > kSpinLimit) break;
        __builtin_amdgcn_s_sleep(1);
      }
    }
    if (lane == 0) {
      *ok = done ? 1 : 0;
      if (!done) st_flag(ctrl + 1, 1u);
    }
  }
  __syncthreads();
  return *ok != 0;
}

// Orders a wave's LDS stores before its next loads (a wave's LDS accesses
// run in issue order; the fences keep the compiler from moving them).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- the kernel -----------------------------------------------------------

template <int LOGD, int BITS, int MT>
__global__ __launch_bounds__(kThreadsC) void chain_kernel(ChainArgs a) {
  using P = ChainPlan<LOGD>;
  constexpr int D = P::D, BB = P::BB, LB = P::LB, NRB = P::NRB, TB = P::TB, QPT = P::QPT;
  constexpr int NG = P::NG, GPL = P::GPL;
  constexpr int LOG = LOGD;
  constexpr int NWG = 2 * BITS;            // uint32 words per quantization group
  constexpr int RW = kRowsC / kWavesC;     // feature rows per wave (2)
  constexpr int SEGC = BITS == 2 ? 16 : 8; // codes per inner segment
  constexpr float kCodeScale = BITS == 3 ? 1.0f : kFp8CodeScale;  // codes as q 2^-9
  // LDS floats: the product's padded x~ and group sums, or the rotation
  // role's sub-block and (4096-wide layers) its staged (cos, sin) pairs.
  // At most 80 KB, so that two workgroups run per CU: the next layer's
  // product workgroups are resident (and their weights in flight) while the
  // current layer runs.
  constexpr bool kCoefLds = LOGD == 12;
  constexpr int kLdsValu = MT * (D / 64) * kGS + MT * (D / 64) + MT * kRowsC;
  constexpr int kLdsRot = BB + (kCoefLds ? 2 * TB * LB * 4 * 2 : 0);
  constexpr int kLds = kLdsValu > kLdsRot ? kLdsValu : kLdsRot;
  static_assert(kLds * 4 <= 80 * 1024, "two workgroups per CU");
  __shared__ __attribute__((aligned(16))) float smem[kLds];
  __shared__ int ok_flag;

  const int tid = threadIdx.x;
  const int nR = 8 * a.M;
  const int L = a.n_layers;
  uint32_t* ctrl = a.ws;
  const uint32_t epoch = ld_flag(ctrl) + 1u;
  uint32_t* flagsR = a.ws + kChainFlagsOffset;                   // [phase][copy][32]
  float* zbuf = reinterpret_cast<float*>(a.ws + kChainDataOffset);              // [phase][M][D]
  u32x2* ypbuf = reinterpret_cast<u32x2*>(
      zbuf + static_cast<size_t>(kChainMaxLayers + 1) * kChainMaxM * D);        // [layer][M][D]

  // The rotation role of phase rl (F_U^T of layer rl, then the first
  // stages of layer rl + 1), sub-block ri; false if a wait ran out.
  auto rot_role = [&](const int rl, const int ri) -> bool {
    // ======================= rotation workgroup =======================
    const int m = ri >> 3;
    const int wsub = ri & 7;
    const bool has_u = rl >= 0;
    const bool has_v = rl + 1 < L;
    const bool uthr = tid < TB;
    const bool vthr = tid >= TB && tid < 2 * TB;
    const int tp = uthr ? tid : tid - TB;
    float* u = smem;                                     // [BB]
    auto cu = [&](int s, int i) { return s * (D / 2) + del_bit(i, s); };
    // 1. coefficients first (they do not depend on the data)
    // sub-block stage pairs, F_U^T for uthr and F_V for vthr: in registers,
    // or (kCoefLds) staged in LDS behind the sub-block, one private row per
    // thread, so that the role needs few registers next to the product's
    // prefetched weights
    float2 hb[kCoefLds ? 1 : LB][4];
    float2* coefl = reinterpret_cast<float2*>(smem + BB) +
                    static_cast<size_t>((uthr ? 0 : TB) + tp) * LB * 4;
    uint32_t sbits = 0;
    if ((uthr && has_u) || (vthr && has_v)) {
      const ChainLayer& Ls = a.layer[uthr ? rl : rl + 1];
      const float2* cs = uthr ? Ls.cs_u : Ls.cs_v;
      const uint32_t* sg = uthr ? Ls.sign_u : Ls.sign_v;
  #pragma unroll
      for (int r = 0; r < NRB; ++r) {
        const int s0 = 3 * r;
        const int R = round_w(r, LB);
  #pragma unroll
        for (int k = 0; k < 3; ++k) {
          if (k < R) {
  #pragma unroll
            for (int p = 0; p < 4; ++p)
            {
              const float2 c2 = cs[cu(s0 + k, wsub * BB + elem_index8(tp, zero_bit(p, k), s0, R))];
              if constexpr (kCoefLds) coefl[(s0 + k) * 4 + p] = c2;
              else hb[s0 + k][p] = c2;
            }
          }
        }
      }
      const int g0 = wsub * BB + tp * 8;
      sbits = sg[g0 >> 5] >> (g0 & 31);
    }
    // Both sides on the same wave (4096-wide layers: a side's rounds take one
    // wave and the coefficients of both sides sit in LDS): F_U^T's last
    // round and F_V's first one cover the same elements per thread, so they
    // run back to back in registers.  Otherwise F_U^T on the first TB
    // threads and F_V on the next TB.
    constexpr bool kFuse = kCoefLds && TB <= kWave;
    static_assert(kFuse || !kCoefLds, "LDS-staged coefficients come with one-wave rounds");
    uint32_t vbits = sbits;
    if constexpr (kFuse) {
      if (uthr && has_v) {
        const int g0 = wsub * BB + tp * 8;
        vbits = a.layer[rl + 1].sign_v[g0 >> 5] >> (g0 & 31);
      }
    }
    const float2* coef_u = reinterpret_cast<const float2*>(smem + BB) +
                           static_cast<size_t>(tp) * LB * 4;
    const float2* coef_v = coef_u + static_cast<size_t>(kFuse ? TB : 0) * LB * 4;
    auto pair_u = [&](int st, int p) -> float2 {
      if constexpr (kCoefLds) return coef_u[st * 4 + p];
      else return hb[st][p];
    };
    auto pair_v = [&](int st, int p) -> float2 {
      if constexpr (kCoefLds) return coef_v[st * 4 + p];
      else return hb[st][p];
    };
    auto load8 = [&](int r, float (&v)[8]) {
  #pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = u[elem_index8(tp, j, 3 * r, round_w(r, LB))];
    };
    auto store8 = [&](int r, const float (&v)[8]) {
  #pragma unroll
      for (int j = 0; j < 8; ++j) u[elem_index8(tp, j, 3 * r, round_w(r, LB))] = v[j];
    };
    // F_U^T's stages of round r (descending)
    auto u_stages = [&](int r, float (&v)[8]) {
      const int s0 = 3 * r;
      const int R = round_w(r, LB);
  #pragma unroll
      for (int kk = 0; kk < 3; ++kk) {
        const int k = 2 - kk;
        if (k < R) {
  #pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int j1 = zero_bit(p, k);
            bfly(v[j1], v[j1 | (1 << k)], pair_u(s0 + k, p));
          }
        }
      }
    };
    // after round 0: the sign flip and the layer output y_rl (contiguous
    // elements 8 tp .. 8 tp + 7); the value kept is the stored one
    auto u_out = [&](float (&v)[8]) {
  #pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = flip_sign(v[j], (sbits >> j) & 1u);
      const size_t off = static_cast<size_t>(m) * D + wsub * BB + tp * 8;
      if (a.y_bf16) {
        u32x4 pk;
  #pragma unroll
        for (int j = 0; j < 4; ++j) pk[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.layer[rl].y) + off) = pk;
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[2 * j] = __uint_as_float(pk[j] << 16);
          v[2 * j + 1] = __uint_as_float(pk[j] & 0xffff0000u);
        }
      } else {
        float* yo = static_cast<float*>(a.layer[rl].y) + off;
        *reinterpret_cast<float4*>(yo) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(yo + 4) = make_float4(v[4], v[5], v[6], v[7]);
      }
    };
    // the next layer's input sign flip (before round 0) and F_V's stages of
    // round r (ascending)
    auto v_stages = [&](int r, float (&v)[8]) {
      const int s0 = 3 * r;
      const int R = round_w(r, LB);
      if (r == 0) {
  #pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = flip_sign(v[j], (vbits >> j) & 1u);
      }
  #pragma unroll
      for (int k = 0; k < 3; ++k) {
        if (k < R) {
  #pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int j1 = zero_bit(p, k);
            bfly(v[j1], v[j1 | (1 << k)], pair_v(s0 + k, p));
          }
        }
      }
    };
    // 2. the input of this sub-block: y'_l after F_U^T's widest three
    //    stages (applied by the product workgroups), or the chain input x
    //    for the first phase
    int failed = 0;
    if (has_u) {
      const u32x2* yp = ypbuf + (static_cast<size_t>(rl) * kChainMaxM + m) * D;
      float v[QPT];
      if (!poll_pairs<QPT>(yp + static_cast<size_t>(wsub) * BB + tid, kThreadsC, epoch, v))
        failed = 1;
  #pragma unroll
      for (int qi = 0; qi < QPT; ++qi) u[tid + kThreadsC * qi] = v[qi];
      if (failed && (tid & (kWave - 1)) == 0) st_flag(ctrl + 1, 1u);
    } else {
      for (int i = tid; i < BB; i += kThreadsC) {
        const size_t off = static_cast<size_t>(m) * D + wsub * BB + i;
        u[i] = a.x_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(a.x)[off])
                        : static_cast<const float*>(a.x)[off];
      }
    }
    if (__syncthreads_or(failed)) return false;
    if constexpr (kFuse) {
      // 3-4. one wave: F_U^T's rounds (descending), the output, the next
      //      layer's sign flip and F_V's rounds (ascending).  Each round's
      //      (cos, sin) pairs are read from LDS during the round before, so
      //      that a round waits only for its elements.
      typedef float2 Coef[3][4];
      auto load_c = [&](const float2* base, int r, Coef& c) {
  #pragma unroll
        for (int k = 0; k < 3; ++k)
          if (k < round_w(r, LB))
  #pragma unroll
            for (int p = 0; p < 4; ++p) c[k][p] = base[(3 * r + k) * 4 + p];
      };
      auto stages_c = [&](bool descending, int r, float (&v)[8], const Coef& c) {
        const int R = round_w(r, LB);
  #pragma unroll
        for (int kk = 0; kk < 3; ++kk) {
          const int k = descending ? 2 - kk : kk;
          if (k < R) {
  #pragma unroll
            for (int p = 0; p < 4; ++p) {
              const int j1 = zero_bit(p, k);
              bfly(v[j1], v[j1 | (1 << k)], c[k][p]);
            }
          }
        }
      };
      auto flip_v = [&](float (&v)[8]) {
  #pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = flip_sign(v[j], (vbits >> j) & 1u);
      };
      if (uthr) {
        float v[8];
        Coef c, cn;
        if (has_u) {
          load_c(coef_u, NRB - 1, c);
  #pragma unroll
          for (int qq = 0; qq + 1 < NRB; ++qq) {
            const int r = NRB - 1 - qq;
            load8(r, v);
            load_c(coef_u, r - 1, cn);
            stages_c(true, r, v, c);
            store8(r, v);
  #pragma unroll
            for (int k = 0; k < 3; ++k)
  #pragma unroll
              for (int p = 0; p < 4; ++p) c[k][p] = cn[k][p];
            wave_sync();
          }
          load8(0, v);
          if (has_v) load_c(coef_v, 0, cn);
          stages_c(true, 0, v, c);
          u_out(v);
          if (has_v) {
            if (NRB > 1) load_c(coef_v, 1, c);
            flip_v(v);
            stages_c(false, 0, v, cn);
          }
          store8(0, v);
        } else {
          load8(0, v);
          load_c(coef_v, 0, cn);
          if (NRB > 1) load_c(coef_v, 1, c);
          flip_v(v);
          stages_c(false, 0, v, cn);
          store8(0, v);
        }
        if (has_v) {
  #pragma unroll
          for (int r = 1; r < NRB; ++r) {
            wave_sync();
            load8(r, v);
            if (r + 1 < NRB) load_c(coef_v, r + 1, cn);
            stages_c(false, r, v, c);
            store8(r, v);
  #pragma unroll
            for (int k = 0; k < 3; ++k)
  #pragma unroll
              for (int p = 0; p < 4; ++p) c[k][p] = cn[k][p];
          }
        }
      }
      __syncthreads();
      if (!has_v) return true;
    } else {
      // 3. F_U^T's stages inside the sub-block (descending), the sign flip,
      //    the rl output.  One sub-block round per three stages; when the
      //    round's threads are a single wave (TB <= 64) only that wave's LDS
      //    order is needed between rounds, else a workgroup barrier.
      constexpr bool kWaveRounds = TB <= kWave;
      auto u_round = [&](int r) {
        float v[8];
        load8(r, v);
        u_stages(r, v);
        if (r == 0) u_out(v);
        store8(r, v);
      };
      if (has_u) {
        if constexpr (kWaveRounds) {
          if (uthr) {
  #pragma unroll
            for (int qq = 0; qq < NRB; ++qq) {
              u_round(NRB - 1 - qq);
              if (qq + 1 < NRB) wave_sync();
            }
          }
          __syncthreads();
        } else {
  #pragma unroll
          for (int qq = 0; qq < NRB; ++qq) {
            if (uthr) u_round(NRB - 1 - qq);
            __syncthreads();
          }
        }
      }
      if (!has_v) return true;
      // 4. the next rl's input sign flip and stages 0 .. LB-1 (ascending)
      auto v_round = [&](int r) {
        float v[8];
        load8(r, v);
        v_stages(r, v);
        store8(r, v);
      };
      if constexpr (kWaveRounds) {
        if (vthr) {
  #pragma unroll
          for (int r = 0; r < NRB; ++r) {
            v_round(r);
            if (r + 1 < NRB) wave_sync();
          }
        }
        __syncthreads();
      } else {
  #pragma unroll
        for (int r = 0; r < NRB; ++r) {
          if (vthr) v_round(r);
          __syncthreads();
        }
      }
    }
    // 5. z_{l+1}: the sub-block to the next rl's product workgroups (256 of
    //    them read all of z, so plain values and a flag rather than tagged
    //    pairs, which would double that traffic)
    float* zo = zbuf + (static_cast<size_t>(rl + 1) * kChainMaxM + m) * D + wsub * BB;
    for (int i = tid; i < BB / 4; i += kThreadsC)
      st_sc1x4(zo + 4 * i, *reinterpret_cast<const floatx4*>(&u[4 * i]));
    wait_stores();
    __syncthreads();
    // one copy of the flag per group of product workgroups, so that their
    // polls spread over several lines
    if (tid < kChainFlagCopies)
      st_flag(flagsR + ((rl + 1) * kChainFlagCopies + tid) * 32 + ri, epoch);
    return true;
  };

  // Roles by position: per layer its D/16 product workgroups, the first 8 M
  // of which first run the previous phase's rotation role (for layer 0: the
  // chain input x -> z_0); at the end the last layer's rotation workgroups.
  // Every layer is exactly one workgroup per CU-slot's worth (D/16 = 256 at
  // D = 4096 for two slots on 256 CUs... per layer one slot per CU), so a
  // workgroup that ends frees the slot the workgroup two layers later takes.
  int layer, idx;
  bool is_g, dual = false;
  {
    const int b = blockIdx.x;
    if (b < L * NG) {
      layer = b / NG;
      idx = b - layer * NG;
      is_g = true;
      dual = idx < nR;
    } else {
      layer = L - 1;
      is_g = false;
      idx = b - L * NG;
    }
  }
  if (!is_g) {
    rot_role(layer, idx);
    // The last of the final rotation workgroups to end advances the epoch
    // for the next launch.  Every other workgroup has read the epoch by
    // then: each one feeds, through the chain of waits, the data that every
    // final rotation workgroup has consumed.
    __syncthreads();
    if (tid == 0 && __hip_atomic_fetch_add(ctrl + 2, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT) == static_cast<uint32_t>(nR - 1)) {
      st_flag(ctrl + 2, 0u);
      st_flag(ctrl, epoch);
    }
    return;
  }
  {
    // ======================= product workgroup =======================
    const ChainLayer& Ly = a.layer[layer];
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    constexpr int G = D / kGroup;
    // local row j = wave RW + r is feature q + BB p of residue q = 2 idx +
    // j / 8, p = j % 8: the eight features that F_U^T's widest three stages
    // mix, for two residues
    auto row_of = [&](int j) { return 2 * idx + (j >> 3) + BB * (j & 7); };
    const size_t WPR = static_cast<size_t>(D) * BITS / 32;
    // 1. this lane's groups of the wave's feature rows
    uint32_t w[GPL][RW][NWG];
    uint16_t s16[GPL][RW], z16[GPL][RW];
#pragma unroll
    for (int gl = 0; gl < GPL; ++gl)
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const int n = row_of(wave * RW + r);
        const int g = lane + kWave * gl;
        load_group<BITS>(Ly.qw + static_cast<size_t>(n) * WPR + static_cast<size_t>(g) * NWG,
                         w[gl][r]);
        s16[gl][r] = Ly.sc[static_cast<size_t>(n) * G + g];
        z16[gl][r] = Ly.zr[static_cast<size_t>(n) * G + g];
      }
    // F_U^T's widest three stages for lane (m, j) of wave 0, j = lane % 16:
    // the pairs of position q + BB p at strides D/2, D/4, D/8
    float2 hc[3];
    if (wave == 0) {
      const int j = lane & (kRowsC - 1);
      const int q = 2 * idx + (j >> 3), p = j & 7;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int s = LOG - 1 - k;
        const int plow = p & ~(4 >> k);
        hc[k] = Ly.cs_u[s * (D / 2) + del_bit(q + BB * plow, s)];
      }
    }
    // 2. (the first 8 M workgroups of a layer: the previous layer's
    //    rotation role first), then z_l from the rotation role
    if (dual && !rot_role(layer - 1, idx)) return;
    float2 ct[QPT][3][4];
#pragma unroll
    for (int qi = 0; qi < QPT; ++qi) {
      const int q = tid + kThreadsC * qi;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int s = LB + k;
#pragma unroll
        for (int p = 0; p < 4; ++p)
          ct[qi][k][p] = Ly.cs_v[s * (D / 2) + del_bit(q + BB * zero_bit(p, k), s)];
      }
    }
    if (!wait_flags(flagsR + (layer * kChainFlagCopies + idx % kChainFlagCopies) * 32, nR, epoch,
                    ctrl, &ok_flag))
      return;
    const float* zin = zbuf + static_cast<size_t>(layer) * kChainMaxM * D;
    float* xs = smem;                                    // [MT][G * kGS]
    float* sxs = smem + MT * G * kGS;                    // [MT][G]
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int qi = 0; qi < QPT; ++qi) {
        const int q = tid + kThreadsC * qi;
        float v[8];
        if (m < a.M) {
          ld8_sc1(zin + static_cast<size_t>(m) * D + q, BB, v);
#pragma unroll
          for (int k = 0; k < 3; ++k)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const int j1 = zero_bit(p, k);
              bfly(v[j1], v[j1 | (1 << k)], ct[qi][k][p]);
            }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) xs[m * G * kGS + padg(q + BB * j)] = v[j];
      }
    }
    __syncthreads();
    // 3. per-group sums of x~ (16 lanes per group, fixed order)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int h = 0; h < G * 16 / kThreadsC; ++h) {
        const int f = tid + h * kThreadsC;
        const int gi = f >> 4;
        const float4 v = *reinterpret_cast<const float4*>(&xs[m * G * kGS + gi * kGS + (f & 15) * 4]);
        float part = (v.x + v.y) + (v.z + v.w);
        part += shfl_xor(part, 8);
        part += shfl_xor(part, 4);
        part += shfl_xor(part, 2);
        part += shfl_xor(part, 1);
        if ((f & 15) == 0) sxs[m * G + gi] = part;
      }
    }
    __syncthreads();
    // 4. the product: s (sum q x~ - z sum x~) per group, float32
    constexpr int V = RW * MT;
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int gl = 0; gl < GPL; ++gl) {
      const int g = lane + kWave * gl;
      float dot[RW][MT];
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) dot[r][m] = 0.0f;
#pragma unroll
      for (int i = 0; i < kGroup / SEGC; ++i) {
        float q[RW][SEGC];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          // 2 and 4 bits: FP8 decodes of the masked codes, q 2^-9 exactly
          if constexpr (BITS == 2) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const uint32_t mm = (w[gl][r][i] >> (2 * t)) & 0x03030303u;
              fp8_codes4(mm, q[r][t], q[r][t + 4], q[r][t + 8], q[r][t + 12]);
            }
          } else if constexpr (BITS == 4) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const uint32_t mm = (w[gl][r][i] >> (4 * t)) & 0x0f0f0f0fu;
              fp8_codes4(mm, q[r][t], q[r][t + 2], q[r][t + 4], q[r][t + 6]);
            }
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) q[r][j] = static_cast<float>(code_at<3, 6>(w[gl][r], 8 * i + j));
          }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float xv[SEGC];
#pragma unroll
          for (int c = 0; c < SEGC / 4; ++c) {
            const float4 v = *reinterpret_cast<const float4*>(&xs[m * G * kGS + g * kGS + i * SEGC + 4 * c]);
            xv[4 * c + 0] = v.x;
            xv[4 * c + 1] = v.y;
            xv[4 * c + 2] = v.z;
            xv[4 * c + 3] = v.w;
          }
#pragma unroll
          for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int j = 0; j < SEGC; ++j) dot[r][m] = fmaf(q[r][j], xv[j], dot[r][m]);
        }
      }
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const float s = f16_to_f32(s16[gl][r]);
        const float z = f16_to_f32(z16[gl][r]);
#pragma unroll
        for (int m = 0; m < MT; ++m)
          acc[r * MT + m] = fmaf(s, fmaf(-z, sxs[m * G + g], dot[r][m] * kCodeScale),
                                 acc[r * MT + m]);
      }
    }
    wave_transpose_reduce<V>(acc, lane);
    // y'_l through F_U^T's widest three stages (strides D/2, D/4, D/8),
    // whose butterflies stay inside this workgroup's rows: lane (m, j) of
    // wave 0 ends with position q + BB p, the input of sub-block p.  Stored
    // as (value, epoch) pairs in position order, so that sub-block p reads
    // one contiguous run of BB pairs (polling a strided eighth of every line
    // took ~0.5 us longer to see the last value); the rotation roles poll
    // the values themselves (no acknowledgement wait and no flag).
    float* yg = sxs + MT * G;                            // [MT][kRowsC]
#pragma unroll
    for (int tv = 0; tv < V; ++tv) {
      if (lane == lane_of_value<V>(tv)) {
        const int r = tv / MT;
        const int m = tv - r * MT;
        yg[m * kRowsC + wave * RW + r] = acc[0];
      }
    }
    __syncthreads();
    if (wave == 0) {
      static_assert(MT * kRowsC <= kWave, "one wave holds every row of every input");
      const int m = lane / kRowsC;
      const int j = lane & (kRowsC - 1);
      float v = lane < MT * kRowsC ? yg[lane] : 0.0f;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int bit = 4 >> k;
        v = bfly_lane(v, bit, (j & bit) != 0, hc[k]);
      }
      if (m < a.M)
        st_pair_sc1(ypbuf + (static_cast<size_t>(layer) * kChainMaxM + m) * D +
                        static_cast<size_t>(j & 7) * BB + 2 * idx + (j >> 3),
                    v, epoch);
    }
    return;
  }

}

template <int LOGD, int BITS, int MT>
hipError_t launch_chain_t(const ChainArgs& a, hipStream_t stream) {
  using P = ChainPlan<LOGD>;
  const int nR = 8 * a.M;
  const dim3 grid(a.n_layers * P::NG + nR);
  hipLaunchKernelGGL((chain_kernel<LOGD, BITS, MT>), grid, dim3(kThreadsC), 0, stream, a);
  return hipGetLastError();
}

template <int LOGD, int BITS>
hipError_t launch_chain_m(const ChainArgs& a, hipStream_t stream) {
  if (a.M == 1) return launch_chain_t<LOGD, BITS, 1>(a, stream);
  if (a.M == 2) return launch_chain_t<LOGD, BITS, 2>(a, stream);
  if constexpr (LOGD == 12) return launch_chain_t<LOGD, BITS, 4>(a, stream);
  return hipErrorInvalidValue;
}

template <int LOGD>
hipError_t launch_chain_d(const ChainArgs& a, int bits, hipStream_t stream) {
  switch (bits) {
    case 2: return launch_chain_m<LOGD, 2>(a, stream);
    case 3: return launch_chain_m<LOGD, 3>(a, stream);
    case 4: return launch_chain_m<LOGD, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_chain(const ChainArgs& a, int dim, int bits, hipStream_t stream) {
  if (dim == 4096) return launch_chain_d<12>(a, bits, stream);
  if (dim == 8192) return launch_chain_d<13>(a, bits, stream);
  return hipErrorInvalidValue;
}

}  // namespace harp
