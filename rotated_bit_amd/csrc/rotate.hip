// Butterfly rotation kernels: x~ = F x and y = F^T y'.
//
// HARP technical summary §2.1-2.2 ("HARP: Hadamard-Preconditioned Adaptive
// Rotation Processor for Extreme LLM Quantization", gist.science): the map
// is a product of L = log2(b) sparse stages; stage s applies a 2x2 block
// [[c, s], [s, -c]] to every pair (i, i + 2^s) with bit s of i clear, and
// the pair's index in the stage is i with bit s deleted.  F = B_{L-1} .. B_0 D
// and F^T = D B_0 .. B_{L-1}.  Technical summary §2.4: the stride stages are
// applied without materialising a permutation.
//
// gfx950 mapping.  One workgroup slot owns one length-b block of one row.
// Each thread holds E = 8 elements in registers, so up to three consecutive
// stages run in registers per round (a radix-8 sub-butterfly over the
// strides 2^s0, 2^(s0+1), 2^(s0+2)); rounds exchange through LDS with one
// barrier each.  The first round reads global memory and the last writes
// it, so b = 4096 needs three LDS exchanges for twelve stages.  All of a
// thread's (cos, sin) pairs are loaded into registers before the first
// round, so their memory latency is paid once.
//
// Angles stored as int8 codes (technical summary §2.4: the HARP parameters
// may be kept in eight bits): t = pi/4 + code * step.  Every workgroup
// evaluates (cos t, sin t) once for all 256 codes into an LDS table while
// its code loads are in flight, then gathers its pairs from the table, so a
// block's coefficient fetch is one byte per pair instead of eight.
#include "f4_planes.hpp"
#include "launch.hpp"
#include "validate.hpp"

#include <type_traits>
#include "device_common.hpp"

namespace harp {
namespace {

// EL_ = log2 elements per thread (stages per register round).  The default
// 3 keeps 8 elements per thread; 2 gives a b = 4096 block 1024 threads,
// which is what a single CU needs to pull a block's 196 KB of (cos, sin)
// pairs at full rate when only a few blocks are in flight.
template <int LOGB, int EL_ = (LOGB < 3 ? LOGB : 3)>
struct Plan {
  static constexpr int L = LOGB;
  static constexpr int EL = EL_;
  static constexpr int E = 1 << EL;
  static constexpr int B = 1 << LOGB;
  static constexpr int TPB = B >> EL;                  // threads per block row
  static constexpr int NR = (L + EL - 1) / EL;         // register rounds
  static constexpr int SLOTS = TPB >= 256 ? 1 : 256 / TPB;
  static constexpr int THREADS = TPB * SLOTS;
};

__host__ __device__ constexpr int round_width(int r, int EL, int L) {
  return (L - r * EL) < EL ? (L - r * EL) : EL;
}

// Index inside the block of local element j of thread t in a round that
// covers stages s0 .. s0+R-1: the low R bits of j select the position along
// those strides, the remaining bits (thread index, high bits of j) fill the
// other index bits in order.
template <int E>
__device__ __forceinline__ int elem_index(int t, int j, int s0, int R) {
  const int rest = t * (E >> R) + (j >> R);
  const int jl = j & ((1 << R) - 1);
  const int lo = rest & ((1 << s0) - 1);
  const int hi = rest >> s0;
  return (hi << (s0 + R)) | (jl << s0) | lo;
}

__device__ __forceinline__ int insert_zero_bit(int p, int k) {
  return ((p >> k) << (k + 1)) | (p & ((1 << k) - 1));
}

__device__ __forceinline__ int delete_bit(int i, int s) {
  return ((i >> (s + 1)) << s) | (i & ((1 << s) - 1));
}

// Element access in the boundary dtypes (float32, or bf16 as uint16).
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
__device__ __forceinline__ void from_f32(float& d, float v) { d = v; }
__device__ __forceinline__ void from_f32(uint16_t& d, float v) { d = f32_to_bf16(v); }

// E contiguous elements starting at p (E-aligned), as one or two vector
// accesses.
template <typename T, int E>
struct alignas(sizeof(T) * E < 16 ? sizeof(T) * E : 16) Pack { T v[E]; };

template <typename T, int E>
__device__ __forceinline__ void load_contig(const T* p, float (&v)[E]) {
  const Pack<T, E> pk = *reinterpret_cast<const Pack<T, E>*>(p);
#pragma unroll
  for (int j = 0; j < E; ++j) v[j] = to_f32(pk.v[j]);
}

template <typename T, int E>
__device__ __forceinline__ void store_contig(T* p, const float (&v)[E]) {
  Pack<T, E> pk;
#pragma unroll
  for (int j = 0; j < E; ++j) from_f32(pk.v[j], v[j]);
  *reinterpret_cast<Pack<T, E>*>(p) = pk;
}

// Orders one round's LDS stores before the next round's loads.  Across a
// workgroup that is a barrier; inside one wave, whose LDS accesses execute
// in issue order, it is a wave-scope fence that also keeps the compiler
// from moving the loads above the stores.
template <bool WAVE_LOCAL>
__device__ __forceinline__ void slot_sync() {
  if constexpr (WAVE_LOCAL) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    __syncthreads();
  }
}

// SUB_ = 0: blocks of b = 2^LOGB with their own pairs.  SUB_ = 3: the
// blocks are the eight sub-blocks of a block of 8b and the stages applied
// are that block's first LOGB stages (which never leave a sub-block); the
// pairs are then addressed in the big block's layout.
template <int LOGB, int EL_, bool TRANSPOSE, bool Q8, typename TIn, typename TOut, int SUB_ = 0>
__global__ __launch_bounds__((Plan<LOGB, EL_>::THREADS)) void rotate_kernel(
    const TIn* __restrict__ in, TOut* __restrict__ out,
    const float2* __restrict__ cs, const int8_t* __restrict__ codes, float step,
    const uint32_t* __restrict__ sign, int dim, int M, int rows_per_slot) {
  using P = Plan<LOGB, EL_>;
  constexpr int B = P::B;
  constexpr int E = P::E;
  constexpr int EL = P::EL;
  constexpr int L = P::L;
  constexpr int NR = P::NR;
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ float2 table[Q8 ? 256 : 1];   // (cos t, sin t) by code + 128

  // A block row of at most 64 threads lies inside one wave, and its LDS
  // exchange region belongs to it alone: the rounds then only need the
  // wave's own LDS order, not a workgroup barrier.
  constexpr bool kWaveLocal = P::TPB <= kWave;
  // small blocks: all slots of the workgroup share the block's pairs
  constexpr bool kCoefLds = kWaveLocal && !Q8 && NR > 1 && SUB_ == 0;
  const int tid = threadIdx.x;
  const int slot = tid / P::TPB;
  const int t = tid - slot * P::TPB;
  const int blk = blockIdx.x;
  float* u = lds + slot * B;

  // The first round's input of a row, fetched raw (not converted, not
  // sign-flipped) so that nothing waits for it before the coefficient
  // loads are issued; rows past M read as zeros.
  constexpr int kR0 = TRANSPOSE ? NR - 1 : 0;       // round executed first
  constexpr int kS00 = kR0 * EL;
  constexpr int kW0 = round_width(kR0, EL, L);
  auto fetch = [&](int it, TIn (&raw)[E]) {
    const int row = (blockIdx.y * rows_per_slot + it) * P::SLOTS + slot;
    if (row < M) {
      const TIn* src = in + static_cast<size_t>(row) * dim + static_cast<size_t>(blk) * B;
      if constexpr (kS00 == 0) {
        const Pack<TIn, E> pk = *reinterpret_cast<const Pack<TIn, E>*>(src + t * E);
#pragma unroll
        for (int j = 0; j < E; ++j) raw[j] = pk.v[j];
      } else {
#pragma unroll
        for (int j = 0; j < E; ++j) raw[j] = src[elem_index<E>(t, j, kS00, kW0)];
      }
    } else {
#pragma unroll
      for (int j = 0; j < E; ++j) raw[j] = TIn(0);
    }
  };
  TIn raw[E];
  fetch(0, raw);

  // (cos, sin) of every pair this thread touches, stage-major.  Rounds are
  // loaded in execution order; when they would not all fit in registers
  // next to the data (b = 8192 at 1024 threads), the last ones are loaded
  // once the first round has released its registers.
  float2 cf[L][E / 2];
  // pairs of stage s of this block: blk_off + s * kStageStride + pair
  constexpr int kStageStride = (B << SUB_) / 2;
  const size_t blk_off =
      SUB_ == 0 ? static_cast<size_t>(blk) * L * (B / 2)
                : static_cast<size_t>(blk >> SUB_) * (L + SUB_) * kStageStride +
                      static_cast<size_t>(blk & ((1 << SUB_) - 1)) * (B / 2);
  constexpr int kEarly = (L * E) > 96 ? 3 : NR;   // rounds loaded up front
  // f(s, p, c): pair p of stage s of this thread has coefficient index c.
  auto for_round = [&](int q, auto&& f) {
    const int r = TRANSPOSE ? NR - 1 - q : q;
    const int s0 = r * EL;
    const int R = round_width(r, EL, L);
#pragma unroll
    for (int k = 0; k < EL; ++k) {
      if (k < R) {
        const int s = s0 + k;
#pragma unroll
        for (int p = 0; p < E / 2; ++p) {
          const int i = elem_index<E>(t, insert_zero_bit(p, k), s0, R);
          f(s, p, s * kStageStride + delete_bit(i, s));
        }
      }
    }
  };
  // int8 codes: all of them stay in registers (one per pair).  The table
  // lookups happen once up front when every pair fits in registers, else
  // round by round just before each round runs.
  constexpr bool kLookupOnce = kEarly == NR;
  int qc[Q8 ? L : 1][E / 2];
  if constexpr (Q8) {
    const int8_t* qb = codes + blk_off;
#pragma unroll
    for (int q = 0; q < NR; ++q)
      for_round(q, [&](int s, int p, int c) { qc[s][p] = qb[c]; });
    for (int i = tid; i < 256; i += P::THREADS) {
      float sn, cn;
      sincosf(fmaf(static_cast<float>(i - 128), step, 0.785398163397448310f), &sn, &cn);
      table[i] = make_float2(cn, sn);
    }
    __syncthreads();
    if constexpr (kLookupOnce) {
#pragma unroll
      for (int q = 0; q < NR; ++q)
        for_round(q, [&](int s, int p, int) { cf[s][p] = table[qc[s][p] + 128]; });
    }
  } else if constexpr (kCoefLds) {
    // the block's L x B/2 pairs, fetched once per workgroup with coalesced
    // 16-byte loads into LDS behind the slots' exchange rows; every slot
    // then picks its own pairs from there
    float2* csl = reinterpret_cast<float2*>(lds + P::SLOTS * B);
    const float4* src = reinterpret_cast<const float4*>(cs + blk_off);
    float4* dst = reinterpret_cast<float4*>(csl);
    for (int i = tid; i < L * B / 4; i += P::THREADS) dst[i] = src[i];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kEarly; ++q)
      for_round(q, [&](int s, int p, int c) { cf[s][p] = csl[c]; });
  } else {
    const float2* csb = cs + blk_off;
#pragma unroll
    for (int q = 0; q < kEarly; ++q)
      for_round(q, [&](int s, int p, int c) { cf[s][p] = csb[c]; });
  }
  static_assert(!kCoefLds || kEarly == NR, "LDS-staged pairs are all loaded up front");
  constexpr bool kPrefetchRow = Q8 || kEarly == NR;
  auto load_round = [&](int q) {
    const float2* csb = cs + blk_off;
    for_round(q, [&](int s, int p, int c) { cf[s][p] = csb[c]; });
  };
  // the E sign bits of this thread's contiguous elements t*E .. t*E+E-1
  const int g0 = blk * B + t * E;
  const uint32_t sbits = sign[g0 >> 5] >> (g0 & 31);

  for (int it = 0; it < rows_per_slot; ++it) {
    const int row = (blockIdx.y * rows_per_slot + it) * P::SLOTS + slot;
    const bool active = row < M;
    const size_t base = static_cast<size_t>(active ? row : 0) * dim +
                        static_cast<size_t>(blk) * B;
    if (NR > 1 && it > 0) slot_sync<kWaveLocal>();   // LDS reuse across rows
    if (!kPrefetchRow && it > 0) fetch(it, raw);
    float v[E];
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const int r = TRANSPOSE ? NR - 1 - q : q;
      const int s0 = r * EL;
      const int R = round_width(r, EL, L);
      if constexpr (Q8 && !kLookupOnce) {
        for_round(q, [&](int s, int p, int) { cf[s][p] = table[qc[s][p] + 128]; });
      } else if (!Q8 && q == 1 && it == 0) {
#pragma unroll
        for (int ql = kEarly; ql < NR; ++ql) load_round(ql);
      }
      if (q == 0) {
#pragma unroll
        for (int j = 0; j < E; ++j) v[j] = to_f32(raw[j]);
        if (!TRANSPOSE && s0 == 0) {
#pragma unroll
          for (int j = 0; j < E; ++j) v[j] = flip_sign(v[j], (sbits >> j) & 1u);
        }
        // the next row's input is in flight during this row's rounds, unless
        // the float32 pairs already fill the registers (b = 8192)
        if (kPrefetchRow && it + 1 < rows_per_slot) fetch(it + 1, raw);
      } else {
#pragma unroll
        for (int j = 0; j < E; ++j) v[j] = u[elem_index<E>(t, j, s0, R)];
      }
      // stages of this round, ascending for F, descending for F^T
#pragma unroll
      for (int kk = 0; kk < EL; ++kk) {
        const int k = TRANSPOSE ? EL - 1 - kk : kk;
        if (k < R) {
          const int s = s0 + k;
#pragma unroll
          for (int p = 0; p < E / 2; ++p) {
            const int j = insert_zero_bit(p, k);
            const int j2 = j | (1 << k);
            const float a = v[j];
            const float b = v[j2];
            const float c = cf[s][p].x;
            const float sn = cf[s][p].y;
            v[j] = fmaf(c, a, sn * b);
            v[j2] = fmaf(sn, a, -(c * b));
          }
        }
      }
      if (q == NR - 1) {
        if (s0 == 0) {
          if (TRANSPOSE) {
#pragma unroll
            for (int j = 0; j < E; ++j) v[j] = flip_sign(v[j], (sbits >> j) & 1u);
          }
          if (active) store_contig<TOut, E>(out + base + t * E, v);
        } else if (active) {
#pragma unroll
          for (int j = 0; j < E; ++j)
            from_f32(out[base + elem_index<E>(t, j, s0, R)], v[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < E; ++j) u[elem_index<E>(t, j, s0, R)] = v[j];
        slot_sync<kWaveLocal>();
      }
    }
  }
}

// Output rotation of a few rows with the block split over eight
// workgroups.  F^T applies the stages in descending order: the first three
// (strides B/2, B/4, B/8) mix the eight elements q + j B/8 (j = 0..7) of
// each residue q < B/8, and every later stage stays inside one of the eight
// sub-blocks [w B/8, (w + 1) B/8).  Workgroup w therefore reads the whole
// row (its sub-block depends on all of it), applies to every residue only
// the seven first-three-stage butterflies that lead to element j = w (all
// four of the widest stage, the two of the next on the half holding w, the
// one of the third), keeps that element in LDS, and finishes its sub-block
// alone with the register rounds of rotate_kernel.  Its coefficient reads
// are those seven pairs per residue and its own sub-block's share of the
// other stages, about a quarter of the block's, and the eight workgroups
// run on eight CUs instead of one CU reading all of them.
constexpr int kSplitParts = 8;
constexpr int kSplitThreads = 512;
// Rows up to this count take the split form: each row is one grid row of
// eight workgroups, so the form holds for any M; past 64 rows the block
// kernel's shared coefficient registers read less and win.
constexpr int kSplitMaxM = 64;

// a where mask bits are set, else b.  The mask comes through an empty asm
// so that the selects between register elements stay selects (the compiler
// would otherwise fold them into one runtime-indexed array access, which it
// places in LDS).
__device__ __forceinline__ float bit_select(uint32_t mask, float a, float b) {
  return __uint_as_float((mask & __float_as_uint(a)) | (~mask & __float_as_uint(b)));
}

__device__ __forceinline__ uint32_t mask_of(bool c) {
  uint32_t m = c ? 0xffffffffu : 0u;
  asm volatile("" : "+v"(m));
  return m;
}

__device__ __forceinline__ void butterfly(float& a, float& b, float2 cs) {
  const float x = a;
  const float y = b;
  a = fmaf(cs.x, x, cs.y * y);
  b = fmaf(cs.y, x, -(cs.x * y));
}

template <int LOGB, bool Q8, typename TOut>
__global__ __launch_bounds__(kSplitThreads) void rotate_out_split_kernel(
    const float* __restrict__ in, TOut* __restrict__ out, const float2* __restrict__ cs,
    const int8_t* __restrict__ codes, float step, const uint32_t* __restrict__ sign, int dim) {
  constexpr int B = 1 << LOGB;
  constexpr int BB = B / kSplitParts;           // sub-block
  constexpr int LB = LOGB - 3;                  // stages inside a sub-block
  constexpr int QPT = BB / kSplitThreads;       // residues per thread
  constexpr int E = 8;
  constexpr int TB = BB / E;                    // threads of the sub-block rounds
  constexpr int NRB = (LB + 2) / 3;             // their register rounds
  static_assert(QPT >= 1 && BB % kSplitThreads == 0, "sub-blocks of 512 or more");
  __shared__ float u[BB];
  __shared__ float2 table[Q8 ? 256 : 1];        // (cos t, sin t) by code + 128

  const int tid = threadIdx.x;
  const int w = blockIdx.x % kSplitParts;
  const int blk = blockIdx.x / kSplitParts;
  const size_t row = blockIdx.y;
  const float* src = in + row * dim + static_cast<size_t>(blk) * B;
  const size_t coff = static_cast<size_t>(blk) * LOGB * (B / 2);
  // A coefficient is fetched as a handle (the float32 pair, or the int8
  // code) and resolved once the code table exists.
  using Handle = typename std::conditional<Q8, int, float2>::type;
  auto fetch = [&](int c) -> Handle {
    if constexpr (Q8) return codes[coff + c];
    else return cs[coff + c];
  };
  auto resolve = [&](Handle h) -> float2 {
    if constexpr (Q8) return table[h + 128];
    else return h;
  };
  auto cidx = [&](int sg, int i) { return sg * (B / 2) + delete_bit(i, sg); };

  // loads first: the sub-block rounds' coefficients, the row, the seven
  // pairs per residue
  Handle hb[LB][E / 2];
  if (tid < TB) {
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const int s0 = 3 * r;
      const int R = round_width(r, 3, LB);
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        if (k < R) {
#pragma unroll
          for (int p = 0; p < E / 2; ++p) {
            const int i = w * BB + elem_index<E>(tid, insert_zero_bit(p, k), s0, R);
            hb[s0 + k][p] = fetch(cidx(s0 + k, i));
          }
        }
      }
    }
  }
  const int half = w & 4;                       // elements j of the half holding w
  float x[QPT][E];
  Handle h2[QPT][4], h1[QPT][2], h0[QPT];
#pragma unroll
  for (int qi = 0; qi < QPT; ++qi) {
    const int q = tid + qi * kSplitThreads;
#pragma unroll
    for (int j = 0; j < E; ++j) x[qi][j] = src[q + BB * j];
#pragma unroll
    for (int p = 0; p < 4; ++p) h2[qi][p] = fetch(cidx(LB + 2, q + BB * p));
#pragma unroll
    for (int m = 0; m < 2; ++m) h1[qi][m] = fetch(cidx(LB + 1, q + BB * (half + m)));
    h0[qi] = fetch(cidx(LB, q + BB * (w & 6)));
  }
  if constexpr (Q8) {
    for (int i = tid; i < 256; i += kSplitThreads) {
      float sn, cn;
      sincosf(fmaf(static_cast<float>(i - 128), step, 0.785398163397448310f), &sn, &cn);
      table[i] = make_float2(cn, sn);
    }
    __syncthreads();
  }

  const uint32_t m4 = mask_of(w & 4), m2 = mask_of(w & 2), m1 = mask_of(w & 1);
#pragma unroll
  for (int qi = 0; qi < QPT; ++qi) {
    const int q = tid + qi * kSplitThreads;
    float* v = x[qi];
#pragma unroll
    for (int p = 0; p < 4; ++p) butterfly(v[p], v[p | 4], resolve(h2[qi][p]));   // stride B/2
    float y[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) y[m] = bit_select(m4, v[4 + m], v[m]);
    butterfly(y[0], y[2], resolve(h1[qi][0]));                                     // stride B/4
    butterfly(y[1], y[3], resolve(h1[qi][1]));
    float z0 = bit_select(m2, y[2], y[0]);
    float z1 = bit_select(m2, y[3], y[1]);
    butterfly(z0, z1, resolve(h0[qi]));                                            // stride B/8
    u[q] = bit_select(m1, z1, z0);
  }
  __syncthreads();

  // the sub-block's stages LB-1 .. 0
#pragma unroll
  for (int qq = 0; qq < NRB; ++qq) {
    const int r = NRB - 1 - qq;
    const int s0 = 3 * r;
    const int R = round_width(r, 3, LB);
    if (tid < TB) {
      float v[E];
#pragma unroll
      for (int j = 0; j < E; ++j) v[j] = u[elem_index<E>(tid, j, s0, R)];
#pragma unroll
      for (int kk = 0; kk < 3; ++kk) {
        const int k = 2 - kk;
        if (k < R) {
#pragma unroll
          for (int p = 0; p < E / 2; ++p) {
            const int j = insert_zero_bit(p, k);
            butterfly(v[j], v[j | (1 << k)], resolve(hb[s0 + k][p]));
          }
        }
      }
      if (r == 0) {   // contiguous elements 8 tid .. 8 tid + 7: signs, store
        const int g = blk * B + w * BB + tid * E;
        const uint32_t sbits = sign[g >> 5] >> (g & 31);
#pragma unroll
        for (int j = 0; j < E; ++j) v[j] = flip_sign(v[j], (sbits >> j) & 1u);
        store_contig<TOut, E>(out + row * dim + static_cast<size_t>(g), v);
      } else {
#pragma unroll
        for (int j = 0; j < E; ++j) u[elem_index<E>(tid, j, s0, R)] = v[j];
      }
    }
    if (r > 0) __syncthreads();
  }
}

template <int LOGB, bool Q8, typename TOut>
hipError_t launch_split(const harp_rotation& R, const void* in, void* out, int M,
                        hipStream_t stream) {
  const int nblk = R.dim >> LOGB;
  const dim3 grid(nblk * kSplitParts, M);
  hipLaunchKernelGGL((rotate_out_split_kernel<LOGB, Q8, TOut>), grid, dim3(kSplitThreads), 0,
                     stream, static_cast<const float*>(in), static_cast<TOut*>(out),
                     reinterpret_cast<const float2*>(R.cs), R.phi_codes, R.phi_step,
                     R.sign_bits, R.dim);
  return hipGetLastError();
}

template <int LOGB, int EL_, bool TRANSPOSE, bool Q8, typename TIn, typename TOut, int SUB_ = 0>
hipError_t launch_typed(const harp_rotation& R, const void* in, void* out, int M,
                        hipStream_t stream) {
  using P = Plan<LOGB, EL_>;
  const int nblk = R.dim >> LOGB;
  const int ygroups = (M + P::SLOTS - 1) / P::SLOTS;
  // Rows per slot: about one workgroup per CU; beyond that, a workgroup
  // reuses its coefficient registers over several rows.  Blocks of 256 or
  // fewer fetch their pairs (at most 8 KB) once per workgroup into LDS, so
  // they aim at about four workgroups per CU instead.
  int rps = (nblk * ygroups) / 256;
  if (rps < 1) rps = 1;
  if (rps > 8) rps = 8;
  if (LOGB <= 8) { rps = (nblk * ygroups) / 1024; if (rps < 1) rps = 1; }
  const int need = (ygroups + 65534) / 65535;
  if (rps < need) rps = need;
  const dim3 grid(nblk, (ygroups + rps - 1) / rps);
  size_t shmem = P::NR > 1 ? sizeof(float) * P::SLOTS * P::B : 0;
  if (P::NR > 1 && P::TPB <= kWave && !Q8 && SUB_ == 0)
    shmem += sizeof(float2) * P::L * (P::B / 2);
  hipLaunchKernelGGL((rotate_kernel<LOGB, EL_, TRANSPOSE, Q8, TIn, TOut, SUB_>), grid,
                     dim3(P::THREADS), shmem, stream,
                     static_cast<const TIn*>(in), static_cast<TOut*>(out),
                     reinterpret_cast<const float2*>(R.cs), R.phi_codes,
                     R.phi_step, R.sign_bits, R.dim, M, rps);
  return hipGetLastError();
}


// Input rotation of a few rows at b = 4096 / 8192 in two launches: the first
// LOGB - 3 stages never leave a sub-block of b/8 elements, so eight
// workgroups per block run them (the block kernel on sub-blocks, the sign
// flip included) into the float32 output; then this kernel applies the last
// three stages (strides b/8, b/4, b/2) in place: residue q < b/8 owns the
// eight elements q + (b/8) j, and stage LOGB - 3 + k pairs j with j ^ 2^k.
// Each block's pairs are then read by a few workgroups instead of all
// passing through one CU.
constexpr int kTailThreads = 256;

// The last three stages of residue q of block blk on the eight elements v[j]
// = element q + (b/8) j (tab: the int8 angle table when Q8).
template <int LOGB, bool Q8>
__device__ __forceinline__ void tail_stages(float (&v)[8], int q, int blk,
                                            const float2* __restrict__ cs,
                                            const int8_t* __restrict__ codes,
                                            const float2* tab) {
  constexpr int B = 1 << LOGB;
  constexpr int L = LOGB;
  constexpr int SB = B / 8;
  const size_t coff = static_cast<size_t>(blk) * L * (B / 2);
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int s = L - 3 + k;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int j = insert_zero_bit(p, k);
      const int j2 = j | (1 << k);
      const size_t c = coff + static_cast<size_t>(s) * (B / 2) + delete_bit(q + SB * j, s);
      float2 t;
      if constexpr (Q8) t = tab[codes[c] + 128];
      else t = cs[c];
      const float a = v[j];
      const float b = v[j2];
      v[j] = fmaf(t.x, a, t.y * b);
      v[j2] = fmaf(t.y, a, -(t.x * b));
    }
  }
}

template <int LOGB, bool Q8>
__device__ __forceinline__ void tail_table(float2* table, float step) {
  if constexpr (Q8) {
    float sn, cn;
    sincosf(fmaf(static_cast<float>(static_cast<int>(threadIdx.x) - 128), step,
                 0.785398163397448310f), &sn, &cn);
    table[threadIdx.x] = make_float2(cn, sn);
    __syncthreads();
  }
}

template <int LOGB, bool Q8, typename TOut>
__global__ __launch_bounds__(kTailThreads) void rotate_in_tail_kernel(
    const float* src, TOut* dst, const float2* __restrict__ cs,
    const int8_t* __restrict__ codes, float step, int dim) {
  constexpr int B = 1 << LOGB;
  constexpr int SB = B / 8;
  constexpr int kParts = SB / kTailThreads;   // workgroups per block row
  static_assert(kParts >= 1 && SB % kTailThreads == 0, "sub-blocks of 256 or more");
  __shared__ float2 table[Q8 ? 256 : 1];
  tail_table<LOGB, Q8>(table, step);
  const int blk = blockIdx.x / kParts;
  const int q = (blockIdx.x - blk * kParts) * kTailThreads + threadIdx.x;
  // src and dst may be the same float32 rows: each thread reads its eight
  // elements before it writes them
  const size_t e0 = static_cast<size_t>(blockIdx.y) * dim + static_cast<size_t>(blk) * B + q;
  const float* sb = src + e0;
  TOut* db = dst + e0;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = sb[j * SB];
  tail_stages<LOGB, Q8>(v, q, blk, cs, codes, table);
#pragma unroll
  for (int j = 0; j < 8; ++j) from_f32(db[j * SB], v[j]);
}

// The same last three stages for one row, finished into the planes of the
// one-row FP4 matrix-core product (f4_planes.hpp) instead of float32 x~: a
// workgroup's residues q0 .. q0 + 255 hold, for j = 0..7, the 256
// consecutive inputs blk b + (b/8) j + q0 .. +255, i.e. one pair of product
// steps each.  Its first four waves apply the stages and leave the values
// in LDS; then each of its sixteen waves builds and writes one step.
constexpr int kTailF4Threads = 16 * kWave;

template <int LOGB, bool Q8>
__global__ __launch_bounds__(kTailF4Threads) void rotate_in_tail_f4_kernel(
    const float* src, const float2* __restrict__ cs, const int8_t* __restrict__ codes,
    float step, u32x4* __restrict__ pl, uint32_t* __restrict__ psc, float* __restrict__ gsx) {
  constexpr int B = 1 << LOGB;
  constexpr int SB = B / 8;
  constexpr int kParts = SB / kTailThreads;
  static_assert(kParts >= 1 && SB % kTailThreads == 0 && kTailThreads == 256,
                "sub-blocks of 256 or more, one step pair per residue span");
  __shared__ float2 table[Q8 ? 256 : 1];
  __shared__ float xl[8][kTailThreads];
  __shared__ __attribute__((aligned(16))) uint8_t stage[16][f4::kStepLds + kWave];
  __shared__ float ssx[16][4];
  const int blk = blockIdx.x / kParts;
  const int part = blockIdx.x - blk * kParts;
  if constexpr (Q8) {
    if (threadIdx.x < 256) {
      float sn, cn;
      sincosf(fmaf(static_cast<float>(static_cast<int>(threadIdx.x) - 128), step,
                   0.785398163397448310f), &sn, &cn);
      table[threadIdx.x] = make_float2(cn, sn);
    }
    __syncthreads();
  }
  if (threadIdx.x < kTailThreads) {
    const int q = part * kTailThreads + threadIdx.x;
    const float* sb = src + static_cast<size_t>(blk) * B + q;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = sb[j * SB];
    tail_stages<LOGB, Q8>(v, q, blk, cs, codes, table);
#pragma unroll
    for (int j = 0; j < 8; ++j) xl[j][threadIdx.x] = v[j];
  }
  __syncthreads();
  const int w = threadIdx.x >> 6;   // step w of the sixteen
  const int lane = threadIdx.x & (kWave - 1);
  const int j = w >> 1;
  const int e = w & 1;
  const int s = 2 * ((blk * B + SB * j + kTailThreads * part) / 256) + e;
  f4::build_step(&xl[j][64 * e], stage[w], stage[w] + f4::kStepLds, ssx[w], lane);
  f4::emit_step(stage[w], ssx[w], s, pl, psc, gsx, lane);
}

// x~ = F x for one row at b = 256, finished into the planes of the one-row
// FP4 matrix-core product (f4_planes.hpp) instead of float32 x~: one
// workgroup per block, which is one pair of product steps.  The sign flip
// and the eight stages run in LDS (thread t < 128 takes pair t of each
// stage; its eight coefficients are requested first), then two waves build
// the block's two steps.
template <bool Q8, typename TIn>
__global__ __launch_bounds__(256) void rotate_in_b256_f4_kernel(
    const TIn* __restrict__ x, const float2* __restrict__ cs, const int8_t* __restrict__ codes,
    float step, const uint32_t* __restrict__ sign, u32x4* __restrict__ pl,
    uint32_t* __restrict__ psc, float* __restrict__ gsx) {
  constexpr int B = 256;
  constexpr int L = 8;
  __shared__ float2 table[Q8 ? 256 : 1];
  __shared__ float xl[B];
  __shared__ __attribute__((aligned(16))) uint8_t stage[2][f4::kStepLds + kWave];
  __shared__ float ssx[2][4];
  const int blk = blockIdx.x;
  const int t = threadIdx.x;
  if constexpr (Q8) {
    float sn, cn;
    sincosf(fmaf(static_cast<float>(t - 128), step, 0.785398163397448310f), &sn, &cn);
    table[t] = make_float2(cn, sn);
  }
  const int g = blk * B + t;
  const size_t coff = static_cast<size_t>(blk) * L * (B / 2);
  float2 c[L];
  int8_t qc[L];
  if (t < B / 2) {
#pragma unroll
    for (int st = 0; st < L; ++st) {
      if constexpr (Q8) qc[st] = codes[coff + st * (B / 2) + t];
      else c[st] = cs[coff + st * (B / 2) + t];
    }
  }
  xl[t] = flip_sign(to_f32(x[g]), (sign[g >> 5] >> (g & 31)) & 1u);
  __syncthreads();
#pragma unroll
  for (int st = 0; st < L; ++st) {
    if (t < B / 2) {
      float2 cf;
      if constexpr (Q8) cf = table[qc[st] + 128];
      else cf = c[st];
      const int i = insert_zero_bit(t, st);
      const int i2 = i | (1 << st);
      const float a = xl[i];
      const float b = xl[i2];
      xl[i] = fmaf(cf.x, a, cf.y * b);
      xl[i2] = fmaf(cf.y, a, -(cf.x * b));
    }
    __syncthreads();
  }
  if (t < 2 * kWave) {
    const int w = t >> 6;
    const int lane = t & (kWave - 1);
    f4::build_step(&xl[64 * w], stage[w], stage[w] + f4::kStepLds, ssx[w], lane);
    f4::emit_step(stage[w], ssx[w], 2 * blk + w, pl, psc, gsx, lane);
  }
}

// The first launch writes the float32 intermediate to scratch (M x dim
// floats); the second writes the output (in place when out is scratch).
template <int LOGB, bool Q8, typename TIn, typename TOut>
hipError_t launch_in_split(const harp_rotation& R, const void* in, float* scratch, TOut* out,
                           int M, hipStream_t stream) {
  hipError_t e = launch_typed<LOGB - 3, 3, false, Q8, TIn, float, 3>(R, in, scratch, M, stream);
  if (e != hipSuccess) return e;
  const int nblk = R.dim >> LOGB;
  const dim3 grid(nblk * ((1 << LOGB) / 8 / kTailThreads), M);
  hipLaunchKernelGGL((rotate_in_tail_kernel<LOGB, Q8, TOut>), grid, dim3(kTailThreads), 0,
                     stream, scratch, out, reinterpret_cast<const float2*>(R.cs), R.phi_codes,
                     R.phi_step, R.dim);
  return hipGetLastError();
}

template <int LOGB, typename TOut>
hipError_t launch_in_split_any(const harp_rotation& R, const void* in, int in_dt,
                               float* scratch, TOut* out, int M, hipStream_t stream) {
  const bool ib = in_dt == HARP_BF16;
  if (R.phi_codes != nullptr)
    return ib ? launch_in_split<LOGB, true, uint16_t, TOut>(R, in, scratch, out, M, stream)
              : launch_in_split<LOGB, true, float, TOut>(R, in, scratch, out, M, stream);
  return ib ? launch_in_split<LOGB, false, uint16_t, TOut>(R, in, scratch, out, M, stream)
            : launch_in_split<LOGB, false, float, TOut>(R, in, scratch, out, M, stream);
}

template <int LOGB, bool Q8, typename TIn>
hipError_t launch_in_split_f4(const harp_rotation& R, const void* in, float* scratch,
                              uint8_t* f4r, hipStream_t stream) {
  hipError_t e = launch_typed<LOGB - 3, 3, false, Q8, TIn, float, 3>(R, in, scratch, 1, stream);
  if (e != hipSuccess) return e;
  const int nblk = R.dim >> LOGB;
  const dim3 grid(nblk * ((1 << LOGB) / 8 / kTailThreads), 1);
  hipLaunchKernelGGL((rotate_in_tail_f4_kernel<LOGB, Q8>), grid, dim3(kTailF4Threads), 0, stream,
                     scratch, reinterpret_cast<const float2*>(R.cs), R.phi_codes, R.phi_step,
                     reinterpret_cast<u32x4*>(f4r),
                     reinterpret_cast<uint32_t*>(f4r + f4_psc_offset(R.dim)),
                     reinterpret_cast<float*>(f4r + f4_sx_offset(R.dim)));
  return hipGetLastError();
}

template <int LOGB>
hipError_t launch_in_split_f4_any(const harp_rotation& R, const void* in, int in_dt,
                                  float* scratch, uint8_t* f4r, hipStream_t stream) {
  const bool ib = in_dt == HARP_BF16;
  if (R.phi_codes != nullptr)
    return ib ? launch_in_split_f4<LOGB, true, uint16_t>(R, in, scratch, f4r, stream)
              : launch_in_split_f4<LOGB, true, float>(R, in, scratch, f4r, stream);
  return ib ? launch_in_split_f4<LOGB, false, uint16_t>(R, in, scratch, f4r, stream)
            : launch_in_split_f4<LOGB, false, float>(R, in, scratch, f4r, stream);
}

template <int LOGB, int EL_, bool Q8>
hipError_t launch_q(const harp_rotation& R, const void* in, int in_dt,
                    void* out, int out_dt, int M, bool transpose,
                    hipStream_t stream) {
  const bool ib = in_dt == HARP_BF16;
  const bool ob = out_dt == HARP_BF16;
  if (transpose) {   // y' is always float32
    if (ob) return launch_typed<LOGB, EL_, true, Q8, float, uint16_t>(R, in, out, M, stream);
    return launch_typed<LOGB, EL_, true, Q8, float, float>(R, in, out, M, stream);
  }
  if (ib && ob)
    return launch_typed<LOGB, EL_, false, Q8, uint16_t, uint16_t>(R, in, out, M, stream);
  if (ib) return launch_typed<LOGB, EL_, false, Q8, uint16_t, float>(R, in, out, M, stream);
  if (ob) return launch_typed<LOGB, EL_, false, Q8, float, uint16_t>(R, in, out, M, stream);
  return launch_typed<LOGB, EL_, false, Q8, float, float>(R, in, out, M, stream);
}

template <int LOGB, int EL_>
hipError_t launch_el(const harp_rotation& R, const void* in, int in_dt,
                     void* out, int out_dt, int M, bool transpose,
                     hipStream_t stream) {
  if (R.phi_codes != nullptr)
    return launch_q<LOGB, EL_, true>(R, in, in_dt, out, out_dt, M, transpose, stream);
  return launch_q<LOGB, EL_, false>(R, in, in_dt, out, out_dt, M, transpose, stream);
}

template <int LOGB>
hipError_t launch_logb(const harp_rotation& R, const void* in, int in_dt,
                       void* out, int out_dt, int M, bool transpose,
                       hipStream_t stream) {
  if constexpr (LOGB == 12 || LOGB == 13) {
    // few rows of the input rotation into float32: two launches (above)
    if (!transpose && out_dt == HARP_F32 && M <= kSplitMaxM) {
      float* o = static_cast<float*>(out);
      return launch_in_split_any<LOGB, float>(R, in, in_dt, o, o, M, stream);
    }
    // few rows of the output rotation: eight workgroups per block
    if (transpose && M <= kSplitMaxM) {
      const bool ob = out_dt == HARP_BF16;
      if (R.phi_codes != nullptr)
        return ob ? launch_split<LOGB, true, uint16_t>(R, in, out, M, stream)
                  : launch_split<LOGB, true, float>(R, in, out, M, stream);
      return ob ? launch_split<LOGB, false, uint16_t>(R, in, out, M, stream)
                : launch_split<LOGB, false, float>(R, in, out, M, stream);
    }
  }
  if constexpr (LOGB == 12) {
    // few b = 4096 blocks in flight: 1024 threads per block (see Plan)
    if ((R.dim >> LOGB) * M <= 64)
      return launch_el<LOGB, 2>(R, in, in_dt, out, out_dt, M, transpose, stream);
  }
  return launch_el<LOGB, (LOGB < 3 ? LOGB : 3)>(R, in, in_dt, out, out_dt, M,
                                                 transpose, stream);
}

}  // namespace

hipError_t launch_rotate_in_scratch(const harp_rotation& R, const void* in, int in_dt,
                                    uint16_t* out, float* scratch, int M,
                                    hipStream_t stream) {
  if (M <= kSplitMaxM) {
    if (R.block == 4096)
      return launch_in_split_any<12, uint16_t>(R, in, in_dt, scratch, out, M, stream);
    if (R.block == 8192)
      return launch_in_split_any<13, uint16_t>(R, in, in_dt, scratch, out, M, stream);
  }
  return launch_rotate(R, in, in_dt, out, HARP_BF16, M, false, stream);
}

bool rotate_in_f4_supported(const harp_rotation& R, int M) {
  return M == 1 && (R.block == 256 || R.block == 4096 || R.block == 8192);
}

hipError_t launch_rotate_in_f4(const harp_rotation& R, const void* in, int in_dt,
                               float* scratch, uint8_t* f4r, hipStream_t stream) {
  if (R.block == 256) {
    u32x4* pl = reinterpret_cast<u32x4*>(f4r);
    uint32_t* psc = reinterpret_cast<uint32_t*>(f4r + f4_psc_offset(R.dim));
    float* sx = reinterpret_cast<float*>(f4r + f4_sx_offset(R.dim));
    const float2* cs = reinterpret_cast<const float2*>(R.cs);
    const dim3 grid(R.dim / 256);
    const bool ib = in_dt == HARP_BF16;
    if (R.phi_codes != nullptr) {
      if (ib)
        hipLaunchKernelGGL((rotate_in_b256_f4_kernel<true, uint16_t>), grid, dim3(256), 0,
                           stream, static_cast<const uint16_t*>(in), cs, R.phi_codes,
                           R.phi_step, R.sign_bits, pl, psc, sx);
      else
        hipLaunchKernelGGL((rotate_in_b256_f4_kernel<true, float>), grid, dim3(256), 0, stream,
                           static_cast<const float*>(in), cs, R.phi_codes, R.phi_step,
                           R.sign_bits, pl, psc, sx);
    } else if (ib) {
      hipLaunchKernelGGL((rotate_in_b256_f4_kernel<false, uint16_t>), grid, dim3(256), 0,
                         stream, static_cast<const uint16_t*>(in), cs, R.phi_codes, R.phi_step,
                         R.sign_bits, pl, psc, sx);
    } else {
      hipLaunchKernelGGL((rotate_in_b256_f4_kernel<false, float>), grid, dim3(256), 0, stream,
                         static_cast<const float*>(in), cs, R.phi_codes, R.phi_step,
                         R.sign_bits, pl, psc, sx);
    }
    return hipGetLastError();
  }
  if (R.block == 4096) return launch_in_split_f4_any<12>(R, in, in_dt, scratch, f4r, stream);
  if (R.block == 8192) return launch_in_split_f4_any<13>(R, in, in_dt, scratch, f4r, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_rotate(const harp_rotation& R, const void* in, int in_dt,
                         void* out, int out_dt, int M, bool transpose,
                         hipStream_t stream) {
  switch (__builtin_ctz(static_cast<unsigned>(R.block))) {
    case 1: return launch_logb<1>(R, in, in_dt, out, out_dt, M, transpose, stream);
    case 2: return launch_logb<2>(R, in, in_dt, out, out_dt, M, transpose, stream);
    case 3: return launch_logb<3>(R, in, in_dt, out, out_dt, M, transpose, stream);
    case 4: return launch_logb<4>(R, in, in_dt, out, out_dt, M, transpose, stream);
    case 5: return launch_logb<5>(R, in, in_dt, out, out_dt, M, transpose, stream);
    case 6: return launch_logb<6>(R, in, in_dt, out, out_dt, M, transpose, stream);
    case 7: return launch_logb<7>(R, in, in_dt, out, out_dt, M, transpose, stream);
    case 8: return launch_logb<8>(R, in, in_dt, out, out_dt, M, transpose, stream);
    case 9: return launch_logb<9>(R, in, in_dt, out, out_dt, M, transpose, stream);
    case 10: return launch_logb<10>(R, in, in_dt, out, out_dt, M, transpose, stream);
    case 11: return launch_logb<11>(R, in, in_dt, out, out_dt, M, transpose, stream);
    case 12: return launch_logb<12>(R, in, in_dt, out, out_dt, M, transpose, stream);
    case 13: return launch_logb<13>(R, in, in_dt, out, out_dt, M, transpose, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace harp
