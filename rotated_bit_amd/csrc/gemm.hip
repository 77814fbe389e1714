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

constexpr int kThreads = 512;   // 8 waves: 4 output quadrants x 2 k-halves

// Weight codes one thread loads per K step: 16 (a quarter of the group) for
// 2- and 4-bit codes (one / two words, so all 512 threads load); 32 for
// 3-bit codes, whose 32-code runs span three words (256 threads load).
template <int BITS> struct BSplit;
template <> struct BSplit<2> { static constexpr int CODES = 16, WORDS = 1, LOADERS = 512; };
template <> struct BSplit<4> { static constexpr int CODES = 16, WORDS = 2, LOADERS = 512; };
template <> struct BSplit<3> { static constexpr int CODES = 32, WORDS = 3, LOADERS = 256; };

// Global operands of one K step, held in registers between the load and
// the LDS store (the software-pipelined prefetch).
template <int BITS>
struct StepRegs {
  u32x4 a[2];                        // 8 bf16 of x~ rows ar and ar + 64
  uint32_t w[BSplit<BITS>::WORDS];   // this thread's codes of weight row br
};

// Scales and zeros are staged in LDS for kSzBlock groups at a time: one
// 16-byte load per row instead of a 2-byte gather per row and step.
constexpr int kSzBlock = 8;

// Row pointers are clamped to valid rows: rows past M (x~) or N (weights)
// only feed accumulators of outputs that are never stored.  x~ is read with
// eight lanes per 128-byte row segment, so each load covers whole lines.
template <int BITS>
__device__ __forceinline__ void load_step(StepRegs<BITS>& r, int kt,
                                          const uint16_t* __restrict__ arow0,
                                          const uint16_t* __restrict__ arow1,
                                          const uint32_t* __restrict__ brow) {
  using SP = BSplit<BITS>;
  r.a[0] = *reinterpret_cast<const u32x4*>(arow0 + kt * BK);
  r.a[1] = *reinterpret_cast<const u32x4*>(arow1 + kt * BK);
  const uint32_t* wp = brow + kt * 2 * BITS;
  if constexpr (SP::WORDS == 1) {
    r.w[0] = wp[0];
  } else if constexpr (SP::WORDS == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(wp);
    r.w[0] = v.x;
    r.w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < SP::WORDS; ++i) r.w[i] = wp[i];
  }
}

// kSzBlock scales (threads 0..127) or zeros (threads 128..255) of one row,
// groups g0 .. g0 + kSzBlock - 1 (entries past G are never read).
struct SzRegs { u32x4 v; };

__device__ __forceinline__ void load_sz(SzRegs& r, const uint16_t* __restrict__ row,
                                        int g0, int G, bool vec_ok) {
  if (vec_ok && g0 + kSzBlock <= G) {
    r.v = *reinterpret_cast<const u32x4*>(row + g0);
  } else {
    uint32_t h[kSzBlock / 2];
#pragma unroll
    for (int i = 0; i < kSzBlock / 2; ++i) {
      const uint32_t lo = g0 + 2 * i < G ? row[g0 + 2 * i] : 0u;
      const uint32_t hi = g0 + 2 * i + 1 < G ? row[g0 + 2 * i + 1] : 0u;
      h[i] = lo | (hi << 16);
    }
    r.v = u32x4{h[0], h[1], h[2], h[3]};
  }
}

template <int BITS>
__device__ __forceinline__ void store_step(const StepRegs<BITS>& r, uint16_t* sA,
                                           uint16_t* sB, uint16_t s16, uint16_t z16,
                                           int ar, int a8, int br, int bpart,
                                           bool b_loader) {
  using SP = BSplit<BITS>;
  *reinterpret_cast<u32x4*>(sA + ar * LDK + a8 * 8) = r.a[0];
  *reinterpret_cast<u32x4*>(sA + (ar + 64) * LDK + a8 * 8) = r.a[1];
  if (b_loader) {
    float f[SP::CODES];
    const float s = f16_to_f32(s16);
    const float nzs = -f16_to_f32(z16) * s;
    if constexpr (BITS == 3) {
      float q[32];
      codes_run32<3>(r.w, q);
#pragma unroll
      for (int j = 0; j < 32; ++j) f[j] = fmaf(q[j], s, nzs);
    } else {
      float q[16];
      codes_16<BITS>(r.w, q);
#pragma unroll
      for (int j = 0; j < 16; ++j) f[j] = fmaf(q[j], s, nzs);
    }
    u32x4* db = reinterpret_cast<u32x4*>(sB + br * LDK + bpart * SP::CODES);
#pragma unroll
    for (int i = 0; i < SP::CODES / 8; ++i) {
      const u32x4 b = {pack_bf16x2(f[8 * i + 0], f[8 * i + 1]),
                       pack_bf16x2(f[8 * i + 2], f[8 * i + 3]),
                       pack_bf16x2(f[8 * i + 4], f[8 * i + 5]),
                       pack_bf16x2(f[8 * i + 6], f[8 * i + 7])};
      db[i] = b;
    }
  }
}

// Matrix-core work of one K step for one wave: k-slices kk0, kk0 + 1 of the
// step (16 k each) on the wave's 64 x 64 quadrant.
__device__ __forceinline__ void mfma_step(const uint16_t* pa, const uint16_t* pb,
                                          int wm, int wn, int kk0, int frag_row,
                                          int frag_k, floatx16 (&acc)[2][2]) {
#pragma unroll
  for (int kq = 0; kq < 2; ++kq) {
    const int kk = kk0 + kq;
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

struct StepCtx {
  int ar, a8, br, bpart;
  bool b_loader;
  int wm, wn, kk0, frag_row, frag_k;
  bool sz_loader;        // threads 0..255 stage scales (0..127) or zeros
  bool sz_vec;           // 16-byte scale/zero loads are aligned
  int G;
  int ge;                // end (exclusive) of this K slice, in groups
};

// LDS block of scales and zeros: [buffer][scale|zero][row][group in block].
typedef uint16_t SzLds[2][2][BN][kSzBlock];

// One K step: dequantize the prefetched step into LDS stage kt & 1, then
// (after the barrier) issue the loads of step kt + 3 into the same
// registers and run the step's matrix-core work.  At the last step of a
// scale block the next block is written to LDS (made visible by this
// step's barrier) and the one after it is prefetched.
template <int BITS>
__device__ __forceinline__ void gemm_step(
    StepRegs<BITS>& r, int kt, bool prefetch, uint16_t (*sA)[BM * LDK],
    uint16_t (*sB)[BN * LDK], SzLds& szl, SzRegs& szr, const StepCtx& c,
    const uint16_t* __restrict__ arow0, const uint16_t* __restrict__ arow1,
    const uint32_t* __restrict__ brow, const uint16_t* __restrict__ szrow,
    floatx16 (&acc)[2][2]) {
  const int st = kt & 1;
  const int blk = kt / kSzBlock;
  const int gi = kt - blk * kSzBlock;
  const uint16_t s16 = szl[blk & 1][0][c.br][gi];
  const uint16_t z16 = szl[blk & 1][1][c.br][gi];
  store_step<BITS>(r, sA[st], sB[st], s16, z16, c.ar, c.a8, c.br, c.bpart, c.b_loader);
  const bool block_end = gi == kSzBlock - 1;
  if (block_end && c.sz_loader) {
    *reinterpret_cast<u32x4*>(&szl[(blk + 1) & 1][threadIdx.x >> 7][threadIdx.x & 127][0]) = szr.v;
    load_sz(szr, szrow, (blk + 2) * kSzBlock, c.G, c.sz_vec);
  }
  __syncthreads();   // stage st complete; stage st^1 no longer read
  if (prefetch) load_step<BITS>(r, min(kt + 3, c.ge - 1), arow0, arow1, brow);
  mfma_step(sA[st], sB[st], c.wm, c.wn, c.kk0, c.frag_row, c.frag_k, acc);
}

// Split K: per slice and tile one float32 partial tile in the layout the
// four output waves hold it (coalesced), and one uint32 arrival counter per
// tile (the caller places the counters at a fixed offset of its workspace).
constexpr int kTileFloats = BM * BN;

template <int BITS>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint16_t* __restrict__ zr, const uint16_t* __restrict__ xt,
    float* __restrict__ yt, int N, int K, int M, float* __restrict__ partials,
    uint32_t* __restrict__ counters) {
  using SP = BSplit<BITS>;
  // Two LDS stages: step kt is read from stage kt & 1 while step kt + 1 is
  // written to the other.  One allocation (72 KB) holds both operand
  // stages; at the end it is reused (64 KB) to combine the k-halves.
  constexpr int kStageElems = 2 * (BM + BN) * LDK;
  constexpr int kReduceFloats = 4 * 4 * 16 * kWave;
  static_assert(kStageElems * sizeof(uint16_t) >= kReduceFloats * sizeof(float),
                "LDS stage buffers must hold the k-half reduction");
  __shared__ __attribute__((aligned(16))) uint16_t smem[kStageElems];
  __shared__ __attribute__((aligned(16))) SzLds szl;
  uint16_t (*sA)[BM * LDK] = reinterpret_cast<uint16_t (*)[BM * LDK]>(smem);
  uint16_t (*sB)[BN * LDK] = reinterpret_cast<uint16_t (*)[BN * LDK]>(smem + 2 * BM * LDK);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const size_t WPR = static_cast<size_t>(K) * BITS / 32;
  const int G = K / kGroup;

  StepCtx c;
  c.G = G;
  c.wm = ((wave & 3) >> 1) * 64;
  c.wn = (wave & 1) * 64;
  c.kk0 = (wave >> 2) * 2;           // this wave's two 16-wide k-slices
  c.frag_row = lane & 31;
  c.frag_k = 8 * (lane >> 5);
  // x~ loader: rows ar and ar + 64, 16-byte segment a8 of the 128-byte row
  c.ar = tid >> 3;
  c.a8 = tid & 7;
  // weight loader: row br, part bpart (SP::CODES codes)
  constexpr int parts = kGroup / SP::CODES;
  c.b_loader = tid < SP::LOADERS;
  c.br = (tid % SP::LOADERS) / parts;
  c.bpart = (tid % SP::LOADERS) % parts;
  // scale / zero stager: row tid & 127
  c.sz_loader = tid < 2 * BN;
  c.sz_vec = (G % kSzBlock) == 0;
  const uint16_t* arow0 = xt + static_cast<size_t>(min(m0 + c.ar, M - 1)) * K + c.a8 * 8;
  const uint16_t* arow1 = xt + static_cast<size_t>(min(m0 + c.ar + 64, M - 1)) * K + c.a8 * 8;
  const int bn = min(n0 + c.br, N - 1);
  const uint32_t* brow = qw + static_cast<size_t>(bn) * WPR + c.bpart * SP::WORDS;
  const int szn = min(n0 + (tid & 127), N - 1);
  const uint16_t* szrow = ((tid >> 7) ? zr : sc) + static_cast<size_t>(szn) * G;

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // This workgroup's K slice: groups [gb, ge), boundaries multiples of the
  // scale block so 16-byte scale/zero loads stay aligned.
  const int S = gridDim.z;
  const int z = blockIdx.z;
  const int gb = (z * G / S) & ~(kSzBlock - 1);
  const int ge = (z + 1 == S) ? G : (((z + 1) * G / S) & ~(kSzBlock - 1));
  c.ge = ge;

  // Scale/zero blocks: the first to LDS now, the next in registers.
  const int b0 = gb / kSzBlock;
  SzRegs szr;
  if (c.sz_loader) {
    load_sz(szr, szrow, b0 * kSzBlock, G, c.sz_vec);
    *reinterpret_cast<u32x4*>(&szl[b0 & 1][tid >> 7][tid & 127][0]) = szr.v;
    load_sz(szr, szrow, (b0 + 1) * kSzBlock, G, c.sz_vec);
  }

  // Prefetch ring of three steps: the global loads of step k + 3 are issued
  // while step k is computed, so three steps of matrix-core work cover the
  // memory latency.  Steps past the slice end re-load its last step (valid
  // memory, unused).  Named registers (not an array) keep the ring out of
  // scratch memory.
  StepRegs<BITS> r0, r1, r2;
  load_step<BITS>(r0, gb, arow0, arow1, brow);
  load_step<BITS>(r1, min(gb + 1, ge - 1), arow0, arow1, brow);
  load_step<BITS>(r2, min(gb + 2, ge - 1), arow0, arow1, brow);
  __syncthreads();   // first scale/zero block visible
  int kt = gb;
  for (; kt + 3 <= ge; kt += 3) {
    gemm_step<BITS>(r0, kt, true, sA, sB, szl, szr, c, arow0, arow1, brow, szrow, acc);
    gemm_step<BITS>(r1, kt + 1, true, sA, sB, szl, szr, c, arow0, arow1, brow, szrow, acc);
    gemm_step<BITS>(r2, kt + 2, true, sA, sB, szl, szr, c, arow0, arow1, brow, szrow, acc);
  }
  if (kt < ge)       // tail: at most two steps, already loaded
    gemm_step<BITS>(r0, kt, false, sA, sB, szl, szr, c, arow0, arow1, brow, szrow, acc);
  if (kt + 1 < ge)
    gemm_step<BITS>(r1, kt + 1, false, sA, sB, szl, szr, c, arow0, arow1, brow, szrow, acc);

  // Combine the two k-halves: waves 4..7 hand their partial quadrant to
  // waves 0..3 through LDS (64 KB, reusing the stage buffers), in a fixed
  // order.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  const int quad = wave & 3;
  if (wave >= 4) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          red[((quad * 4 + i * 2 + j) * 16 + v) * kWave + lane] = acc[i][j][v];
  }
  __syncthreads();
  if (wave < 4) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          acc[i][j][v] += red[((quad * 4 + i * 2 + j) * 16 + v) * kWave + lane];
  }

  const int tile = blockIdx.y * gridDim.x + blockIdx.x;
  if (S > 1) {
    // Split K: every slice writes its partial tile; the last slice to arrive
    // (per-tile counter) sums all partials in slice order 0..S-1, so the
    // result does not depend on arrival order, and resets the counter.
    __shared__ uint32_t last_flag;
    float* mine = partials + (static_cast<size_t>(z) * gridDim.x * gridDim.y + tile) * kTileFloats;
    if (wave < 4) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            __hip_atomic_store(&mine[((quad * 4 + i * 2 + j) * 16 + v) * kWave + lane],
                               acc[i][j][v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // The partial stores above are agent-scope atomics, written through to
    // the device coherence point (the L2 of each XCD is not coherent with
    // the others).  Waiting for their acknowledgement (vmcnt = 0) before the
    // barrier makes them visible device-wide before thread 0 counts the
    // arrival; this replaces a full agent fence, whose L2 writeback and
    // invalidate would also evict the operands of tiles still running on
    // this XCD.
    // vmcnt(0) only (the assembler encodes the counter fields; the LDS and
    // export counters are left alone).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      last_flag = prev == static_cast<uint32_t>(S - 1);
    }
    __syncthreads();
    if (!last_flag) return;
    // Last arrival: every other slice's partial was acknowledged before its
    // count, so agent-scope loads issued now read them.
    if (wave < 4) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
      for (int zz = 0; zz < S; ++zz) {
        const float* p = partials + (static_cast<size_t>(zz) * gridDim.x * gridDim.y + tile) * kTileFloats;
        // An accumulator's loads first, then its adds: the loads overlap
        // instead of each waiting for the previous one.
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            float part[16];
#pragma unroll
            for (int v = 0; v < 16; ++v)
              part[v] = __hip_atomic_load(&p[((quad * 4 + i * 2 + j) * 16 + v) * kWave + lane],
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] += part[v];
          }
      }
    }
    if (tid == 0)   // ready for the next call
      __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if (wave < 4) {
    // 32x32 accumulator layout: column = lane % 32,
    // row = 8 * (v / 4) + 4 * (lane / 32) + v % 4.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + c.wn + 32 * j + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + c.wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if (m < M && n < N) yt[static_cast<size_t>(m) * N + n] = acc[i][j][v];
        }
      }
    }
  }
}

template <int BITS>
hipError_t launch_bits(const harp_qweight& W, const uint16_t* xt, float* yt,
                       int M, int splits, float* partials, uint32_t* counters,
                       hipStream_t stream) {
  const int tn = (W.N + BN - 1) / BN;
  const int tm = (M + BM - 1) / BM;
  const dim3 grid(tn, tm, splits);
  hipLaunchKernelGGL((gemm_kernel<BITS>), grid, dim3(kThreads), 0, stream, W.qweight,
                     W.scale, W.zero, xt, yt, W.N, W.K, M,
                     splits > 1 ? partials : nullptr, splits > 1 ? counters : nullptr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const harp_qweight& W, const uint16_t* xt, float* yt,
                       int M, int splits, float* partials, uint32_t* counters,
                       hipStream_t stream) {
  switch (W.bits) {
    case 2: return launch_bits<2>(W, xt, yt, M, splits, partials, counters, stream);
    case 3: return launch_bits<3>(W, xt, yt, M, splits, partials, counters, stream);
    case 4: return launch_bits<4>(W, xt, yt, M, splits, partials, counters, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace harp
