// Small-batch product on wide feature strips (the same product as
// skinny.hip: y'[m][n] = sum_k w_hat[n][k] x~[m][k], float32 accumulate,
// w_hat applied exactly through the codes 1 + q / 2^B and per-group sums).
//
// Why a second kernel.  A workgroup of the 16-feature kernel reads all of
// x~ (M K values) for its 16 features, so x~ crosses the L2 N / 16 times:
// at M = 32 and K = 8192, 28672 features, that is ~1.8 GB per call against
// 59 MB of codes, and the call is bound by it.  Here each wave multiplies
// the x~ operand of a group against FB blocks of 16 features, so x~ crosses
// the L2 N / (16 FB) times and its split into bf16 planes, its re-layout
// and its sum S are done once per FB blocks.
//
// gfx950 mapping.  Eight waves per workgroup own a strip of 16 FB features;
// wave w takes the w-th eighth of the quantization groups (K a multiple of
// 4096, so every wave gets a whole number of eight-group blocks).  Per
// group: x~ (loaded coalesced, split into hi / lo bf16 planes for a
// float32 x~) passes through the wave's LDS rows into operand order; the
// v_mfma_f32_16x16x32_bf16 products give S = sum x~ once and
// T = sum (1 + q / 2^B) x~ for each feature block, whose lane (feature
// l % 16, inputs 8 (l / 16) .. +7 of each k-slice) loads its feature's
// group of codes itself (four lanes share each 16-byte access) and builds
// the operand with one AND-OR per two codes.  Scales and zeros go through
// the wave's LDS in eight-group blocks (one 16-byte load per feature and
// array per block).  The loads of the next groups run ahead in a ring of
// register sets.  The eight waves' partial sums are combined through LDS
// in wave order 0..7, so the result is bitwise reproducible.
#include "launch.hpp"
#include "unpack.hpp"
#include "validate.hpp"

namespace harp {
namespace {

constexpr int kWavesW = 8;
constexpr int kThreadsW = kWavesW * kWave;
constexpr int kXsRowW = kGroup + 8;   // bf16 per padded LDS row of x~
constexpr int kSzBlkW = 8;            // groups per scale / zero block

typedef float floatx4_w __attribute__((ext_vector_type(4)));

// x~ of one group for one lane: rows 16 mb + 8 i + lane / 8, inputs
// 8 (lane % 8) .. +7 of the group (eight lanes per 128-byte row segment).
template <int MB, bool XF32>
struct WARegs {
  static constexpr int V = XF32 ? 2 : 1;
  u32x4 a[MB][2][V];
};

// One group of codes of the lane's feature in each of the FB blocks.
template <int BITS, int FB>
struct WCRegs {
  uint32_t w[FB][2 * BITS];
};

// Per-wave LDS: x~ planes in operand order, and two buffers of scale /
// zero blocks [buffer][feature row][scale | zero][group in block].
template <int MB, bool XF32, int FB>
struct WaveLds {
  static constexpr int P = XF32 ? 2 : 1;
  uint16_t xs[P][MB][16][kXsRowW];
  uint16_t sz[2][16 * FB][2][kSzBlkW];
};

// hi = bf16(x), lo = bf16(x - hi), round to nearest even (x - hi exact).
__device__ __forceinline__ void split_planes(const u32x4 (&f)[2], u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = __uint_as_float(f[k >> 1][2 * (k & 1)]);
    const float b = __uint_as_float(f[k >> 1][2 * (k & 1) + 1]);
    const uint32_t h = pack_bf16x2(a, b);
    hi[k] = h;
    lo[k] = pack_bf16x2(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xffff0000u));
  }
}

// XIN: 0 bf16 x~; 1 float32 x~, split here; 2 float32 x~ already split in
// place by split_chunks_kernel (each 8-element chunk as 8 bf16 hi values,
// then 8 bf16 lo values: the same 32 bytes).
template <int BITS, int MB, int XIN, int FB>
__global__ __launch_bounds__(kThreadsW) void skinny_wide_kernel(
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint16_t* __restrict__ zr, const void* __restrict__ xt,
    float* __restrict__ yt, int N, int K, int M, float* __restrict__ partials,
    uint32_t* __restrict__ counters) {
  constexpr bool XF32 = XIN != 0;
  using L = WaveLds<MB, XF32, FB>;
  constexpr int P = L::P;
  constexpr int NW = 2 * BITS;
  constexpr int kRedBytes = kWavesW * FB * MB * kWave * 16;
  constexpr int kLoopBytes = kWavesW * static_cast<int>(sizeof(L));
  __shared__ __attribute__((aligned(16)))
      unsigned char smem[kRedBytes > kLoopBytes ? kRedBytes : kLoopBytes];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane >> 4;
  const int G = K / kGroup;
  const size_t WPR = static_cast<size_t>(K) * BITS / 32;
  const int n0 = blockIdx.x * 16 * FB;
  const int m0 = blockIdx.y * 16 * MB;
  L& ld = reinterpret_cast<L*>(smem)[wave];

  // the lane's feature in each block (rows past N: loaded, never stored)
  const uint32_t* wrow[FB];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
    wrow[fb] = qw + static_cast<size_t>(min(n0 + 16 * fb + (lane & 15), N - 1)) * WPR;
  // x~ rows (rows past M: read, never stored)
  const char* arow[MB][2];
  const size_t row_bytes = static_cast<size_t>(K) * (XF32 ? 4 : 2);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 2; ++i)
      arow[mb][i] = static_cast<const char*>(xt) +
                    static_cast<size_t>(min(m0 + 16 * mb + 8 * i + (lane >> 3), M - 1)) *
                        row_bytes;
  // scale / zero block role: pairs (feature row, array) p = lane + 64 j
  constexpr int kSzPairs = 2 * 16 * FB;
  constexpr int kSzPerLane = (kSzPairs + kWave - 1) / kWave;
  const uint16_t* szrow[kSzPerLane];
#pragma unroll
  for (int j = 0; j < kSzPerLane; ++j) {
    const int p = min(lane + kWave * j, kSzPairs - 1);
    const int row = min(n0 + (p >> 1), N - 1);
    szrow[j] = ((p & 1) ? zr : sc) + static_cast<size_t>(row) * G;
  }

  floatx4_w acc[FB][MB];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[fb][mb] = floatx4_w{0.0f, 0.0f, 0.0f, 0.0f};

  // This workgroup's K slice (blockIdx.z of gridDim.z, each a multiple of
  // 64 groups) and this wave's groups in it: [gb, gb + cnt), cnt a
  // multiple of kSzBlkW.
  const int S = gridDim.z;
  const int z = blockIdx.z;
  const int cnt = G / S / kWavesW;
  const int gb = z * (G / S) + wave * cnt;
  const int nblk = cnt / kSzBlkW;

  auto load_a = [&](WARegs<MB, XF32>& r, int g) {
    constexpr int kEs = XF32 ? 4 : 2;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const u32x4* p = reinterpret_cast<const u32x4*>(
            arow[mb][i] + static_cast<size_t>(g * kGroup + 8 * (lane & 7)) * kEs);
#pragma unroll
        for (int v = 0; v < WARegs<MB, XF32>::V; ++v) r.a[mb][i][v] = p[v];
      }
  };
  auto load_c = [&](WCRegs<BITS, FB>& cr, int g) {
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) load_group<BITS>(wrow[fb] + static_cast<size_t>(g) * NW, cr.w[fb]);
  };
  u32x4 szr[kSzPerLane];
  auto load_sz = [&](int blk) {   // absolute block index, clamped to the wave's last
    const int g0 = gb + kSzBlkW * min(blk, nblk - 1);
#pragma unroll
    for (int j = 0; j < kSzPerLane; ++j) szr[j] = *reinterpret_cast<const u32x4*>(szrow[j] + g0);
  };
  auto store_sz = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kSzPerLane; ++j) {
      const int p = lane + kWave * j;
      if (p < kSzPairs)
        *reinterpret_cast<u32x4*>(&ld.sz[buf][p >> 1][p & 1][0]) = szr[j];
    }
  };

  constexpr uint32_t kOnes = 0x3f803f80u;   // two bf16 1.0
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{kOnes, kOnes, kOnes, kOnes});
  uint32_t base = kOnes;   // kept in a register (one AND-OR per operand word)
  asm volatile("" : "+v"(base));

  // One group (slot j of block buffer buf): x~ planes to LDS, fragments,
  // S once, then T and the scaled update for every feature block.
  auto group = [&](const WARegs<MB, XF32>& r, const WCRegs<BITS, FB>& cr, int buf, int j) {
    // A wave's LDS accesses run in issue order, so the previous group's
    // fragment reads are done before these stores.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (XIN == 2) {
          *reinterpret_cast<u32x4*>(&ld.xs[0][mb][8 * i + (lane >> 3)][8 * (lane & 7)]) =
              r.a[mb][i][0];
          *reinterpret_cast<u32x4*>(&ld.xs[1][mb][8 * i + (lane >> 3)][8 * (lane & 7)]) =
              r.a[mb][i][1];
        } else if constexpr (XF32) {
          u32x4 hi, lo;
          split_planes(r.a[mb][i], hi, lo);
          *reinterpret_cast<u32x4*>(&ld.xs[0][mb][8 * i + (lane >> 3)][8 * (lane & 7)]) = hi;
          *reinterpret_cast<u32x4*>(&ld.xs[P - 1][mb][8 * i + (lane >> 3)][8 * (lane & 7)]) = lo;
        } else {
          *reinterpret_cast<u32x4*>(&ld.xs[0][mb][8 * i + (lane >> 3)][8 * (lane & 7)]) =
              r.a[mb][i][0];
        }
      }
    bf16x8 a[P][2][MB];
#pragma unroll
    for (int pl = 0; pl < P; ++pl)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          a[pl][h][mb] = *reinterpret_cast<const bf16x8*>(&ld.xs[pl][mb][lane & 15][32 * h + 8 * c]);
    floatx4_w sx[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      sx[mb] = floatx4_w{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int pl = 0; pl < P; ++pl)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          sx[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[pl][h][mb], ones, sx[mb], 0, 0, 0);
    }
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
      bf16x8 b[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        b[h] = __builtin_bit_cast(bf16x8, chunk8_bf16_unit<BITS>(chunk8<BITS>(cr.w[fb], h, c), base));
      floatx4_w t[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        t[mb] = floatx4_w{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int pl = 0; pl < P; ++pl)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            t[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[pl][h][mb], b[h], t[mb], 0, 0, 0);
      }
      // w_hat = 2^B s ((1 + q / 2^B) - (1 + z / 2^B)), both factors exact
      const int frow = 16 * fb + (lane & 15);
      const float s = f16_to_f32(ld.sz[buf][frow][0][j]) * static_cast<float>(1 << BITS);
      const float zo = fmaf(f16_to_f32(ld.sz[buf][frow][1][j]), 1.0f / (1 << BITS), 1.0f);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          acc[fb][mb][v] = fmaf(s, fmaf(-zo, sx[mb][v], t[mb][v]), acc[fb][mb][v]);
    }
  };

  // Rings of two register sets (x~ and codes of groups g and g + 1); the
  // loop is unrolled over a scale / zero block, so every index is static.
  // Loads past the wave's last group re-read it (valid memory, unused).
  WARegs<MB, XF32> ra0, ra1;
  WCRegs<BITS, FB> rc0, rc1;
  const int glast = gb + cnt - 1;
  load_sz(0);
  store_sz(0);
  load_sz(1);
  load_a(ra0, gb);
  load_c(rc0, gb);
  load_a(ra1, min(gb + 1, glast));
  load_c(rc1, min(gb + 1, glast));
  for (int blk = 0; blk < nblk; ++blk) {
    const int g = gb + kSzBlkW * blk;
    const int buf = blk & 1;
#pragma unroll
    for (int j = 0; j < kSzBlkW; j += 2) {
      group(ra0, rc0, buf, j);
      load_a(ra0, min(g + j + 2, glast));
      load_c(rc0, min(g + j + 2, glast));
      group(ra1, rc1, buf, j + 1);
      load_a(ra1, min(g + j + 3, glast));
      load_c(rc1, min(g + j + 3, glast));
    }
    // block blk + 1 (loaded during this block) into the other buffer, which
    // this wave last read in block blk - 1; then fetch block blk + 2
    store_sz(buf ^ 1);
    load_sz(blk + 2);
  }

  // Combine the eight K ranges in wave order.  Accumulator layout of a
  // 16x16 block: lane l holds column (feature) l % 16, rows 4 (l / 16) + v.
  __syncthreads();   // every wave is done with its loop buffers
  floatx4_w (*red)[FB][MB][kWave] = reinterpret_cast<floatx4_w (*)[FB][MB][kWave]>(smem);
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[wave][fb][mb][lane] = acc[fb][mb];
  __syncthreads();
  constexpr int kSlots = FB * MB * kWave * 4;
  constexpr int kPerThread = (kSlots + kThreadsW - 1) / kThreadsW;
  float sum[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int slot = tid + k * kThreadsW;
    sum[k] = 0.0f;
    if (slot < kSlots) {
      const int v = slot & 3;
      const int l = (slot >> 2) & (kWave - 1);
      const int mb = (slot >> 8) % MB;
      const int fb = (slot >> 8) / MB;
#pragma unroll
      for (int w = 0; w < kWavesW; ++w) sum[k] += red[w][fb][mb][l][v];
    }
  }
  auto out_index = [&](int slot, int& m, int& nn) {
    const int v = slot & 3;
    const int l = (slot >> 2) & (kWave - 1);
    const int mb = (slot >> 8) % MB;
    const int fb = (slot >> 8) / MB;
    m = m0 + 16 * mb + 4 * (l >> 4) + v;
    nn = n0 + 16 * fb + (l & 15);
  };
  if (S > 1) {
    // Split K: every slice writes its partial strip (device-coherent
    // stores, acknowledged before the arrival is counted); the last slice
    // to arrive adds all S partials in slice order 0..S-1, so the result
    // does not depend on arrival order, and resets the tile's counter.
    __shared__ uint32_t last_flag;
    const size_t plane = static_cast<size_t>(M) * N;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int slot = tid + k * kThreadsW;
      int m, nn;
      out_index(slot, m, nn);
      if (slot < kSlots && m < M && nn < N)
        __hip_atomic_store(&partials[z * plane + static_cast<size_t>(m) * N + nn], sum[k],
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int tile = blockIdx.y * gridDim.x + blockIdx.x;
    if (tid == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      last_flag = prev == static_cast<uint32_t>(S - 1);
    }
    __syncthreads();
    if (!last_flag) return;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int slot = tid + k * kThreadsW;
      int m, nn;
      out_index(slot, m, nn);
      if (slot < kSlots && m < M && nn < N) {
        float t = 0.0f;
        for (int zz = 0; zz < S; ++zz) {
          const float part = __hip_atomic_load(
              &partials[zz * plane + static_cast<size_t>(m) * N + nn], __ATOMIC_RELAXED,
              __HIP_MEMORY_SCOPE_AGENT);
          t = zz == 0 ? part : t + part;
        }
        sum[k] = t;
      }
    }
    if (tid == 0)
      __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int slot = tid + k * kThreadsW;
    int m, nn;
    out_index(slot, m, nn);
    if (slot < kSlots && m < M && nn < N) yt[static_cast<size_t>(m) * N + nn] = sum[k];
  }
}

template <int BITS, int MB, int XIN, int FB>
hipError_t launch_w(const harp_qweight& W, const void* xt, float* yt, int M, int S,
                    float* partials, uint32_t* counters, hipStream_t stream) {
  const dim3 grid((W.N + 16 * FB - 1) / (16 * FB), (M + 16 * MB - 1) / (16 * MB), S);
  hipLaunchKernelGGL((skinny_wide_kernel<BITS, MB, XIN, FB>), grid, dim3(kThreadsW), 0, stream,
                     W.qweight, W.scale, W.zero, xt, yt, W.N, W.K, M, partials, counters);
  return hipGetLastError();
}

template <int BITS, int XIN, int FB>
hipError_t launch_fb(const harp_qweight& W, const void* xt, float* yt, int M, int S,
                     float* partials, uint32_t* counters, hipStream_t stream) {
  // up to 16 rows in one 16-row block, more in tiles of 32 rows
  return M <= 16 ? launch_w<BITS, 1, XIN, FB>(W, xt, yt, M, S, partials, counters, stream)
                 : launch_w<BITS, 2, XIN, FB>(W, xt, yt, M, S, partials, counters, stream);
}

template <int BITS, int XIN>
hipError_t launch_bits_w(const harp_qweight& W, const void* xt, float* yt, int M, int fb,
                         int S, float* partials, uint32_t* counters, hipStream_t stream) {
  return fb == 4 ? launch_fb<BITS, XIN, 4>(W, xt, yt, M, S, partials, counters, stream)
                 : launch_fb<BITS, XIN, 2>(W, xt, yt, M, S, partials, counters, stream);
}

// In place: each 8-element chunk of float32 x~ becomes 8 bf16 hi =
// bf16(x) and then 8 bf16 lo = bf16(x - hi) (nearest even; x - hi exact), in
// the chunk's own 32 bytes, so that the product loads both planes of a
// chunk with the loads it would use for the float32 values.
__global__ __launch_bounds__(256) void split_chunks_kernel(float* __restrict__ xt, size_t chunks) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= chunks) return;
  u32x4* p = reinterpret_cast<u32x4*>(xt + 8 * i);
  const u32x4 f[2] = {p[0], p[1]};
  u32x4 hi, lo;
  split_planes(f, hi, lo);
  p[0] = hi;
  p[1] = lo;
}

}  // namespace

hipError_t launch_skinny_wide(const harp_qweight& W, const void* xt, int xin, float* yt,
                              int M, int fb, int splits, float* partials, uint32_t* counters,
                              hipStream_t stream) {
  if ((fb != 2 && fb != 4) || splits < 1 || xin < 0 || xin > 2 ||
      W.K % (kGroup * kWavesW * kSzBlkW * splits) != 0 ||
      (splits > 1 && (partials == nullptr || counters == nullptr)))
    return hipErrorInvalidValue;
#define HARP_W(B, X) launch_bits_w<B, X>(W, xt, yt, M, fb, splits, partials, counters, stream)
  switch (W.bits) {
    case 2: return xin == 0 ? HARP_W(2, 0) : xin == 1 ? HARP_W(2, 1) : HARP_W(2, 2);
    case 3: return xin == 0 ? HARP_W(3, 0) : xin == 1 ? HARP_W(3, 1) : HARP_W(3, 2);
    case 4: return xin == 0 ? HARP_W(4, 0) : xin == 1 ? HARP_W(4, 1) : HARP_W(4, 2);
    default: return hipErrorInvalidValue;
  }
#undef HARP_W
}

hipError_t launch_split_chunks(float* xt, size_t n, hipStream_t stream) {
  if (n % 8 != 0) return hipErrorInvalidValue;
  const size_t chunks = n / 8;
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(split_chunks_kernel, dim3(static_cast<unsigned>((chunks + 255) / 256)),
                     dim3(256), 0, stream, xt, chunks);
  return hipGetLastError();
}

}  // namespace harp
