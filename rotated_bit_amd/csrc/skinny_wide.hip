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

template <int BITS, int MB, bool XF32, int FB>
__global__ __launch_bounds__(kThreadsW) void skinny_wide_kernel(
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint16_t* __restrict__ zr, const void* __restrict__ xt,
    float* __restrict__ yt, int N, int K, int M) {
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

  // This wave's groups: [gb, gb + cnt), cnt a multiple of kSzBlkW.
  const int cnt = G / kWavesW;
  const int gb = wave * cnt;
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

  // One group (slot j of block buffer buf): x~ planes to LDS, fragments,
  // S once, then T and the scaled update for every feature block.
  auto group = [&](const WARegs<MB, XF32>& r, const WCRegs<BITS, FB>& cr, int buf, int j) {
    // A wave's LDS accesses run in issue order, so the previous group's
    // fragment reads are done before these stores.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (XF32) {
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
        b[h] = __builtin_bit_cast(bf16x8, chunk8_bf16_unit<BITS>(chunk8<BITS>(cr.w[fb], h, c)));
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
  for (int slot = tid; slot < FB * MB * kWave * 4; slot += kThreadsW) {
    const int v = slot & 3;
    const int l = (slot >> 2) & (kWave - 1);
    const int mb = (slot >> 8) % MB;
    const int fb = (slot >> 8) / MB;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWavesW; ++w) sum += red[w][fb][mb][l][v];
    const int m = m0 + 16 * mb + 4 * (l >> 4) + v;
    const int nn = n0 + 16 * fb + (l & 15);
    if (m < M && nn < N) yt[static_cast<size_t>(m) * N + nn] = sum;
  }
}

template <int BITS, int MB, bool XF32, int FB>
hipError_t launch_w(const harp_qweight& W, const void* xt, float* yt, int M,
                    hipStream_t stream) {
  const dim3 grid((W.N + 16 * FB - 1) / (16 * FB), (M + 16 * MB - 1) / (16 * MB));
  hipLaunchKernelGGL((skinny_wide_kernel<BITS, MB, XF32, FB>), grid, dim3(kThreadsW), 0, stream,
                     W.qweight, W.scale, W.zero, xt, yt, W.N, W.K, M);
  return hipGetLastError();
}

template <int BITS, bool XF32, int FB>
hipError_t launch_fb(const harp_qweight& W, const void* xt, float* yt, int M,
                     hipStream_t stream) {
  // up to 16 rows in one 16-row block, more in tiles of 32 rows
  return M <= 16 ? launch_w<BITS, 1, XF32, FB>(W, xt, yt, M, stream)
                 : launch_w<BITS, 2, XF32, FB>(W, xt, yt, M, stream);
}

template <int BITS, bool XF32>
hipError_t launch_bits_w(const harp_qweight& W, const void* xt, float* yt, int M,
                         hipStream_t stream) {
  return skinny_wide_blocks(W.N) >= 4 ? launch_fb<BITS, XF32, 4>(W, xt, yt, M, stream)
                                      : launch_fb<BITS, XF32, 2>(W, xt, yt, M, stream);
}

}  // namespace

// Feature blocks per wave for N output features (0: use the 16-feature
// kernel): as many as keep at least one workgroup per CU (256), at most 4.
int skinny_wide_blocks(int N) {
  const int blocks = N / 16;
  if (blocks >= 4 * 256) return 4;
  if (blocks >= 2 * 256) return 2;
  return 0;
}

bool skinny_wide_supported(const harp_qweight& W, int M) {
  return M >= 1 && M <= 64 && W.K % (kGroup * kWavesW * kSzBlkW) == 0 &&
         skinny_wide_blocks(W.N) > 0;
}

hipError_t launch_skinny_wide(const harp_qweight& W, const void* xt, bool xf32, float* yt,
                              int M, hipStream_t stream) {
  if (!skinny_wide_supported(W, M)) return hipErrorInvalidValue;
  switch (W.bits) {
    case 2: return xf32 ? launch_bits_w<2, true>(W, xt, yt, M, stream)
                        : launch_bits_w<2, false>(W, xt, yt, M, stream);
    case 3: return xf32 ? launch_bits_w<3, true>(W, xt, yt, M, stream)
                        : launch_bits_w<3, false>(W, xt, yt, M, stream);
    case 4: return xf32 ? launch_bits_w<4, true>(W, xt, yt, M, stream)
                        : launch_bits_w<4, false>(W, xt, yt, M, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace harp
