// Dequant GEMM for small batches (M <= 64) on the bf16 matrix cores:
//     y'[m][n] = sum_k w_hat[n][k] * x~[m][k],  float32 accumulate,
// with w_hat = (q - z) s applied exactly: per quantization group g of 64
// inputs the matrix cores form T = sum_k (1 + q_k / 2^B) x~_k (the codes
// enter as the exact bf16 values 1 + q / 2^B) and S = sum_k x~_k (against a
// constant all-ones operand), and the group adds 2^B s (T - (1 + z / 2^B) S)
// in float32.
//
// Two input forms:
// * bf16 x~ (the caller rounded it): one operand plane;
// * float32 x~: each value is split in registers into hi = bf16(x~) and
//   lo = bf16(x~ - hi) (both round to nearest even; x~ - hi is exact), and
//   both planes are multiplied into the same sums.  |x~ - hi - lo| <=
//   2^-16 |x~|, so the product keeps x~ to about 16 significant bits instead
//   of 8: the float32-operand form of the small-batch product.
//
// gfx950 mapping.  A workgroup of eight waves owns a strip of 16 output
// features; wave w takes the w-th eighth of the quantization groups along
// K.  Per group (two k-slices of v_mfma_f32_16x16x32_bf16) lane l supplies
// feature n = l % 16 and inputs 8c .. 8c+7 of each slice, c = l / 16: it
// loads that feature's group of codes (16/24/32 bytes, shared with the three
// other lanes of the feature through the L1) and turns its 16 codes into the
// B operand with one AND-OR per two codes.  x~ is read with coalesced loads
// and passed through a per-wave LDS block into operand order (the float32
// form passes hi, then lo, through the same block).  Each code is fetched
// once; there are no LDS operand tiles and no barriers in the K loop, and
// the loads of the next groups are in flight while a group is multiplied.
// The eight waves' partial sums are combined through LDS in wave order
// 0..7, so the result is bitwise reproducible.
#include "launch.hpp"
#include "unpack.hpp"
#include "validate.hpp"

namespace harp {
namespace {

constexpr int kWavesS = 8;
constexpr int kThreadsS = kWavesS * kWave;   // 512
constexpr int kStrip = 16;                   // output features per workgroup

typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kXsRow = kGroup + 8;        // bf16 per padded LDS row of x~
constexpr int kBlk = 4;                   // groups per coalesced code block

// x~ of one quantization group for one lane, loaded coalesced (eight lanes
// per 128-byte row segment: lane l holds row 16 mb + 8 i + l/8, inputs
// 8 (l % 8) .. +7 of the group) and re-laid out through LDS into the
// matrix-core operand order, where neighbouring lanes read different rows.
// XF32: x~ is float32, eight inputs are two 16-byte vectors.
template <int MB, bool XF32>
struct ARegs {
  static constexpr int V = XF32 ? 2 : 1;
  u32x4 a[MB][2][V];
};

// One lane's share of a code block: feature row l/4 of the strip, group
// g0 + l % 4, so neighbouring lanes read neighbouring groups of a row.
template <int BITS>
struct CodeRegs {
  uint32_t w[2 * BITS];
  uint16_t s16, z16;
};

// Per-wave LDS of a code block: [buffer][feature][group slot][words], rows
// padded by 16 bytes so that the operand-order reads (feature per lane)
// spread over the banks; scale and zero packed in one word per slot.
template <int BITS>
struct CodeLds {
  static constexpr int ROW = kBlk * 2 * BITS + 4;
};

// arow: the byte address of each fragment row (bf16 or float32 elements).
template <int MB, bool XF32>
__device__ __forceinline__ void load_a(ARegs<MB, XF32>& r, int g,
                                       const char* const (&arow)[MB][2], int lane) {
  constexpr int kEs = XF32 ? 4 : 2;   // element bytes
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const u32x4* p = reinterpret_cast<const u32x4*>(
          arow[mb][i] + static_cast<size_t>(g * kGroup + 8 * (lane & 7)) * kEs);
#pragma unroll
      for (int v = 0; v < ARegs<MB, XF32>::V; ++v) r.a[mb][i][v] = p[v];
    }
}

// hi = bf16(x), lo = bf16(x - hi) for eight float32 values (two vectors),
// as bf16 pairs (element 2i in the low half of word i).  Rounding is to
// nearest even; x - hi is exact (hi is within a factor 2^-8 of x).
__device__ __forceinline__ void split_bf16(const u32x4 (&f)[2], u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = __uint_as_float(f[k >> 1][2 * (k & 1)]);
    const float b = __uint_as_float(f[k >> 1][2 * (k & 1) + 1]);
    const uint32_t h = pack_bf16x2(a, b);
    hi[k] = h;
    lo[k] = pack_bf16x2(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xffff0000u));
  }
}

// One group: the lane's feature codes (w) and packed scale/zero (sz) from
// the code block in LDS, x~ from registers via the wave's LDS rows.
template <int BITS, int MB, bool XF32>
__device__ __forceinline__ void mma_group(const ARegs<MB, XF32>& r, const uint32_t (&w)[2 * BITS],
                                          uint32_t sz, int lane, uint16_t (*xs)[16][kXsRow],
                                          uint32_t base, floatx4_t (&acc)[MB]) {
  const int c = lane >> 4;
  constexpr uint32_t kOnes = 0x3f803f80u;    // two bf16 1.0
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{kOnes, kOnes, kOnes, kOnes});
  bf16x8 b[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    b[h] = __builtin_bit_cast(bf16x8, chunk8_bf16_unit<BITS>(chunk8<BITS>(w, h, c), base));
  floatx4_t t[MB], sx[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    t[mb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    sx[mb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  constexpr int kPlanes = XF32 ? 2 : 1;
#pragma unroll
  for (int pl = 0; pl < kPlanes; ++pl) {
    // This wave's x~ block of the group (this plane) into its own LDS rows.
    // No other wave touches them, and a wave's LDS accesses run in issue
    // order, so the previous plane's or group's operand reads are done.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        u32x4 v;
        if constexpr (XF32) {
          u32x4 hi, lo;
          split_bf16(r.a[mb][i], hi, lo);
          v = pl == 0 ? hi : lo;
        } else {
          v = r.a[mb][i][0];
        }
        *reinterpret_cast<u32x4*>(&xs[mb][8 * i + (lane >> 3)][8 * (lane & 7)]) = v;
      }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&xs[mb][lane & 15][32 * h + 8 * c]);
        t[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[h], t[mb], 0, 0, 0);
        sx[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ones, sx[mb], 0, 0, 0);
      }
    }
  }
  // Accumulator layout of a 16x16 block: lane l holds column (feature)
  // l % 16, so one scale and zero per lane.  w_hat = 2^B s ((1 + q / 2^B) -
  // (1 + z / 2^B)); both factors are exact in float32.
  const float s = f16_to_f32(static_cast<uint16_t>(sz & 0xffffu)) * static_cast<float>(1 << BITS);
  const float zo = fmaf(f16_to_f32(static_cast<uint16_t>(sz >> 16)), 1.0f / (1 << BITS), 1.0f);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[mb][v] = fmaf(s, fmaf(-zo, sx[mb][v], t[mb][v]), acc[mb][v]);
}

template <int BITS, int MB, bool XF32>
__global__ __launch_bounds__(kThreadsS) void skinny_kernel(
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint16_t* __restrict__ zr, const void* __restrict__ xt,
    float* __restrict__ yt, int N, int K, int M) {
  constexpr int NW = 2 * BITS;
  constexpr int CROW = CodeLds<BITS>::ROW;
  __shared__ floatx4_t red[kWavesS][MB][kWave];
  __shared__ __attribute__((aligned(16))) uint16_t xsw[kWavesS][MB][16][kXsRow];
  __shared__ __attribute__((aligned(16))) uint32_t cw[kWavesS][2][16][CROW];
  __shared__ uint32_t szw[kWavesS][2][16][kBlk];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int G = K / kGroup;
  const size_t WPR = static_cast<size_t>(K) * BITS / 32;
  const int n0 = blockIdx.x * kStrip;
  const int m0 = blockIdx.y * 16 * MB;   // first row of this workgroup's row tile
  // code-block role: row n0 + l/4 (rows past N: loaded, never stored)
  const int crow = min(n0 + (lane >> 2), N - 1);
  const uint32_t* wrow = qw + static_cast<size_t>(crow) * WPR;
  const uint16_t* srow = sc + static_cast<size_t>(crow) * G;
  const uint16_t* zrow = zr + static_cast<size_t>(crow) * G;
  const char* arow[MB][2];
  const size_t row_bytes = static_cast<size_t>(K) * (XF32 ? 4 : 2);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)   // rows past M: read, never stored
#pragma unroll
    for (int i = 0; i < 2; ++i)
      arow[mb][i] = static_cast<const char*>(xt) +
                    static_cast<size_t>(min(m0 + 16 * mb + 8 * i + (lane >> 3), M - 1)) *
                        row_bytes;
  uint16_t (*xs)[16][kXsRow] = xsw[wave];
  uint32_t (*cl)[16][CROW] = cw[wave];
  uint32_t (*szl)[16][kBlk] = szw[wave];

  floatx4_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
  uint32_t base = 0x3f803f80u;   // two bf16 1.0, kept in a register
  asm volatile("" : "+v"(base));

  // This wave's groups [gb, ge), in blocks of kBlk.  The codes and scales of
  // block b+1 are in flight while block b is multiplied; the x~ of the next
  // groups rides in a ring of register sets (four, or two when the
  // fragments of a set fill the registers: wide batches, float32 x~).  Loads past ge re-read
  // group ge-1 (valid memory, never multiplied).  Named sets, not arrays,
  // keep the rings in registers.
  const int gb = wave * G / kWavesS;
  const int ge = (wave + 1) * G / kWavesS;
  if (gb < ge) {
    const int cnt = ge - gb;
    CodeRegs<BITS> cr;
    auto load_codes = [&](int blk) {
      const int g = min(gb + kBlk * blk + (lane & 3), ge - 1);
      load_group<BITS>(wrow + static_cast<size_t>(g) * NW, cr.w);
      cr.s16 = srow[g];
      cr.z16 = zrow[g];
    };
    auto store_codes = [&](int buf) {
      uint32_t* d = &cl[buf][lane >> 2][(lane & 3) * NW];
#pragma unroll
      for (int i = 0; i < NW; ++i) d[i] = cr.w[i];
      szl[buf][lane >> 2][lane & 3] = static_cast<uint32_t>(cr.s16) |
                                      (static_cast<uint32_t>(cr.z16) << 16);
    };
    // group j of the block in buffer buf, for this lane's feature
    auto group = [&](const ARegs<MB, XF32>& r, int buf, int j) {
      uint32_t w[NW];
      const uint32_t* src = &cl[buf][lane & 15][j * NW];
#pragma unroll
      for (int i = 0; i < NW; ++i) w[i] = src[i];
      mma_group<BITS, MB, XF32>(r, w, szl[buf][lane & 15][j], lane, xs, base, acc);
    };
    auto load = [&](ARegs<MB, XF32>& r, int g) {
      load_a<MB, XF32>(r, min(g, ge - 1), arow, lane);
    };

    load_codes(0);
    store_codes(0);
    load_codes(1);
    int g = gb;
    int blk = 0;
    if constexpr (XF32 ? MB == 1 : MB <= 3) {
      ARegs<MB, XF32> r0, r1, r2, r3;
      load(r0, gb);
      load(r1, gb + 1);
      load(r2, gb + 2);
      load(r3, gb + 3);
      for (; g + kBlk <= ge; g += kBlk, ++blk) {
        const int buf = blk & 1;
        group(r0, buf, 0);
        load(r0, g + 4);
        group(r1, buf, 1);
        load(r1, g + 5);
        group(r2, buf, 2);
        load(r2, g + 6);
        group(r3, buf, 3);
        load(r3, g + 7);
        store_codes(buf ^ 1);          // block blk+1, loaded during this block
        load_codes(blk + 2);
      }
      const int buf = blk & 1;
      if (g < ge) group(r0, buf, 0);
      if (g + 1 < ge) group(r1, buf, 1);
      if (g + 2 < ge) group(r2, buf, 2);
    } else {
      ARegs<MB, XF32> r0, r1;
      load(r0, gb);
      load(r1, gb + 1);
      for (; g + kBlk <= ge; g += kBlk, ++blk) {
        const int buf = blk & 1;
        group(r0, buf, 0);
        load(r0, g + 2);
        group(r1, buf, 1);
        load(r1, g + 3);
        group(r0, buf, 2);
        load(r0, g + 4);
        group(r1, buf, 3);
        load(r1, g + 5);
        store_codes(buf ^ 1);
        load_codes(blk + 2);
      }
      const int buf = blk & 1;
      if (g < ge) group(r0, buf, 0);
      if (g + 1 < ge) group(r1, buf, 1);
      if (g + 2 < ge) {
        load(r0, g + 2);
        group(r0, buf, 2);
      }
    }
    (void)cnt;
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
    const int m = m0 + 16 * mb + 4 * (l >> 4) + v;
    const int nn = n0 + (l & 15);
    if (m < M && nn < N) yt[static_cast<size_t>(m) * N + nn] = sum;
  }
}

// Each workgroup takes 16 MB rows; more rows take more row tiles (grid.y).
template <int BITS, int MB, bool XF32>
hipError_t launch_mb(const harp_qweight& W, const void* xt, float* yt, int M,
                     hipStream_t stream) {
  const dim3 grid((W.N + kStrip - 1) / kStrip, (M + 16 * MB - 1) / (16 * MB));
  hipLaunchKernelGGL((skinny_kernel<BITS, MB, XF32>), grid, dim3(kThreadsS), 0, stream,
                     W.qweight, W.scale, W.zero, xt, yt, W.N, W.K, M);
  return hipGetLastError();
}

template <int BITS, bool XF32>
hipError_t launch_bits(const harp_qweight& W, const void* xt, float* yt, int M,
                       hipStream_t stream) {
  switch ((M + 15) / 16) {
    case 1: return launch_mb<BITS, 1, XF32>(W, xt, yt, M, stream);
    case 2: return launch_mb<BITS, 2, XF32>(W, xt, yt, M, stream);
    case 3: return launch_mb<BITS, 3, XF32>(W, xt, yt, M, stream);
    // float32 x~ holds twice the registers per row: 49..64 rows run as two
    // 32-row tiles (four 16-row blocks would spill)
    case 4:
      if constexpr (XF32) return launch_mb<BITS, 2, XF32>(W, xt, yt, M, stream);
      else return launch_mb<BITS, 4, XF32>(W, xt, yt, M, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool XF32>
hipError_t launch_any(const harp_qweight& W, const void* xt, float* yt, int M,
                      hipStream_t stream) {
  switch (W.bits) {
    case 2: return launch_bits<2, XF32>(W, xt, yt, M, stream);
    case 3: return launch_bits<3, XF32>(W, xt, yt, M, stream);
    case 4: return launch_bits<4, XF32>(W, xt, yt, M, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm_skinny(const harp_qweight& W, const uint16_t* xt, float* yt,
                              int M, hipStream_t stream) {
  const WideSplit w = skinny_wide_split(M, W.N, W.K, false);
  if (w.fb > 0) return launch_skinny_wide(W, xt, 0, yt, M, w.fb, 1, nullptr, nullptr, stream);
  return launch_any<false>(W, xt, yt, M, stream);
}

hipError_t launch_gemm_skinny_split(const harp_qweight& W, const float* xt, float* yt,
                                    int M, hipStream_t stream) {
  const WideSplit w = skinny_wide_split(M, W.N, W.K, false);
  if (w.fb > 0) return launch_skinny_wide(W, xt, 1, yt, M, w.fb, 1, nullptr, nullptr, stream);
  return launch_any<true>(W, xt, yt, M, stream);
}

constexpr size_t kPresplitMinElems = size_t{1} << 17;

hipError_t launch_gemm_skinny_split_k(const harp_qweight& W, const float* xt, float* yt,
                                      int M, float* partials, uint32_t* counters,
                                      hipStream_t stream) {
  const WideSplit w = skinny_wide_split(M, W.N, W.K, true);
  if (w.fb == 0) return launch_any<true>(W, xt, yt, M, stream);
  // x~ is the caller's workspace here: split it once, in place, instead of
  // in every strip's workgroup, where that saves more than the extra launch
  // (measured: not at 16 x 4096)
  if (static_cast<size_t>(M) * W.K < kPresplitMinElems)
    return launch_skinny_wide(W, xt, 1, yt, M, w.fb, w.splits, partials, counters, stream);
  const hipError_t e =
      launch_split_chunks(const_cast<float*>(xt), static_cast<size_t>(M) * W.K, stream);
  if (e != hipSuccess) return e;
  return launch_skinny_wide(W, xt, 2, yt, M, w.fb, w.splits, partials, counters, stream);
}

}  // namespace harp
