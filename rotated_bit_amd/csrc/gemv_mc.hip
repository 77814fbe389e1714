// Small-batch decode product on the bf16 matrix cores, float32 x~ carried
// exactly:
//     y'[m][n] = sum_k w_hat[n][k] x~[m][k],   3 <= M <= 8 rows, 2 or 4 bits,
// w_hat = (q - z) s the stand-in per-group uniform grid (HARP technical
// summary §2.4 leaves the quantizer backend open), applied exactly.  (One or
// two rows, and 3-bit codes, run faster on the vector-ALU product: there the
// matrix cores' 16-row block is mostly empty and the code operands cost as
// much as the vector multiply-adds they replace.)
//
// Operands.  Each x~ value is split into P bf16 planes by repeated rounding
// to nearest even: p_0 = bf16(x), p_1 = bf16(x - p_0), p_2 = bf16(x - p_0 -
// p_1); each difference is exact in float32.  Three planes hold all 24
// significant bits (x = p_0 + p_1 + p_2 exactly; up to five rows); two hold
// 16 of them (|x - p_0 - p_1| <= 2^-16 |x|; six to eight rows).  Row m plane
// p is row P m + p of the 16-row operand block.  Codes enter as the exact
// bf16 values 1 + q / 2^B; every code-plane product is exact in float32.
// Per quantization group of 64 inputs the matrix cores give T = sum (1 + q /
// 2^B) x and, against a constant all-ones operand, S = sum x per plane row,
// and the group adds 2^B s (T - (1 + z / 2^B) S) in float32.
//
// The order of a group's 64 inputs inside the contraction is free as long
// as both operands follow it.  Lane chunk c (= lane / 16) takes inputs 16 c
// .. 16 c + 15 of the group, so its codes are one contiguous piece of the
// packed row (4 bytes at 2 bits, 8 at 4), and inside the chunk codes that
// sit 16 bits apart in a word are paired in one operand dword, so one shift
// and one AND-OR place both (the x~ planes are laid out in the same order).
//
// Loads.  The codes move in blocks of four groups: lane (r, c) loads group
// g0 + c of feature r whole (16 or 32 bytes; the four lanes of a feature read
// 64 or 128 contiguous bytes), and two rounds of v_permlane32_swap /
// v_permlane16_swap (a 4 x 4 transpose across the lane quarters) leave lane
// (r, c) with chunk c of every group of the block; each lane loads one
// group's scale and zero and takes the block's other three from the lanes of
// the other quarters.  A block's x~ and codes leave one block ahead of the
// product, in the order they are consumed.  x~ is loaded coalesced, input l
// of every row by lane l, split once per group, and passed through a
// per-wave LDS block into operand order.
//
// gfx950 mapping.  A workgroup of eight waves owns a strip of 16 J output
// features; wave w takes the w-th eighth of the groups along K.  Per group
// the wave forms S once and reuses both x~ operands for the J 16-feature
// tiles: 2 + 2 J v_mfma_f32_16x16x32_bf16.  The waves' partial sums are
// combined through LDS in wave order and summed over planes in order
// 0 .. P-1, so the result is bitwise reproducible.
#include "launch.hpp"
#include "unpack.hpp"
#include "validate.hpp"

namespace harp {
namespace {

constexpr int kWavesM = 8;
constexpr int kThreadsM = kWavesM * kWave;   // 512

typedef float floatx4_t __attribute__((ext_vector_type(4)));

// The planes of one x~ value, plane p as a bf16 bit pattern.
template <int P>
__device__ __forceinline__ void planes_of(float x, uint16_t (&b)[P]) {
  const uint16_t h0 = f32_to_bf16(x);
  b[0] = h0;
  const float r1 = x - bf16_to_f32(h0);
  if constexpr (P >= 2) {
    const uint16_t h1 = f32_to_bf16(r1);
    b[1] = h1;
    if constexpr (P == 3) b[2] = f32_to_bf16(r1 - bf16_to_f32(h1));
  }
}

// 4 x 4 transpose across the lane quarters: on entry quarter c of d_i holds
// item (c, i), on exit quarter c of d_k holds item (k, c).
__device__ __forceinline__ void transpose4(uint32_t& d0, uint32_t& d1, uint32_t& d2,
                                           uint32_t& d3) {
  const auto a = __builtin_amdgcn_permlane32_swap(d0, d2, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(d1, d3, false, false);
  const auto e = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto f = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  d0 = e[0];
  d1 = e[1];
  d2 = f[0];
  d3 = f[1];
}

// One block of codes for J tiles: 2 bits, one 16-byte group per lane; 4
// bits, 32 bytes; the packed scale and zero (fp16 bits, scale low, zero
// high) of the lane's feature for group g0 + c, and after transpose_block
// for group g0 + k in sz[k].
template <int BITS, int J>
struct Block {
  static constexpr int V = BITS / 2;          // 16-byte vectors per group
  u32x4 w[J][V];
  uint32_t sz[J][4];
};

template <int BITS, int J>
__device__ __forceinline__ void transpose_block(Block<BITS, J>& b) {
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if constexpr (BITS == 2) {
      uint32_t d0 = b.w[j][0][0], d1 = b.w[j][0][1], d2 = b.w[j][0][2], d3 = b.w[j][0][3];
      transpose4(d0, d1, d2, d3);
      b.w[j][0] = u32x4{d0, d1, d2, d3};
    } else {
      // the first and the second word of each chunk
      uint32_t e0 = b.w[j][0][0], e1 = b.w[j][0][2], e2 = b.w[j][1][0], e3 = b.w[j][1][2];
      uint32_t o0 = b.w[j][0][1], o1 = b.w[j][0][3], o2 = b.w[j][1][1], o3 = b.w[j][1][3];
      transpose4(e0, e1, e2, e3);
      transpose4(o0, o1, o2, o3);
      b.w[j][0] = u32x4{e0, e1, e2, e3};
      b.w[j][1] = u32x4{o0, o1, o2, o3};
    }
    // every quarter holds its own group's scale: each lane takes the four
    // of its feature from the lanes of the other quarters
    const uint32_t own = b.sz[j][0];
    const int rl = threadIdx.x & 15;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      b.sz[j][k] = static_cast<uint32_t>(__shfl(static_cast<int>(own), rl + 16 * k, kWave));
  }
}

// Codes to operands.  2 and 4 bits pair codes that sit 16 bits apart in a
// word, so one shift and one AND-OR (with the bf16 1.0 pair in a register)
// place both in the top BITS mantissa bits of their halves: 2 bits, word w
// (codes t at bit 2t), dword i = codes (i, i + 8), slice i / 4; 4 bits,
// words w0, w1 (codes 8 h + t at bit 4t of w_h), dword (h, p) = codes
// (8 h + p, 8 h + p + 4), slice h.  in_pos gives, for a lane's input t
// (0..15), its place among the 16 operand elements (slice 0 then slice 1).
template <int BITS>
__device__ __forceinline__ int in_pos(int t) {
  if constexpr (BITS == 2) {
    const int i = t & 7;
    return 8 * (i >> 2) + 2 * (i & 3) + (t >> 3);
  } else {
    const int tt = t & 7;
    return 8 * (t >> 3) + 2 * (tt & 3) + (tt >> 2);
  }
}

template <int BITS>
__device__ __forceinline__ uint32_t pair_op(uint32_t w, int sh, uint32_t base) {
  constexpr uint32_t kMask = (BITS == 2 ? 0x00030003u : 0x000f000fu) << (7 - BITS);
  const uint32_t x = sh >= 0 ? (w >> sh) : (w << -sh);
  uint32_t o;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(o) : "v"(x), "s"(kMask), "v"(base));
  return o;
}

// Both slices of one lane's codes as operands.
template <int BITS>
__device__ __forceinline__ void codes_op(uint32_t w0, uint32_t w1, uint32_t base,
                                         bf16x8& b0, bf16x8& b1) {
  u32x4 s0, s1;
  if constexpr (BITS == 2) {
    // code t at bit 2t: bring code i to bit 7 - BITS
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s0[i] = pair_op<2>(w0, 2 * i - 5, base);
      s1[i] = pair_op<2>(w0, 2 * (i + 4) - 5, base);
    }
  } else {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      s0[p] = pair_op<4>(w0, 4 * p - 3, base);
      s1[p] = pair_op<4>(w1, 4 * p - 3, base);
    }
  }
  b0 = __builtin_bit_cast(bf16x8, s0);
  b1 = __builtin_bit_cast(bf16x8, s1);
}

// MT: the batch rows the kernel is built for (4, 5 or 8; rows M .. MT-1 read
// row M - 1 and are never stored), P planes per row.
template <int BITS, int MT, int J>
__global__ __launch_bounds__(kThreadsM) __attribute__((amdgpu_waves_per_eu(2, 4)))
void gemv_mc_kernel(const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                    const uint16_t* __restrict__ zr, const float* __restrict__ xt,
                    float* __restrict__ yt, int N, int K, int M) {
  static_assert(BITS == 2 || BITS == 4, "2 or 4 bits");
  constexpr int P = 3 * MT <= 16 ? 3 : 2;
  __shared__ floatx4_t red[kWavesM][J][kWave];
  // per wave: one group's planes, row m P + p, 64 inputs in operand order
  // (plus 16 bytes of padding per row against bank conflicts)
  __shared__ __attribute__((aligned(16))) uint16_t xpl[kWavesM][16][kGroup + 8];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar loop bounds
  const int G = K / kGroup;
  const size_t WPR = static_cast<size_t>(K) * BITS / 32;
  const int n0 = blockIdx.x * 16 * J;
  const int r = lane & 15;                      // operand row / feature column
  const int c = lane >> 4;                      // input chunk / lane quarter
  const int rm = r / P;                         // operand row r: batch row r / P, plane r % P
  const int rp = r - rm * P;
  const bool live = rm < M;                     // rows past the batch stay zero
  const int wpos = (lane & ~15) + in_pos<BITS>(lane & 15);   // this lane's input, operand order
  uint16_t (*xp)[kGroup + 8] = xpl[wave];
  uint32_t base = 0x3f803f80u;                  // two bf16 1.0, kept in a register
  asm volatile("" : "+v"(base));
  const uint32_t* wrow[J];
  const uint16_t* srow[J];
  const uint16_t* zrow[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int n = min(n0 + 16 * j + r, N - 1);  // rows past N: loaded, never stored
    wrow[j] = qw + static_cast<size_t>(n) * WPR;
    srow[j] = sc + static_cast<size_t>(n) * G;
    zrow[j] = zr + static_cast<size_t>(n) * G;
  }

  floatx4_t acc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) acc[j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  constexpr uint32_t kOnes = 0x3f803f80u;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{kOnes, kOnes, kOnes, kOnes});
  const float s_mul = static_cast<float>(1 << BITS);
  const float z_mul = 1.0f / static_cast<float>(1 << BITS);

  // x~ of one group: lane l holds input l of every row
  auto load_x = [&](float (&xv)[MT], int g) {
#pragma unroll
    for (int mm = 0; mm < MT; ++mm)
      xv[mm] = xt[static_cast<size_t>(min(mm, M - 1)) * K + static_cast<size_t>(g) * kGroup + lane];
  };
  // The x~ operands of one group: each lane splits its own inputs once; the
  // wave's LDS block turns them into operand order (a wave's LDS accesses
  // run in issue order, so the previous group's reads are done).
  auto x_operands = [&](const float (&xv)[MT], bf16x8& a0, bf16x8& a1) {
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      uint16_t b[P];
      planes_of<P>(xv[mm], b);
#pragma unroll
      for (int pp = 0; pp < P; ++pp) xp[mm * P + pp][wpos] = b[pp];
    }
    u32x4 a[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
    if (live) {
      a[0] = *reinterpret_cast<const u32x4*>(&xp[rm * P + rp][16 * c]);
      a[1] = *reinterpret_cast<const u32x4*>(&xp[rm * P + rp][16 * c + 8]);
    }
    a0 = __builtin_bit_cast(bf16x8, a[0]);
    a1 = __builtin_bit_cast(bf16x8, a[1]);
  };
  // the group's update of tile j: one scale and zero per lane (lane l holds
  // accumulator column, i.e. feature, l % 16)
  auto scale_group = [&](int j, const floatx4_t& t, const floatx4_t& sx, uint32_t sz) {
    const float s = f16_to_f32(static_cast<uint16_t>(sz & 0xffffu)) * s_mul;
    const float zo = fmaf(f16_to_f32(static_cast<uint16_t>(sz >> 16)), z_mul, 1.0f);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[j][v] = fmaf(s, fmaf(-zo, sx[v], t[v]), acc[j][v]);
  };

  const int gb = wave * G / kWavesM;
  const int ge = (wave + 1) * G / kWavesM;
  if (gb < ge) {
    const int gl = ge - 1;
    // blocks of four groups; loads past ge re-read group ge - 1 (valid
    // memory, never multiplied)
    using B = Block<BITS, J>;
    auto load_block = [&](B& b, int g0) {
      const int gc = min(g0 + c, gl);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const u32x4* p = reinterpret_cast<const u32x4*>(wrow[j] + static_cast<size_t>(gc) * 2 * BITS);
#pragma unroll
        for (int v = 0; v < B::V; ++v) b.w[j][v] = p[v];
        b.sz[j][0] = static_cast<uint32_t>(srow[j][gc]) | (static_cast<uint32_t>(zrow[j][gc]) << 16);
      }
    };
    auto load_xblk = [&](float (&xv)[4][MT], int g0) {
#pragma unroll
      for (int k = 0; k < 4; ++k) load_x(xv[k], min(g0 + k, gl));
    };
    auto run_block = [&](B& b, const float (&xv)[4][MT], int g0) {
      transpose_block<BITS, J>(b);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (g0 + k < ge) {
          bf16x8 a0, a1;
          x_operands(xv[k], a0, a1);
          floatx4_t sx = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
          sx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, ones, sx, 0, 0, 0);
          sx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, ones, sx, 0, 0, 0);
#pragma unroll
          for (int j = 0; j < J; ++j) {
            bf16x8 b0, b1;
            if constexpr (BITS == 2) codes_op<2>(b.w[j][0][k], 0u, base, b0, b1);
            else codes_op<4>(b.w[j][0][k], b.w[j][1][k], base, b0, b1);
            floatx4_t t = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, t, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, t, 0, 0, 0);
            scale_group(j, t, sx, b.sz[j][k]);
          }
        }
      }
    };
    // Loads leave in the order they are consumed (a block's x~, then its
    // codes), one block ahead: the memory counter retires loads in issue
    // order, so waiting for a block never waits for a later one.
    B b0, b1;
    float x0[4][MT], x1[4][MT];
    load_xblk(x0, gb);
    load_block(b0, gb);
    load_xblk(x1, gb + 4);
    load_block(b1, gb + 4);
    for (int g = gb; g < ge; g += 8) {
      run_block(b0, x0, g);
      load_xblk(x0, g + 8);
      load_block(b0, g + 8);
      if (g + 4 < ge) {
        run_block(b1, x1, g + 4);
        load_xblk(x1, g + 12);
        load_block(b1, g + 12);
      }
    }
  }

  // Combine the eight K ranges in wave order, then the planes of each row.
  // Accumulator layout: lane l holds column l % 16, rows 4 (l / 16) + v.
#pragma unroll
  for (int j = 0; j < J; ++j) red[wave][j][lane] = acc[j];
  __syncthreads();
  for (int task = tid; task < J * 16 * M; task += kThreadsM) {
    const int j = task / (16 * M);
    const int rem = task - j * 16 * M;
    const int mm = rem >> 4;
    const int col = rem & 15;
    const int n = n0 + 16 * j + col;
    float sum = 0.0f;
#pragma unroll
    for (int pp = 0; pp < P; ++pp) {
      const int row = mm * P + pp;
      const int l = 16 * (row >> 2) + col;
      float part = 0.0f;
#pragma unroll
      for (int w = 0; w < kWavesM; ++w) part += red[w][j][l][row & 3];
      sum += part;
    }
    if (n < N) yt[static_cast<size_t>(mm) * N + n] = sum;
  }
}

template <int BITS, int MT, int J>
hipError_t launch_mj(const harp_qweight& W, const float* xt, float* yt, int M,
                     hipStream_t stream) {
  const dim3 grid((W.N + 16 * J - 1) / (16 * J));
  hipLaunchKernelGGL((gemv_mc_kernel<BITS, MT, J>), grid, dim3(kThreadsM), 0, stream,
                     W.qweight, W.scale, W.zero, xt, yt, W.N, W.K, M);
  return hipGetLastError();
}

template <int BITS, int MT>
hipError_t launch_m(const harp_qweight& W, const float* xt, float* yt, int M,
                    hipStream_t stream) {
  // two 16-feature tiles per wave once that still leaves two workgroups
  // per CU slot
  if (W.N >= 16 * 2 * 512) return launch_mj<BITS, MT, 2>(W, xt, yt, M, stream);
  return launch_mj<BITS, MT, 1>(W, xt, yt, M, stream);
}

template <int BITS>
hipError_t launch_b(const harp_qweight& W, const float* xt, float* yt, int M,
                    hipStream_t stream) {
  if (M <= 4) return launch_m<BITS, 4>(W, xt, yt, M, stream);
  if (M == 5) return launch_m<BITS, 5>(W, xt, yt, M, stream);
  return launch_m<BITS, 8>(W, xt, yt, M, stream);
}

}  // namespace

hipError_t launch_gemv_mc(const harp_qweight& W, const float* xt, float* yt, int M,
                          hipStream_t stream) {
  if (M < kGemvMcMinM || M > kGemvMcMaxM) return hipErrorInvalidValue;
  switch (W.bits) {
    case 2: return launch_b<2>(W, xt, yt, M, stream);
    case 4: return launch_b<4>(W, xt, yt, M, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace harp
