// The x~ planes of the one-row FP4 x FP8 matrix-core product (gemv_f4.hip):
// the device code that builds one step's planes, shared by the plane kernel
// there and by the input rotation's last launch (rotate.hip), which builds
// them straight from its registers.  The operand layout is described at the
// top of gemv_f4.hip.
#pragma once

#include "device_common.hpp"

namespace harp {
namespace f4 {

constexpr int kPlanes = 8;

// Lane reductions over one 16-lane row with DPP moves (quad swaps, then the
// half-row and row mirrors): every lane of the row ends with the result,
// formed in the same order in each.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp<0xb1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp<0x4e>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp<0x141>(v));   // row_half_mirror
  return fmaxf(v, dpp<0x140>(v));   // row_mirror
}
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<0xb1>(v);
  v += dpp<0x4e>(v);
  v += dpp<0x141>(v);
  return v + dpp<0x140>(v);
}

constexpr int kStepLds = 1024 + 16;       // LDS bytes per step: planes, then 16 zero bytes

// Planes of one step of 128 inputs, built by one wave into LDS.  One
// 16-lane row per 32-input block b, two inputs per lane (block offsets
// u = j and j + 16 for lane j of the row); rows 0-1 and rows 2-3 are the
// step's two quantization groups.  Per group, with 2^E <= max |x~| < 2^(E+1),
// every input becomes the integer X = rint(x~ 2^(27-E)) (|X| < 2^28, error
// at most 2^(E-28)), written in balanced base 16, X = sum_i d_i 16^i with
// digits d_i in [-8, 7] (the nibbles of X + 0x88888888, less 8), and plane
// p holds digit 7 - p, whose weight is 2^(E+1-4p).  Digits are small
// integers, exact in FP8, and one plane of one group shares one scale:
// every product the matrix cores sum for a result is an integer of at most
// 24 times that scale, so their sums are exact (with products spread over
// the whole FP8 range the instruction's sum was measured to lose bits about
// 2^-11 below its largest term).  Groups below 2^-100 (a plane's scale
// would fall below 2^-127) are left as zero.
// xs: the step's inputs (x~ + 256 t + 64 e for step 2t + e).  Planes go to
// pl[lane][16] in operand order: block offset u becomes operand offset
// o = pi^-1(u) and lands in operand lane (p + 8h) + 16 g, byte o % 16, with
// h = b / 2 and g = 2 (b % 2) + o / 16; bytes 1024..1039 are zeroed.  The
// scale byte of plane p (E + 1 - 4p + 127) goes to psc[lane] for the lanes
// that supply operand row p + 8h's scale of the group's blocks; the rows of
// the other group half get 127 (their operand bytes there are zero).  The
// sums of x~ over the step's groups 4t + e and 4t + 2 + e (fixed order) go
// to sx[0] and sx[2].
__device__ __forceinline__ void build_step(const float* __restrict__ xs, uint8_t* pl,
                                           uint8_t* psc, float* sx, int lane) {
  const int j = lane & 15;
  const int b = lane >> 4;
  const int k0 = 128 * (b >> 1) + 32 * (b & 1) + j;
  const float ra = xs[k0];
  const float rb = xs[k0 + 16];
  {
    const float t = row_sum(ra + rb);
    // rows 1 and 3 add lane 15 of rows 0 and 2 (row_bcast:15)
    const float g2 = t + __int_as_float(__builtin_amdgcn_update_dpp(
                             0, __float_as_int(t), 0x142, 0xa, 0xf, false));
    if (j == 15 && (b & 1)) sx[2 * (b >> 1)] = g2;
  }
  if (lane < 4) reinterpret_cast<uint32_t*>(pl + 1024)[lane] = 0u;
  // group maximum: row maximum, then rows 0 <-> 1 and 2 <-> 3 exchanged
  float m = row_max(fmaxf(fabsf(ra), fabsf(rb)));
  {
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m),
                                                     false, false);
    m = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  const int E = static_cast<int>((__float_as_uint(m) >> 23) & 0xff) - 127;   // floor(log2 m)
  const bool live = m > 0.0f && E >= -100;
  const uint32_t ya = live ? static_cast<uint32_t>(__float2int_rn(ldexpf(ra, 27 - E))) + 0x88888888u
                           : 0x88888888u;
  const uint32_t yb = live ? static_cast<uint32_t>(__float2int_rn(ldexpf(rb, 27 - E))) + 0x88888888u
                           : 0x88888888u;
  const int o = 8 * (j & 1) + (j >> 1);   // operand offset of u = j (u = j + 16: o + 16)
  const int h = b >> 1;
  uint8_t* dst = pl + 2 * (b & 1) * 256 + o;
  uint8_t* sdst = psc + 16 * b;
#pragma unroll
  for (int p = 0; p < kPlanes; ++p) {
    const int sh = 4 * (kPlanes - 1 - p);
    const float da = static_cast<float>(static_cast<int>((ya >> sh) & 15u) - 8);
    const float db = static_cast<float>(static_cast<int>((yb >> sh) & 15u) - 8);
    const uint32_t enc = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(da, db, 0, false));
    dst[(p + 8 * h) * 16] = static_cast<uint8_t>(enc & 0xffu);
    dst[256 + (p + 8 * h) * 16] = static_cast<uint8_t>((enc >> 8) & 0xffu);
    if (j == 0) sdst[p + 8 * h] = static_cast<uint8_t>(live ? E + 1 - 4 * p + 127 : 127);
    if (j == 1) sdst[p + 8 * (1 - h)] = 127;
  }
}

// One wave writes the step that build_step left in stage (its planes in
// bytes 0..1023, its 64 scale bytes from kStepLds on) and ssx (the two group
// sums at [0] and [2]) to the f4 region: one 16-byte store per lane (planes pl[step][lane][16]), one 4-byte
// store per lane of the first 16 (scale bytes psc[step][lane]) and two
// floats (group sums gsx[group]).
__device__ __forceinline__ void emit_step(const uint8_t* stage, const float* ssx, int s,
                                          u32x4* __restrict__ pl, uint32_t* __restrict__ psc,
                                          float* __restrict__ gsx, int lane) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  pl[static_cast<size_t>(s) * kWave + lane] = reinterpret_cast<const u32x4*>(stage)[lane];
  if (lane < 16)
    psc[static_cast<size_t>(s) * 16 + lane] =
        reinterpret_cast<const uint32_t*>(stage + kStepLds)[lane];
  if (lane < 2) gsx[4 * (s >> 1) + 2 * lane + (s & 1)] = ssx[2 * lane];
}

}  // namespace f4
}  // namespace harp
