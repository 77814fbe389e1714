// Device unpack and dequant of the packed low-bit weights.
//
// Layout (stand-in quantizer; the HARP pages leave the codebook open):
// a run of 32 consecutive codes of a row occupies exactly BITS uint32 words.
// For BITS 2 and 4 the codes sit least-significant first, 32/BITS per word;
// for BITS 3 the run is one 96-bit little-endian integer, code j at bits
// 3j..3j+2, so codes 10 and 21 straddle two words (read with a funnel
// shift).  Dequant: w_hat = (q - z) * s with s an fp16 scale and z an
// integer fp16 zero per group of 64 codes; |q - z| <= 15 and s has 11
// significant bits, so the float32 product is exact.
//
// Every product kernel and the dequant test hook use these functions.
#pragma once

#include "device_common.hpp"

namespace harp {

constexpr int kGroup = 64;

// Code j (0 <= j < 32*NW/BITS) of a word array holding consecutive codes.
template <int BITS, int NW>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[NW], int j) {
  const int pos = BITS * j;
  const int wi = pos >> 5;
  const int off = pos & 31;
  constexpr uint32_t mask = (1u << BITS) - 1u;
  if (off + BITS <= 32) return (w[wi] >> off) & mask;
  return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], off) & mask;
}

// Load the BITS words of one 32-code run starting at word index `word0`.
template <int BITS>
__device__ __forceinline__ void load_run32(const uint32_t* __restrict__ row,
                                           int word0, uint32_t (&w)[BITS]) {
  if constexpr (BITS == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(row + word0);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (BITS == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + word0);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
#pragma unroll
    for (int i = 0; i < BITS; ++i) w[i] = row[word0 + i];
  }
}

// Keeps a masked dword opaque to the optimizer, so that its byte lanes are
// converted with v_cvt_f32_ubyte0..3 instead of being re-extracted one
// field at a time.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm("" : "+v"(v));
  return v;
}

// Codes of one 32-code run as floats.  2- and 4-bit codes are masked four
// at a time into byte lanes, each then a single byte-to-float convert.
template <int BITS>
__device__ __forceinline__ void codes_run32(const uint32_t (&w)[BITS], float (&q)[32]) {
  if constexpr (BITS == 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t m = opaque((w[h] >> (2 * t)) & 0x03030303u);  // codes t, t+4, t+8, t+12
#pragma unroll
        for (int i = 0; i < 4; ++i)
          q[16 * h + t + 4 * i] = static_cast<float>((m >> (8 * i)) & 0xffu);
      }
    }
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t m = opaque((w[h] >> (4 * t)) & 0x0f0f0f0fu);  // codes t, t+2, t+4, t+6
#pragma unroll
        for (int i = 0; i < 4; ++i)
          q[8 * h + t + 2 * i] = static_cast<float>((m >> (8 * i)) & 0xffu);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) q[j] = static_cast<float>(code_at<BITS, BITS>(w, j));
  }
}

// 16 consecutive codes (a quarter of a group) as floats: one word of
// 2-bit codes or two words of 4-bit codes, masked into byte lanes.
template <int BITS>
__device__ __forceinline__ void codes_16(const uint32_t* w, float (&q)[16]) {
  static_assert(BITS == 2 || BITS == 4, "16-code parts exist for 2 and 4 bits");
  if constexpr (BITS == 2) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t m = opaque((w[0] >> (2 * t)) & 0x03030303u);  // codes t, t+4, t+8, t+12
#pragma unroll
      for (int i = 0; i < 4; ++i) q[t + 4 * i] = static_cast<float>((m >> (8 * i)) & 0xffu);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t m = opaque((w[h] >> (4 * t)) & 0x0f0f0f0fu);  // codes t, t+2, t+4, t+6
#pragma unroll
        for (int i = 0; i < 4; ++i)
          q[8 * h + t + 2 * i] = static_cast<float>((m >> (8 * i)) & 0xffu);
      }
    }
  }
}

// Dequantize one 32-code run to float32, exactly: q*s and z*s are exact
// (at most 4 + 11 significant bits) and so is their difference, so the
// fused multiply-add q*s - z*s equals (q - z)*s in every evaluation order.
template <int BITS>
__device__ __forceinline__ void dequant_run32(const uint32_t (&w)[BITS],
                                              float s, float z,
                                              float (&out)[32]) {
  float q[32];
  codes_run32<BITS>(w, q);
  const float nzs = -z * s;
#pragma unroll
  for (int j = 0; j < 32; ++j) out[j] = fmaf(q[j], s, nzs);
}

}  // namespace harp
