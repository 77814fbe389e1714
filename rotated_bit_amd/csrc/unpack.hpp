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

// Four codes below 16 in the byte lanes of m as floats q 2^-9, two per
// instruction: the packed FP8 (OCP e4m3) decode maps byte values 0..15 to
// exactly q 2^-9 (subnormal below 8, the first binade from 8 to 15).  A
// product formed from them is exactly 2^-9 times the one formed from q
// (every rounding scales with it), so scaling the sum by kFp8CodeScale
// restores it bit for bit.
constexpr float kFp8CodeScale = 512.0f;
__device__ __forceinline__ void fp8_codes4(uint32_t m, float& q0, float& q1, float& q2,
                                           float& q3) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(m), false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(m), true);
  q0 = lo[0];
  q1 = lo[1];
  q2 = hi[0];
  q3 = hi[1];
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

// One group (64 codes) of one row occupies 2*BITS words, loaded as
// 16-byte (2 and 4 bits) or 8-byte (3 bits: the row stride is 24*G bytes)
// vector loads.
template <int BITS>
__device__ __forceinline__ void load_group(const uint32_t* __restrict__ p,
                                           uint32_t (&w)[2 * BITS]) {
  if constexpr (BITS == 2) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if constexpr (BITS == 4) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p);
    const u32x4 b = *reinterpret_cast<const u32x4*>(p + 4);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
    w[4] = b[0]; w[5] = b[1]; w[6] = b[2]; w[7] = b[3];
  } else {
    // 24 bytes per group: 8-byte aligned (the row stride is 24*G bytes).
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const uint2 v = *reinterpret_cast<const uint2*>(p + 2 * i);
      w[2 * i] = v.x;
      w[2 * i + 1] = v.y;
    }
  }
}

// Eight consecutive codes 8c .. 8c+7 (c = 0..3) of 32-code run h of a
// group, packed in the low 8*BITS bits of the result.  h must be a
// compile-time constant after unrolling; c may vary per lane, so the words
// are chosen with selects (an array indexed by c would live in scratch
// memory).
template <int BITS>
__device__ __forceinline__ uint32_t chunk8(const uint32_t (&w)[2 * BITS], int h, int c) {
  // The words pass through opaque() so that the selects below stay selects
  // between registers (the optimizer would otherwise turn them back into an
  // indexed access).
  uint32_t r[BITS];
#pragma unroll
  for (int i = 0; i < BITS; ++i) r[i] = opaque(w[h * BITS + i]);
  if constexpr (BITS == 2) {
    const uint32_t x = (c & 2) ? r[1] : r[0];
    return x >> (16 * (c & 1));
  } else if constexpr (BITS == 4) {
    const uint32_t lo = (c & 1) ? r[1] : r[0];
    const uint32_t hi = (c & 1) ? r[3] : r[2];
    return (c & 2) ? hi : lo;
  } else {
    // 3 bits: 24 bits at bit 24c of the run's 96-bit integer, i.e. word
    // (24c)/32 from bit (24c)%32 on, continued in the next word.
    const uint32_t lo = c == 3 ? r[2] : (c == 2 ? r[1] : r[0]);
    const uint32_t hi = c >= 2 ? r[2] : r[1];
    return __builtin_amdgcn_alignbit(hi, lo, (24 * c) & 31);
  }
}

// The eight codes of a chunk as floats (2 and 4 bits: masked into byte
// lanes, one byte-to-float convert each).
template <int BITS>
__device__ __forceinline__ void chunk8_codes(uint32_t v, float (&q)[8]) {
  if constexpr (BITS == 2) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t m = opaque((v >> (2 * t)) & 0x0303u);   // codes t, t+4
      q[t] = static_cast<float>(m & 0xffu);
      q[t + 4] = static_cast<float>((m >> 8) & 0xffu);
    }
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t m = opaque((v >> (4 * t)) & 0x0f0f0f0fu);  // codes t, t+2, t+4, t+6
#pragma unroll
      for (int i = 0; i < 4; ++i) q[t + 2 * i] = static_cast<float>((m >> (8 * i)) & 0xffu);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = static_cast<float>((v >> (3 * j)) & 7u);
  }
}

// The eight codes of a chunk as the bf16 values 1 + q / 2^BITS, two per
// word, code 2i in the low half of word i.  bf16 1.0 is 0x3f80 and its
// seven stored mantissa bits are 2^-1 .. 2^-7, so q placed in the top BITS
// of them gives 1 + q / 2^BITS exactly: one shift and one AND-OR per word.
// (Codes in the top bits rather than the bottom ones keep the constant part
// of the operand small against the code part, 2^BITS : q instead of 128 : q,
// which is what the per-group sum T - (1 + z / 2^BITS) S cancels.)
// base: two bf16 1.0 (0x3f803f80) held in a register by the caller, so
// that mask and OR fuse into one AND-OR per word (an instruction takes at
// most one literal).
template <int BITS>
__device__ __forceinline__ u32x4 chunk8_bf16_unit(uint32_t v, uint32_t base) {
  const uint32_t kBase = base;
  constexpr int kTop = 7 - BITS;             // bit of the code's LSB in a half
  u32x4 out;
  if constexpr (BITS == 2) {
    const uint32_t v16 = v & 0xffffu;          // the chunk; higher bits are other codes
    const uint32_t u = v16 | (v16 << 14);      // code 2i at bit 4i, code 2i+1 at bit 4i + 16
    constexpr uint32_t kMask = 0x00030003u << kTop;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sh = kTop - 4 * i;             // bring bit 4i to bit kTop
      const uint32_t w = sh >= 0 ? (u << sh) : (u >> -sh);
      out[i] = (w & kMask) | kBase;
    }
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = v >> (8 * i);
      out[i] = ((x & 0x0000000fu) << kTop) | ((x & 0x000000f0u) << (12 + kTop)) | kBase;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out[i] = (((v >> (6 * i)) & 7u) << kTop) | (((v >> (6 * i + 3)) & 7u) << (16 + kTop)) |
               kBase;
  }
  return out;
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
