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

// Dequantize one 32-code run to float32 (exact).
template <int BITS>
__device__ __forceinline__ void dequant_run32(const uint32_t (&w)[BITS],
                                              float s, float z,
                                              float (&out)[32]) {
#pragma unroll
  for (int j = 0; j < 32; ++j)
    out[j] = (static_cast<float>(code_at<BITS, BITS>(w, j)) - z) * s;
}

}  // namespace harp
