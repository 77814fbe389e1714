// Small device helpers shared by the HARP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace harp {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
// Native 16-byte vector (HIP's uint4 class does not stay in registers when
// held in arrays across a pipelined loop).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even (v_cvt_pk_bf16_f32 under the default round mode).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats to a packed bf16 pair (low half = a), round to nearest even;
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Multiply by -1 when bit is 1 (exact).
__device__ __forceinline__ float flip_sign(float v, uint32_t bit) {
  return __uint_as_float(__float_as_uint(v) ^ (bit << 31));
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

// Transposing wave reduction.  On entry each lane holds V partial sums
// (V a power of two, V <= 64).  On exit every lane holds in v[0] the
// wave-wide total of value index  value_of_lane(lane).  Each halving step
// exchanges the half of the values the partner keeps, so V values cost
// V-1 shuffles plus log2(64/V) for the remaining plain steps.
template <int V>
__device__ __forceinline__ void wave_transpose_reduce(float (&v)[V], int lane) {
  static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V power of two <= 64");
  int count = V;
  int offset = 32;
#pragma unroll
  for (int step = 0; step < 6; ++step) {
    if (count > 1) {
      const int half = count >> 1;
      const bool upper = (lane & offset) != 0;
#pragma unroll
      for (int i = 0; i < V / 2; ++i) {
        if (i < half) {
          const float send = upper ? v[i] : v[half + i];
          const float keep = upper ? v[half + i] : v[i];
          v[i] = keep + shfl_xor(send, offset);
        }
      }
      count = half;
    } else {
      v[0] += shfl_xor(v[0], offset);
    }
    offset >>= 1;
  }
}

// Lane whose v[0] holds value index t after wave_transpose_reduce<V>.
template <int V>
__device__ __forceinline__ int lane_of_value(int t) {
  int lane = 0;
  int half = V >> 1;
  int offset = 32;
#pragma unroll
  for (int step = 0; step < 6; ++step) {
    if (half >= 1) {
      if (t & half) lane |= offset;
      half >>= 1;
    }
    offset >>= 1;
  }
  return lane;
}

}  // namespace harp
