// F_U^T of one 256-output block inside a product launch (HARP technical
// summary §2.1-2.2: the transposed stages of a b = 256 block-diagonal side,
// widest first, then the sign flip).  Used by the one-row FP4 decode
// product, whose workgroups own whole 16-row tiles of a 256-output block and
// are all resident at once: each
// workgroup stores its y' rows device-coherent, waits for their
// acknowledgement and counts its arrival on the block's counter; the last
// of the block's `arrivals` workgroups reads the block's 256 values back,
// applies stages 7 .. 0 and the signs in LDS, writes y (float32 or bf16) and
// resets the counter, so the counter area is left at zero.
//
// The block's (cos, sin) pairs (or int8 angle codes) and sign words are
// requested by every workgroup before its acknowledgement wait, and the
// angle table of int8-stored angles is evaluated there, so that the last
// workgroup starts its stages one memory round trip earlier.
#pragma once

#include "device_common.hpp"

namespace harp {

struct Fold256Out {
  const float2* cs;        // float32 pairs of the side, or nullptr
  const int8_t* codes;     // int8 angle codes, or nullptr
  float step;              // angle of one code step
  const uint32_t* sign;    // sign bits of the side
  void* y;                 // float32 or bf16 output
};

struct Fold256Regs {
  float2 cf[8];
  int8_t qc[8];
  uint32_t sgn;
};

// Needs at least 256 threads per workgroup; ob is the 256-output block.
template <bool Q8U>
__device__ __forceinline__ void fold256_prefetch(const Fold256Out& out, int ob, int tid,
                                                 Fold256Regs& r) {
  const size_t coff = static_cast<size_t>(ob) * 8 * 128;
  if (tid < 128) {
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if constexpr (Q8U) r.qc[st] = out.codes[coff + st * 128 + tid];
      else r.cf[st] = out.cs[coff + st * 128 + tid];
    }
  }
  r.sgn = tid < 256 ? out.sign[(ob * 256 + tid) >> 5] : 0u;
}

// After this workgroup's y' stores were issued device-coherent: evaluates
// this thread's angle table entry (int8 angles), waits for the stores'
// acknowledgement (and the prefetch), counts the arrival and, in the last
// workgroup of the block, finishes the block.  xl: 256 floats of LDS, tab:
// 256 float2 of LDS, neither read by the workgroup any more.  Every thread
// of the workgroup calls it.
template <int FOLD, bool Q8U>
__device__ __forceinline__ void fold256_finish(const Fold256Out& out, int ob, int tid,
                                               const Fold256Regs& r, const float* yp,
                                               uint32_t* counters, uint32_t arrivals,
                                               float* xl, float2* tab, uint32_t* last) {
  // the angle table entry of this thread, while the stores are in flight
  float2 tv = make_float2(0.0f, 0.0f);
  if constexpr (Q8U) {
    float sn, cn;
    sincosf(fmaf(static_cast<float>((tid & 255) - 128), out.step, 0.785398163397448310f), &sn,
            &cn);
    tv = make_float2(cn, sn);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    *last = __hip_atomic_fetch_add(&counters[ob], 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT) == arrivals - 1u;
  __syncthreads();
  if (!*last) return;
  if (tid < 256) {
    xl[tid] = __hip_atomic_load(&yp[ob * 256 + tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if constexpr (Q8U) tab[tid] = tv;
  }
  __syncthreads();
#pragma unroll
  for (int st = 7; st >= 0; --st) {
    if (tid < 128) {
      float2 c;
      if constexpr (Q8U) c = tab[r.qc[st] + 128];
      else c = r.cf[st];
      const int i = ((tid >> st) << (st + 1)) | (tid & ((1 << st) - 1));
      const int i2 = i | (1 << st);
      const float a = xl[i];
      const float b = xl[i2];
      xl[i] = fmaf(c.x, a, c.y * b);
      xl[i2] = fmaf(c.y, a, -(c.x * b));
    }
    __syncthreads();
  }
  if (tid < 256) {
    const int o = ob * 256 + tid;
    const float v = flip_sign(xl[tid], (r.sgn >> (o & 31)) & 1u);
    if constexpr (FOLD == 1) static_cast<float*>(out.y)[o] = v;
    else static_cast<uint16_t*>(out.y)[o] = f32_to_bf16(v);
  }
  if (tid == 0) __hip_atomic_store(&counters[ob], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace harp
