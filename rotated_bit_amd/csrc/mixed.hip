// Mixed-radix rotation (HARP technical summary §2.1-2.2): the schedule
// b = (b_0, ..., b_{m-1}) with prod b_t = d; stage t applies one b_t x b_t
// block to each group of coordinates that differ only in mixed-radix digit t
// (stride_t = prod_{s<t} b_s); the group index is the coordinate index with
// digit t deleted, c = (i mod stride_t) + stride_t (i div (stride_t b_t)).
// F = B_{m-1} ... B_0 D; F^T = D B_0^T ... B_{m-1}^T.  Blocks arrive expanded
// (Q(theta) G_{b_t}, row-major: output r = sum_j B[r][j] input j).
//
// gfx950 mapping.  One workgroup of 512 threads owns one row, held in LDS as
// float32 (d <= 32768: at most 128 KB).  A stage gives each thread whole
// groups: it reads the group's b_t coordinates into registers, forms the
// b_t outputs from the group's block (read from global memory, where the
// L2 keeps it for the other rows), and writes them back in place; one
// barrier per stage.  The register arrays are sized by the next power of two
// of the radix, a compile-time bound chosen per stage.
#include "launch.hpp"
#include "device_common.hpp"

namespace harp {
namespace {

constexpr int kMixedThreads = 512;

struct MixedPlan {
  int dim;
  int n;
  int radix[HARP_MAX_STAGES];
  int stride[HARP_MAX_STAGES];
  long long offset[HARP_MAX_STAGES];   // first float of stage t's blocks
};

__device__ __forceinline__ float load_elem(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ void store_elem(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_elem(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }

// One stage on the LDS row u: groups c = tid, tid + T, ...  BMAX >= b.
template <int BMAX, bool TRANSPOSE>
__device__ __forceinline__ void mixed_stage(float* u, const float* __restrict__ blk, int dim,
                                            int b, int stride) {
  const int groups = dim / b;
  for (int c = threadIdx.x; c < groups; c += kMixedThreads) {
    const int lo = c % stride;
    const int hi = c / stride;
    const int base = lo + hi * stride * b;
    float xin[BMAX];
#pragma unroll
    for (int j = 0; j < BMAX; ++j) xin[j] = j < b ? u[base + j * stride] : 0.0f;
    const float* B = blk + static_cast<size_t>(c) * b * b;
    for (int r = 0; r < b; ++r) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < BMAX; ++j) {
        if (j < b) {
          const float coef = TRANSPOSE ? B[j * b + r] : B[r * b + j];
          acc = fmaf(coef, xin[j], acc);
        }
      }
      u[base + r * stride] = acc;
    }
  }
}

template <bool TRANSPOSE>
__device__ __forceinline__ void run_stage(float* u, const float* blk, int dim, int b, int stride) {
  if (b <= 2) mixed_stage<2, TRANSPOSE>(u, blk, dim, b, stride);
  else if (b <= 4) mixed_stage<4, TRANSPOSE>(u, blk, dim, b, stride);
  else if (b <= 8) mixed_stage<8, TRANSPOSE>(u, blk, dim, b, stride);
  else if (b <= 16) mixed_stage<16, TRANSPOSE>(u, blk, dim, b, stride);
  else if (b <= 32) mixed_stage<32, TRANSPOSE>(u, blk, dim, b, stride);
  else mixed_stage<64, TRANSPOSE>(u, blk, dim, b, stride);
}

template <bool TRANSPOSE, typename TIn, typename TOut>
__global__ __launch_bounds__(kMixedThreads) void mixed_kernel(
    const TIn* __restrict__ in, TOut* __restrict__ out, const float* __restrict__ blocks,
    const uint32_t* __restrict__ sign, MixedPlan plan) {
  extern __shared__ float u[];
  const int dim = plan.dim;
  const size_t row = blockIdx.x;
  const TIn* src = in + row * dim;
  TOut* dst = out + row * dim;
  for (int i = threadIdx.x; i < dim; i += kMixedThreads) {
    float v = load_elem(src, i);
    if (!TRANSPOSE) v = flip_sign(v, (sign[i >> 5] >> (i & 31)) & 1u);
    u[i] = v;
  }
  __syncthreads();
  for (int q = 0; q < plan.n; ++q) {
    const int t = TRANSPOSE ? plan.n - 1 - q : q;
    run_stage<TRANSPOSE>(u, blocks + plan.offset[t], dim, plan.radix[t], plan.stride[t]);
    __syncthreads();
  }
  for (int i = threadIdx.x; i < dim; i += kMixedThreads) {
    float v = u[i];
    if (TRANSPOSE) v = flip_sign(v, (sign[i >> 5] >> (i & 31)) & 1u);
    store_elem(dst, i, v);
  }
}

MixedPlan make_plan(const harp_mixed_rotation& R) {
  MixedPlan p{};
  p.dim = R.dim;
  p.n = R.n_stages;
  int stride = 1;
  long long off = 0;
  for (int t = 0; t < R.n_stages; ++t) {
    p.radix[t] = R.radix[t];
    p.stride[t] = stride;
    p.offset[t] = off;
    off += static_cast<long long>(R.dim) * R.radix[t];
    stride *= R.radix[t];
  }
  return p;
}

template <bool TRANSPOSE, typename TIn, typename TOut>
hipError_t launch_typed(const harp_mixed_rotation& R, const void* in, void* out, int M,
                        hipStream_t stream) {
  const MixedPlan plan = make_plan(R);
  const size_t shmem = sizeof(float) * static_cast<size_t>(R.dim);
  if (shmem > 65536) {   // rows above 16384 floats: raise the dynamic LDS limit
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&mixed_kernel<TRANSPOSE, TIn, TOut>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shmem));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((mixed_kernel<TRANSPOSE, TIn, TOut>), dim3(M), dim3(kMixedThreads), shmem,
                     stream, static_cast<const TIn*>(in), static_cast<TOut*>(out), R.blocks,
                     R.sign_bits, plan);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rotate_mixed(const harp_mixed_rotation& R, const void* in, int in_dt,
                               void* out, int out_dt, int M, bool transpose,
                               hipStream_t stream) {
  const bool ib = in_dt == HARP_BF16;
  const bool ob = out_dt == HARP_BF16;
  if (transpose) {   // y' is float32
    if (ob) return launch_typed<true, float, uint16_t>(R, in, out, M, stream);
    return launch_typed<true, float, float>(R, in, out, M, stream);
  }
  if (ib && ob) return launch_typed<false, uint16_t, uint16_t>(R, in, out, M, stream);
  if (ib) return launch_typed<false, uint16_t, float>(R, in, out, M, stream);
  if (ob) return launch_typed<false, float, uint16_t>(R, in, out, M, stream);
  return launch_typed<false, float, float>(R, in, out, M, stream);
}

}  // namespace harp
