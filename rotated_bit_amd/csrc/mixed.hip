// Mixed-radix rotation (HARP technical summary §2.1-2.2): the schedule
// b = (b_0, ..., b_{m-1}) with prod b_t = d; stage t applies one b_t x b_t
// block to each group of coordinates that differ only in mixed-radix digit t
// (stride_t = prod_{s<t} b_s); the group index is the coordinate index with
// digit t deleted, c = (i mod stride_t) + stride_t (i div (stride_t b_t)).
// F = B_{m-1} ... B_0 D; F^T = D B_0^T ... B_{m-1}^T.  Blocks arrive expanded
// (Q(theta) G_{b_t}, row-major: output r = sum_j B[r][j] input j).
//
// gfx950 mapping.  A group of radix b takes the next power of two of b
// lanes of one wave, lane r forming output r from the group's inputs and
// row (or column) r of its block, so that a wave's coefficient loads are
// contiguous.  The stages run one launch each over the whole chip, in place
// in a float32 buffer (a group's inputs and outputs are the same
// coordinates, and groups are disjoint): the output itself for a float32
// output, the caller's workspace for a bf16 one, whose last stage writes
// the output.  Each lane keeps its block row in registers for a tile of
// rows.  For small batches the leading stages whose radices multiply to at
// most 512 act inside contiguous sub-rows and run as one launch, one
// workgroup per sub-row in LDS.  A bf16 output without a workspace falls
// back to one workgroup of 512 threads per row, the row held in LDS as
// float32 (d <= 32768: at most 128 KB), one barrier per stage, the blocks
// streaming from global memory where the L2 keeps them for the other rows.
// Register arrays are sized by the next power of two of the radix, a
// compile-time bound chosen per stage.
#include "launch.hpp"
#include "device_common.hpp"

#include <algorithm>
#include <type_traits>

namespace harp {
namespace {

constexpr int kMixedThreads = 512;
constexpr int kStageMaxRows = 32;     // rows per workgroup of a stage launch
constexpr int kStageTargetWaves = 8192;  // waves a stage launch aims for
constexpr int kStageWideM = 64;         // batches from this size use 8-wave workgroups
constexpr int kRowFormMaxDim = 16384;   // bf16 outputs: row form limits (see launch_typed)
constexpr int kRowFormMaxRadix = 16;

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

// Lane mapping of a stage: BMAX lanes per group (BMAX the next power of two
// of the radix b, at most one wave), lane r of a group forming output r from
// all b inputs of the group and row r of its block (column r for F^T).
// Neighbouring lanes then read neighbouring block rows (or columns), so the
// coefficient loads of a wave are contiguous.
template <int BMAX>
struct StageLanes {
  static constexpr int PER_WAVE = kWave / BMAX;   // groups per wave
  int sub, r;                                     // group slot in the wave, output row
  __device__ explicit StageLanes(int lane) : sub(lane / BMAX), r(lane % BMAX) {}
};

// Lane r's coefficients: row r of the block B (b x b, row-major), or
// column r for F^T; zero beyond b.  Neighbouring lanes of a column read
// neighbouring floats.  A row is read as 16-byte vectors, which gfx950
// loads from any 4-byte boundary, and a scalar tail of b mod 4 floats, so
// that no load leaves the row.
template <int BMAX, bool TRANSPOSE>
__device__ __forceinline__ void load_coef(const float* __restrict__ B, int b, int r,
                                          float (&coef)[BMAX]) {
  if constexpr (!TRANSPOSE && BMAX >= 4) {
    const float* row = B + r * b;
#pragma unroll
    for (int j = 0; j < BMAX; j += 4) {
      if (j + 4 <= b) {
        float4 v;
        __builtin_memcpy(&v, row + j, sizeof(v));
        coef[j] = v.x;
        coef[j + 1] = v.y;
        coef[j + 2] = v.z;
        coef[j + 3] = v.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) coef[j + i] = j + i < b ? row[j + i] : 0.0f;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < BMAX; ++j)
      coef[j] = j < b ? (TRANSPOSE ? B[j * b + r] : B[r * b + j]) : 0.0f;
  }
}

// One stage on the LDS row u (one workgroup per row).
template <int BMAX, bool TRANSPOSE>
__device__ __forceinline__ void mixed_stage(float* u, const float* __restrict__ blk, int dim,
                                            int b, int stride) {
  const StageLanes<BMAX> ln(threadIdx.x & (kWave - 1));
  const int wave = threadIdx.x >> 6;
  const int groups = dim / b;
  constexpr int kUnits = (kMixedThreads / kWave) * StageLanes<BMAX>::PER_WAVE;
  // every group of a wave is read before any is written (one wave, program
  // order; the groups of a wave are disjoint from other waves' groups)
  for (int c0 = wave * StageLanes<BMAX>::PER_WAVE; c0 < groups; c0 += kUnits) {
    const int c = c0 + ln.sub;
    const bool act = c < groups && ln.r < b;
    const int cc = min(c, groups - 1);
    const int lo = cc % stride;
    const int hi = cc / stride;
    const int base = lo + hi * stride * b;
    float xin[BMAX];
#pragma unroll
    for (int j = 0; j < BMAX; ++j) xin[j] = j < b ? u[base + j * stride] : 0.0f;
    const float* B = blk + static_cast<size_t>(cc) * b * b;
    const int rr = min(ln.r, b - 1);
    float acc = 0.0f;
    if (!TRANSPOSE && b == BMAX) {   // whole aligned rows as vectors
      float coef[BMAX];
      load_coef<BMAX, TRANSPOSE>(B, b, rr, coef);
#pragma unroll
      for (int j = 0; j < BMAX; ++j) acc = fmaf(coef[j], xin[j], acc);
    } else {
#pragma unroll
      for (int j = 0; j < BMAX; ++j)
        if (j < b) acc = fmaf(TRANSPOSE ? B[j * b + rr] : B[rr * b + j], xin[j], acc);
    }
    if (act) u[base + ln.r * stride] = acc;
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

// One stage over global memory: groups spread over blockIdx.x (WAVES waves
// per workgroup), a tile of `rows` rows over blockIdx.y.  Lane (group slot, r) loads coordinate
// o = base + r stride of each row, which is also the coordinate it writes,
// so running in place needs no ordering between lanes.  The wave passes the
// group's inputs through its own LDS slot (one wave: in-order LDS), and each
// lane reads its group's b inputs back as vectors; its block row (column for
// F^T) stays in registers for the whole tile.  src is the input of the first
// stage (sign flip on read for the forward map) or dst itself; the last
// stage of the transposed map flips signs on write.
constexpr int kStageRB = 8;   // rows per load batch

template <int BMAX>
__device__ __forceinline__ void read_group(const float* p, float (&xin)[BMAX]) {
  if constexpr (BMAX == 2) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    xin[0] = v.x;
    xin[1] = v.y;
  } else {
#pragma unroll
    for (int j = 0; j < BMAX; j += 4) {
      const float4 v = *reinterpret_cast<const float4*>(p + j);
      xin[j] = v.x;
      xin[j + 1] = v.y;
      xin[j + 2] = v.z;
      xin[j + 3] = v.w;
    }
  }
}

template <int BMAX, int WAVES, bool TRANSPOSE, typename TIn, typename TOut>
__global__ __launch_bounds__(WAVES * kWave) void mixed_stage_kernel(
    const TIn* src, TOut* dst, const float* __restrict__ blk,
    const uint32_t* __restrict__ sign, int dim, int b, int stride, int M, int rows,
    int sign_in, int sign_out) {
  __shared__ __attribute__((aligned(16))) float xsw[WAVES][kStageRB][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  float (*xs)[kWave] = xsw[wave];
  const int groups = dim / b;
  const StageLanes<BMAX> ln(lane);
  const int c = (blockIdx.x * WAVES + wave) * StageLanes<BMAX>::PER_WAVE + ln.sub;
  const bool act = c < groups && ln.r < b;
  const int cc = min(c, groups - 1);
  const int rr = min(ln.r, b - 1);
  const int lo = cc % stride;
  const int hi = cc / stride;
  const int o = lo + hi * stride * b + rr * stride;
  const float* B = blk + static_cast<size_t>(cc) * b * b;
  float coef[BMAX];
  load_coef<BMAX, TRANSPOSE>(B, b, rr, coef);
  const uint32_t sgn = (sign[o >> 5] >> (o & 31)) & 1u;
  const uint32_t sgn_in = sign_in ? sgn : 0u;
  const uint32_t sgn_out = sign_out ? sgn : 0u;
  const float* grp = &xs[0][ln.sub * BMAX];

  const int m0 = blockIdx.y * rows;
  const int m1 = min(M, m0 + rows);
  for (int mb = m0; mb < m1; mb += kStageRB) {
    float v[kStageRB];
#pragma unroll
    for (int k = 0; k < kStageRB; ++k) {
      const int m = min(mb + k, m1 - 1);
      v[k] = act ? flip_sign(load_elem(src + static_cast<size_t>(m) * dim, o), sgn_in) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kStageRB; ++k) xs[k][lane] = v[k];
#pragma unroll
    for (int k = 0; k < kStageRB; ++k) {
      float xin[BMAX];
      read_group<BMAX>(grp + k * kWave, xin);
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < BMAX; ++j) acc = fmaf(coef[j], xin[j], acc);
      if (act && mb + k < m1)
        store_elem(dst, static_cast<size_t>(mb + k) * dim + o, flip_sign(acc, sgn_out));
    }
  }
}

// Stages 0 .. seg_n - 1 act inside contiguous sub-rows of G = b_0 ... b_{seg_n-1}
// elements (sub-row h of a row holds the groups h G / b_t ..., whose blocks
// start h G b_t floats into stage t's).  One workgroup takes one sub-row
// into LDS and applies those stages (ascending for F, descending for F^T);
// with seg_n = n and G = dim it rotates a whole row.  The sign flip is
// applied on load for F (these stages come first) and on store for F^T
// (they come last).
template <bool TRANSPOSE, typename TIn, typename TOut>
__global__ __launch_bounds__(kMixedThreads) void mixed_kernel(
    const TIn* __restrict__ in, TOut* __restrict__ out, const float* __restrict__ blocks,
    const uint32_t* __restrict__ sign, MixedPlan plan, int seg_n, int G) {
  extern __shared__ float u[];
  const int dim = plan.dim;
  const int subs = dim / G;
  const size_t row = blockIdx.x / subs;
  const int h = blockIdx.x - static_cast<int>(row) * subs;
  const size_t base = row * dim + static_cast<size_t>(h) * G;
  const TIn* src = in + base;
  TOut* dst = out + base;
  for (int i = threadIdx.x; i < G; i += kMixedThreads) {
    float v = load_elem(src, i);
    const int gi = h * G + i;
    if (!TRANSPOSE) v = flip_sign(v, (sign[gi >> 5] >> (gi & 31)) & 1u);
    u[i] = v;
  }
  __syncthreads();
  for (int q = 0; q < seg_n; ++q) {
    const int t = TRANSPOSE ? seg_n - 1 - q : q;
    const float* blk = blocks + plan.offset[t] + static_cast<size_t>(h) * G * plan.radix[t];
    run_stage<TRANSPOSE>(u, blk, G, plan.radix[t], plan.stride[t]);
    __syncthreads();
  }
  for (int i = threadIdx.x; i < G; i += kMixedThreads) {
    float v = u[i];
    const int gi = h * G + i;
    if (TRANSPOSE) v = flip_sign(v, (sign[gi >> 5] >> (gi & 31)) & 1u);
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

template <int BMAX, int WAVES, bool TRANSPOSE, typename TIn, typename TOut>
hipError_t launch_stage_waves(const TIn* src, TOut* dst, const float* blk, const uint32_t* sign,
                              int dim, int b, int stride, int M, bool sign_in, bool sign_out,
                              hipStream_t stream) {
  const int groups = dim / b;
  const int per_wg = WAVES * StageLanes<BMAX>::PER_WAVE;
  const int gtiles = (groups + per_wg - 1) / per_wg;
  // rows per workgroup: enough workgroups to fill the chip, block rows
  // reused over as many rows as that allows
  const int rows =
      std::max(1, std::min(kStageMaxRows, M * gtiles * WAVES / kStageTargetWaves));
  const dim3 grid(gtiles, (M + rows - 1) / rows);
  hipLaunchKernelGGL((mixed_stage_kernel<BMAX, WAVES, TRANSPOSE, TIn, TOut>), grid,
                     dim3(WAVES * kWave), 0, stream, src, dst, blk, sign, dim, b, stride, M,
                     rows, sign_in ? 1 : 0, sign_out ? 1 : 0);
  return hipGetLastError();
}

// Small batches: one-wave workgroups, spread over as many compute units as
// there are groups.  Larger batches: eight waves on neighbouring groups
// share a compute unit, so that their strided rows share cache lines.
template <int BMAX, bool TRANSPOSE, typename TIn, typename TOut>
hipError_t launch_stage_bmax(const TIn* src, TOut* dst, const float* blk, const uint32_t* sign,
                             int dim, int b, int stride, int M, bool sign_in, bool sign_out,
                             hipStream_t stream) {
  if (M < kStageWideM)
    return launch_stage_waves<BMAX, 1, TRANSPOSE, TIn, TOut>(src, dst, blk, sign, dim, b, stride,
                                                             M, sign_in, sign_out, stream);
  return launch_stage_waves<BMAX, 8, TRANSPOSE, TIn, TOut>(src, dst, blk, sign, dim, b, stride, M,
                                                           sign_in, sign_out, stream);
}

template <bool TRANSPOSE, typename TIn, typename TOut>
hipError_t launch_stage(const TIn* src, TOut* dst, const float* blk, const uint32_t* sign,
                        int dim, int b, int stride, int M, bool sign_in, bool sign_out,
                        hipStream_t stream) {
#define HARP_STAGE(BM) \
  launch_stage_bmax<BM, TRANSPOSE, TIn, TOut>(src, dst, blk, sign, dim, b, stride, M, sign_in, \
                                              sign_out, stream)
  if (b <= 2) return HARP_STAGE(2);
  if (b <= 4) return HARP_STAGE(4);
  if (b <= 8) return HARP_STAGE(8);
  if (b <= 16) return HARP_STAGE(16);
  if (b <= 32) return HARP_STAGE(32);
  return HARP_STAGE(64);
#undef HARP_STAGE
}

// The leading stages whose radices multiply to at most kSegMaxLen act
// inside contiguous sub-rows of that length: for small batches they run as
// one launch, one workgroup per sub-row in LDS, when there are at least two
// of them.
constexpr int kSegMaxLen = 512;

int lead_segment(const MixedPlan& p, int* G) {
  int g = 1, k = 0;
  while (k < p.n && g * p.radix[k] <= kSegMaxLen) g *= p.radix[k++];
  *G = g;
  return k;
}

template <bool TRANSPOSE, typename TIn, typename TOut>
hipError_t launch_rows(const MixedPlan& plan, int seg_n, int G, const TIn* in, TOut* out,
                       const float* blocks, const uint32_t* sign, int M, hipStream_t stream) {
  const size_t shmem = sizeof(float) * static_cast<size_t>(G);
  if (shmem > 65536) {   // rows above 16384 floats: raise the dynamic LDS limit
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&mixed_kernel<TRANSPOSE, TIn, TOut>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shmem));
    if (e != hipSuccess) return e;
  }
  const dim3 grid(static_cast<unsigned>(static_cast<size_t>(M) * (plan.dim / G)));
  hipLaunchKernelGGL((mixed_kernel<TRANSPOSE, TIn, TOut>), grid, dim3(kMixedThreads), shmem,
                     stream, in, out, blocks, sign, plan, seg_n, G);
  return hipGetLastError();
}

// Launch by launch: the fused leading segment (first for F, last for F^T)
// and one launch per other stage.  The first launch reads the input, the
// others run in place in the float32 buffer ws (the output itself for a
// float32 output), and the last writes the output.
template <bool TRANSPOSE, typename TIn, typename TOut>
hipError_t launch_by_stage(const harp_mixed_rotation& R, const void* in, float* ws, TOut* out,
                           int M, hipStream_t stream) {
  const MixedPlan plan = make_plan(R);
  int G = 1;
  const int k = lead_segment(plan, &G);
  // one workgroup per sub-row fetches its sub-row's blocks for one row only:
  // large batches keep the per-stage launches, which reuse block rows
  // across a tile of rows
  const bool seg = k >= 2 && M < kStageWideM;
  const int nops = seg ? plan.n - k + 1 : plan.n;
  const TIn* src = static_cast<const TIn*>(in);
  for (int q = 0; q < nops; ++q) {
    const bool first = q == 0;
    const bool last = q == nops - 1;
    const bool is_seg = seg && (TRANSPOSE ? last : first);
    hipError_t e;
    if (is_seg) {
      if (first && last)
        e = launch_rows<TRANSPOSE, TIn, TOut>(plan, k, G, src, out, R.blocks, R.sign_bits, M,
                                              stream);
      else if (first)
        e = launch_rows<TRANSPOSE, TIn, float>(plan, k, G, src, ws, R.blocks, R.sign_bits, M,
                                               stream);
      else
        e = launch_rows<TRANSPOSE, float, TOut>(plan, k, G, ws, out, R.blocks, R.sign_bits, M,
                                                stream);
    } else {
      const int t = TRANSPOSE ? plan.n - 1 - q : (seg ? k + q - 1 : q);
      const float* blk = R.blocks + plan.offset[t];
      const bool flip_in = first && !TRANSPOSE;
      const bool flip_out = last && TRANSPOSE;
      if (first && last)
        e = launch_stage<TRANSPOSE, TIn, TOut>(src, out, blk, R.sign_bits, plan.dim,
                                               plan.radix[t], plan.stride[t], M, flip_in,
                                               flip_out, stream);
      else if (first)
        e = launch_stage<TRANSPOSE, TIn, float>(src, ws, blk, R.sign_bits, plan.dim,
                                                plan.radix[t], plan.stride[t], M, flip_in,
                                                flip_out, stream);
      else if (last)
        e = launch_stage<TRANSPOSE, float, TOut>(ws, out, blk, R.sign_bits, plan.dim,
                                                 plan.radix[t], plan.stride[t], M, flip_in,
                                                 flip_out, stream);
      else
        e = launch_stage<TRANSPOSE, float, float>(ws, ws, blk, R.sign_bits, plan.dim,
                                                  plan.radix[t], plan.stride[t], M, flip_in,
                                                  flip_out, stream);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <bool TRANSPOSE, typename TIn, typename TOut>
hipError_t launch_typed(const harp_mixed_rotation& R, const void* in, void* out, int M,
                        float* workspace, hipStream_t stream) {
  if constexpr (std::is_same<TOut, float>::value) {
    float* o = static_cast<float*>(out);
    return launch_by_stage<TRANSPOSE, TIn, float>(R, in, o, o, M, stream);
  } else {
    // With a workspace the stages run over the whole chip, except for large
    // batches of small power-of-two-ish radices on rows that leave room for
    // two workgroups per CU, where the one-workgroup-per-row form (blocks
    // reused from the L2 across rows, one HBM pass) was measured faster.
    int rmax = 0;
    for (int t = 0; t < R.n_stages; ++t) rmax = std::max(rmax, R.radix[t]);
    const bool row_form = M >= kStageWideM && R.dim <= kRowFormMaxDim && rmax <= kRowFormMaxRadix;
    if (workspace != nullptr && !row_form)
      return launch_by_stage<TRANSPOSE, TIn, TOut>(R, in, workspace, static_cast<TOut*>(out), M,
                                                   stream);
    const MixedPlan plan = make_plan(R);
    return launch_rows<TRANSPOSE, TIn, TOut>(plan, plan.n, plan.dim, static_cast<const TIn*>(in),
                                             static_cast<TOut*>(out), R.blocks, R.sign_bits, M,
                                             stream);
  }
}

}  // namespace

hipError_t launch_rotate_mixed(const harp_mixed_rotation& R, const void* in, int in_dt,
                               void* out, int out_dt, int M, bool transpose,
                               float* workspace, hipStream_t stream) {
  const bool ib = in_dt == HARP_BF16;
  const bool ob = out_dt == HARP_BF16;
  float* ws = workspace;
  if (transpose) {   // y' is float32
    if (ob) return launch_typed<true, float, uint16_t>(R, in, out, M, ws, stream);
    return launch_typed<true, float, float>(R, in, out, M, ws, stream);
  }
  if (ib && ob) return launch_typed<false, uint16_t, uint16_t>(R, in, out, M, ws, stream);
  if (ib) return launch_typed<false, uint16_t, float>(R, in, out, M, ws, stream);
  if (ob) return launch_typed<false, float, uint16_t>(R, in, out, M, ws, stream);
  return launch_typed<false, float, float>(R, in, out, M, ws, stream);
}

}  // namespace harp
