// Dequant GEMV for decode batches: y'[m][n] = sum_k w_hat[n][k] x~[m][k],
// float32 throughout (w_hat is exact in float32, x~ is not rounded).
//
// gfx950 mapping.  A workgroup (4 waves) owns ROWS output rows and MT rows
// of x~.  Its 256 threads split K into units of KU consecutive inputs
// (2-bit: 16 codes = one word; 4-bit: 16 codes = two words; 3-bit: 32 codes
// = three words); thread t takes units t, t+256, ...  For each unit it loads
// x~ once (coalesced across threads) and streams the unit's words of all
// ROWS rows, so every weight byte is read once and x~ is read once per
// workgroup.  The workgroup's fp16 scales and zeros are staged in LDS with
// one coalesced pass.  Per group the product is factored as
//     sum_k (q_k - z) s x~_k = s (sum_k q_k x~_k - z sum_k x~_k),
// which leaves one convert and MT fused multiply-adds per code.  The
// ROWS*MT partial sums are combined with a transposing wave reduction and
// one LDS pass across the four waves, in a fixed order (bitwise
// deterministic).
#include "launch.hpp"
#include "unpack.hpp"

namespace harp {
namespace {

template <int BITS> struct GemvUnit;
template <> struct GemvUnit<2> { static constexpr int KU = 16, NW = 1; };
template <> struct GemvUnit<3> { static constexpr int KU = 32, NW = 3; };
template <> struct GemvUnit<4> { static constexpr int KU = 16, NW = 2; };

// Codes of one unit as floats.  2- and 4-bit codes are masked four at a
// time into byte lanes so each becomes one byte-to-float convert.
template <int BITS, int NW, int KU>
__device__ __forceinline__ void unit_codes(const uint32_t (&w)[NW], float (&q)[KU]) {
  if constexpr (BITS == 2) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t m = opaque((w[0] >> (2 * t)) & 0x03030303u);  // codes t, t+4, t+8, t+12
#pragma unroll
      for (int i = 0; i < 4; ++i) q[t + 4 * i] = static_cast<float>((m >> (8 * i)) & 0xffu);
    }
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t m = opaque((w[h] >> (4 * t)) & 0x0f0f0f0fu);  // codes 8h+t, +2, +4, +6
#pragma unroll
        for (int i = 0; i < 4; ++i)
          q[8 * h + t + 2 * i] = static_cast<float>((m >> (8 * i)) & 0xffu);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < KU; ++j) q[j] = static_cast<float>(code_at<BITS, NW>(w, j));
  }
}

// One K unit of the operands: x~ for MT rows, the unit's words, scales and
// zeros for ROWS weight rows.  Loaded as a batch so that every load of a
// unit is in flight before the first use.
template <int BITS, int MT, int ROWS>
struct UnitData {
  static constexpr int KU = GemvUnit<BITS>::KU;
  static constexpr int NW = GemvUnit<BITS>::NW;
  float xv[MT][KU];
  uint32_t w[ROWS][NW];
};

template <int BITS, int MT, int ROWS>
__device__ __forceinline__ void load_unit(UnitData<BITS, MT, ROWS>& d, int u,
                                          const uint32_t* __restrict__ qw,
                                          const float* __restrict__ xt, int N,
                                          int K, int M, int row0, int m0,
                                          size_t WPR) {
  constexpr int KU = GemvUnit<BITS>::KU;
  constexpr int NW = GemvUnit<BITS>::NW;
  const int k0 = u * KU;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int n = min(row0 + r, N - 1);
    const uint32_t* wp = qw + static_cast<size_t>(n) * WPR + static_cast<size_t>(u) * NW;
    if constexpr (NW == 2) {
      const uint2 v2 = *reinterpret_cast<const uint2*>(wp);
      d.w[r][0] = v2.x;
      d.w[r][1] = v2.y;
    } else {
#pragma unroll
      for (int i = 0; i < NW; ++i) d.w[r][i] = wp[i];
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int mm = min(m0 + m, M - 1);     // rows past M: loaded, never stored
    const float4* p = reinterpret_cast<const float4*>(xt + static_cast<size_t>(mm) * K + k0);
#pragma unroll
    for (int c = 0; c < KU / 4; ++c) {
      const float4 f = p[c];
      d.xv[m][4 * c + 0] = f.x;
      d.xv[m][4 * c + 1] = f.y;
      d.xv[m][4 * c + 2] = f.z;
      d.xv[m][4 * c + 3] = f.w;
    }
  }
}

// s_lds / z_lds: the workgroup's scales and zeros, [ROWS][G] fp16 bits.
template <int BITS, int MT, int ROWS>
__device__ __forceinline__ void compute_unit(const UnitData<BITS, MT, ROWS>& d,
                                             int u, const uint16_t* s_lds,
                                             const uint16_t* z_lds, int G,
                                             float (&acc)[ROWS * MT]) {
  constexpr int KU = GemvUnit<BITS>::KU;
  constexpr int NW = GemvUnit<BITS>::NW;
  float sx[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float t = 0.0f;
#pragma unroll
    for (int j = 0; j < KU; ++j) t += d.xv[m][j];
    sx[m] = t;
  }
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    float q[KU];
    unit_codes<BITS, NW, KU>(d.w[r], q);
    float dot[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) dot[m] = 0.0f;
#pragma unroll
    for (int j = 0; j < KU; ++j) {
#pragma unroll
      for (int m = 0; m < MT; ++m) dot[m] = fmaf(q[j], d.xv[m][j], dot[m]);
    }
    const int gi = r * G + u * KU / kGroup;
    const float s = f16_to_f32(s_lds[gi]);
    const float z = f16_to_f32(z_lds[gi]);
#pragma unroll
    for (int m = 0; m < MT; ++m)
      acc[r * MT + m] = fmaf(s, fmaf(-z, sx[m], dot[m]), acc[r * MT + m]);
  }
}

template <int BITS, int MT, int ROWS>
__global__ __launch_bounds__(256) void gemv_kernel(
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint16_t* __restrict__ zr, const float* __restrict__ xt,
    float* __restrict__ yt, int N, int K, int M) {
  using U = GemvUnit<BITS>;
  constexpr int KU = U::KU;
  constexpr int V = ROWS * MT;
  __shared__ float red[4][kWave];
  extern __shared__ uint16_t sz_lds[];   // [2][ROWS][G]: scales, then zeros

  const int NU = K / KU;
  const size_t WPR = static_cast<size_t>(K) * BITS / 32;
  const int G = K / kGroup;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int row0 = blockIdx.x * ROWS;
  const int m0 = blockIdx.y * MT;

  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.0f;

  // First unit's operands in flight, then this workgroup's scales and zeros
  // (ROWS consecutive rows = one contiguous run of ROWS*G halves) to LDS.
  int u = tid;
  UnitData<BITS, MT, ROWS> cur;
  if (u < NU) load_unit<BITS, MT, ROWS>(cur, u, qw, xt, N, K, M, row0, m0, WPR);
  {
    const int rows = min(ROWS, N - row0);
    const size_t base = static_cast<size_t>(row0) * G;
    for (int i = tid; i < ROWS * G; i += 256) {
      const bool ok = i < rows * G;
      sz_lds[i] = ok ? sc[base + i] : uint16_t(0);
      sz_lds[ROWS * G + i] = ok ? zr[base + i] : uint16_t(0);
    }
  }
  __syncthreads();
  const uint16_t* s_lds = sz_lds;
  const uint16_t* z_lds = sz_lds + ROWS * G;

  // Software pipeline over this thread's K units: the next unit's loads
  // are issued before the current unit is computed.
  if (u < NU) {
    for (;;) {
      const int un = u + 256;
      if (un < NU) {
        UnitData<BITS, MT, ROWS> nxt;
        load_unit<BITS, MT, ROWS>(nxt, un, qw, xt, N, K, M, row0, m0, WPR);
        compute_unit<BITS, MT, ROWS>(cur, u, s_lds, z_lds, G, acc);
        cur = nxt;
        u = un;
      } else {
        compute_unit<BITS, MT, ROWS>(cur, u, s_lds, z_lds, G, acc);
        break;
      }
    }
  }

  wave_transpose_reduce<V>(acc, lane);
  red[wave][lane] = acc[0];
  __syncthreads();
  if (tid < V) {
    const int src = lane_of_value<V>(tid);
    const float total = ((red[0][src] + red[1][src]) + red[2][src]) + red[3][src];
    const int r = tid / MT;
    const int m = tid - r * MT;
    const int n = row0 + r;
    if (n < N && m0 + m < M) yt[static_cast<size_t>(m0 + m) * N + n] = total;
  }
}

template <int BITS, int MT, int ROWS>
hipError_t launch_cfg(const harp_qweight& W, const float* xt, float* yt, int M,
                      hipStream_t stream) {
  const dim3 grid((W.N + ROWS - 1) / ROWS, (M + MT - 1) / MT);
  const size_t shmem = sizeof(uint16_t) * 2 * ROWS * (W.K / kGroup);
  hipLaunchKernelGGL((gemv_kernel<BITS, MT, ROWS>), grid, dim3(256), shmem, stream,
                     W.qweight, W.scale, W.zero, xt, yt, W.N, W.K, M);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const harp_qweight& W, const float* xt, float* yt, int M,
                       hipStream_t stream) {
  // MT x~ rows per pass (grid.y passes); more rows per pass would spill
  // the double-buffered operands.
  if (M == 1) return launch_cfg<BITS, 1, 8>(W, xt, yt, M, stream);
  if (M == 2) return launch_cfg<BITS, 2, 16>(W, xt, yt, M, stream);
  return launch_cfg<BITS, 4, 8>(W, xt, yt, M, stream);
}

}  // namespace

hipError_t launch_gemv(const harp_qweight& W, const float* xt, float* yt, int M,
                       hipStream_t stream) {
  switch (W.bits) {
    case 2: return launch_bits<2>(W, xt, yt, M, stream);
    case 3: return launch_bits<3>(W, xt, yt, M, stream);
    case 4: return launch_bits<4>(W, xt, yt, M, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace harp
