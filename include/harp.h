/*
 * harp.h -- C ABI of libharp: the inference hot path of HARP, a two-sided
 * learnable structured orthogonal processor around a low-bit linear layer,
 *
 *     y = U . deq(Wq) . V^T . x        with  V^T = F_V,  U = F_U^T.
 *
 * Source: "HARP: Hadamard-Preconditioned Adaptive Rotation Processor for
 * Extreme LLM Quantization" (gist.science technical summary of arXiv
 * 2605.29843).  Technical summary §2.4 describes the processor as a
 * drop-in replacement for the fixed randomized-Hadamard pre-processing of
 * QuIP#/QTIP pipelines; this ABI mirrors that role: rotate in, quantized
 * matmul, rotate out, plus the whole linear in one call.
 *
 * One side's rotation (technical summary §2.1-2.2), for a vector of length
 * dim split into dim/b independent blocks of size b = 2^L:
 *
 *     F = blockdiag_j( B^(j)_{L-1} ... B^(j)_0 ) . D
 *
 * D is a +-1 diagonal; stage s of block j pairs coordinates (i, i + 2^s) for
 * every i with bit s clear and applies [[c, s], [s, -c]] with
 * (c, s) = (cos t, sin t) of that pair's angle.  This is the page's
 * Hadamard-preconditioned block Q(phi) G_2 with t = pi/4 + phi, so zero
 * angles phi give the randomized Hadamard transform (technical summary
 * §2.2).  The pair's index within the stage is i with bit s deleted.
 *
 * Weights (stand-in quantizer; the pages leave the codebook open): per
 * output row n and per group g of 64 consecutive inputs,
 *     w_hat[n][k] = (q[n][k] - z[n][g]) * s[n][g],   g = k / 64,
 * with q a B-bit code, s an fp16 scale and z an integer-valued fp16 zero.
 *
 * Conventions for every call
 * --------------------------
 * Ownership: the caller owns every buffer.  The library never allocates or
 *   frees device memory and keeps no state beyond a per-thread HIP error.
 * Memory: all data pointers are device pointers, 16-byte aligned, row-major,
 *   without padding.  Outputs must not overlap inputs.
 * Streams: work is enqueued on `stream` (a hipStream_t; NULL is the null
 *   stream); calls return once it is enqueued.
 * Errors: arguments are checked before anything is launched.  A failed check
 *   returns its status, launches nothing and leaves the outputs untouched.
 *   A failed launch returns HARP_ERR_HIP; harp_last_hip_error() then holds
 *   the hipError_t.  No C++ exception crosses this ABI.
 * Empty input: M == 0 is valid and does nothing; data pointers may then be
 *   NULL (the structure pointers and their fields are still checked).
 * Determinism: results are bitwise reproducible run to run for identical
 *   inputs and launch configuration (no floating-point atomics).
 * Threads: every call is thread-safe; calls on different streams may run
 *   concurrently.
 */
#ifndef HARP_H
#define HARP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum harp_status {
  HARP_OK = 0,
  HARP_ERR_NULL = 1,         /* a required pointer is NULL                    */
  HARP_ERR_SHAPE = 2,        /* inconsistent or out-of-range dimension/value  */
  HARP_ERR_DTYPE = 3,        /* dtype value not in harp_dtype                 */
  HARP_ERR_ALIGN = 4,        /* a data pointer is not 16-byte aligned         */
  HARP_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than required       */
  HARP_ERR_UNSUPPORTED = 6,  /* bits not in {2,3,4}, group != 64, b > 8192    */
  HARP_ERR_HIP = 7           /* a HIP launch failed; see harp_last_hip_error  */
} harp_status;

typedef enum harp_dtype {
  HARP_F32 = 0,              /* IEEE binary32                                 */
  HARP_BF16 = 1              /* bfloat16, stored as uint16 bit patterns       */
} harp_dtype;

typedef void *harp_stream;   /* hipStream_t */

/* Largest dimension, block and batch the library accepts. */
#define HARP_MAX_DIM 262144
#define HARP_MAX_BLOCK 8192
#define HARP_MAX_M 65536

/*
 * One side of the processor (technical summary §2.1-2.2).
 *   dim        vector length (K on the input side, N on the output side)
 *   block      b: power of two, 2 <= b <= 8192, dim % b == 0
 *   cs         [dim/b][log2 b][b/2][2] float32: (cos t, sin t) for block j,
 *              stage s, pair index c (i with bit s deleted); NULL when the
 *              angles are given as phi_codes
 *   sign_bits  [ceil(dim/32)] uint32: bit i of word i/32 set means D_ii = -1
 *   phi_codes  [dim/b][log2 b][b/2] int8, same index order as cs: the angles
 *              stored in eight bits (technical summary §2.4, storage of the
 *              HARP parameters), t = pi/4 + phi_codes * phi_step; every int8
 *              value is valid; NULL when cs is given
 *   phi_step   float32 step of phi_codes, finite; not read when cs is given
 * Exactly one of cs and phi_codes is set (neither: HARP_ERR_NULL, both:
 * HARP_ERR_SHAPE).  With phi_codes the kernels evaluate cos t and sin t in
 * float32 for the 256 code values.  All pointers are device memory owned by
 * the caller, 16-byte aligned, and only read.
 */
typedef struct harp_rotation {
  int32_t dim;
  int32_t block;
  const float *cs;
  const uint32_t *sign_bits;
  const int8_t *phi_codes;
  float phi_step;
} harp_rotation;

/*
 * One side with a mixed-radix schedule (technical summary §2.1: stage t
 * applies a block-diagonal orthogonal matrix to groups of coordinates a
 * stride apart; radices need not be powers of two, e.g. 5120 = 8*8*8*5*2).
 *   dim        prod radix[0 .. n_stages-1], at most HARP_MAX_MIXED_DIM
 *   n_stages   1 .. HARP_MAX_STAGES;  radix[t] in 2 .. HARP_MAX_RADIX
 *   blocks     float32, the stages one after the other; stage t holds
 *              [dim / b_t][b_t][b_t] row-major blocks B (output r =
 *              sum_j B[r][j] input j) for the groups c = (i mod s_t) +
 *              s_t (i div (s_t b_t)) of the coordinates i that differ only in
 *              mixed-radix digit t, s_t = b_0 ... b_{t-1}.  The blocks are
 *              the expanded learnable blocks Q(theta) G_{b_t} (technical
 *              summary §2.2: Cayley map times the fixed mixer, or the QR
 *              factor of a fixed Gaussian for radices that are not powers of
 *              two); the library only applies them.
 *   sign_bits  [ceil(dim/32)] uint32: bit i set means D_ii = -1
 * Device pointers owned by the caller, 16-byte aligned, only read.
 */
#define HARP_MAX_STAGES 16
#define HARP_MAX_RADIX 64
#define HARP_MAX_MIXED_DIM 32768
typedef struct harp_mixed_rotation {
  int32_t dim;
  int32_t n_stages;
  int32_t radix[HARP_MAX_STAGES];
  const float *blocks;
  const uint32_t *sign_bits;
} harp_mixed_rotation;

/*
 * Packed low-bit weight W_hat [N][K] (out x in).
 *   bits     2, 3 or 4;  group must be 64;  K % 64 == 0
 *   qweight  [N][K*bits/32] uint32.  bits 2 and 4: code k in word k/(32/bits)
 *            at bits bits*(k % (32/bits)), least significant first.  bits 3:
 *            each run of 32 codes is a 96-bit little-endian integer in three
 *            words (first word = bits 0..31), code k of the run at bits 3k.
 *   scale    [N][K/64] fp16 bit patterns
 *   zero     [N][K/64] fp16 bit patterns holding integers in [0, 2^bits-1]
 */
typedef struct harp_qweight {
  int32_t N;
  int32_t K;
  int32_t bits;
  int32_t group;
  const uint32_t *qweight;
  const uint16_t *scale;
  const uint16_t *zero;
} harp_qweight;

/*
 * x~ = F_V x for each of M rows (technical summary §2.1-2.2: sign flip, then
 * stages 0..L-1 in place; §2.4: stride stages without a materialised
 * permutation).
 *   x   [M][V->dim] of x_dt;  xt  [M][V->dim] of xt_dt.
 * Arithmetic is float32; a bf16 xt is rounded to nearest even at the end.
 */
harp_status harp_rotate_in(const harp_rotation *V, const void *x,
                           harp_dtype x_dt, void *xt, harp_dtype xt_dt,
                           int32_t M, harp_stream stream);

/*
 * y = F_U^T y' for each of M rows: the output side U = F_U^T of the
 * two-sided processor (technical summary §2.1-2.2 for the stages; §5: the
 * processor is an exact change of basis, so U undoes the F_U applied to the
 * weight offline).  Stages L-1..0 (each stage is its own transpose), then
 * the sign flip; float32 arithmetic.
 *   yt  [M][U->dim] float32;  y  [M][U->dim] of y_dt (bf16: nearest even).
 */
harp_status harp_rotate_out(const harp_rotation *U, const float *yt, void *y,
                            harp_dtype y_dt, int32_t M, harp_stream stream);

/*
 * x~ = F x (stages 0 .. m-1 after the sign flip) and y = F^T y' (transposed
 * blocks, stages m-1 .. 0, then the sign flip) for M rows of a mixed-radix
 * side; float32 arithmetic, a bf16 output rounds to nearest even.
 *   x  [M][dim] of x_dt;  xt [M][dim] of xt_dt;  yt [M][dim] float32;
 *   y  [M][dim] of y_dt.
 *   workspace  optional, used only for a bf16 output: at least
 *              harp_rotate_mixed_workspace_bytes(dim, M, HARP_BF16) bytes,
 *              16-byte aligned (HARP_ERR_WORKSPACE if smaller).  With it the
 *              stages run one launch each over the whole chip in float32 in
 *              the workspace and the last stage writes the bf16 output; with
 *              NULL one workgroup rotates each row in LDS (slower, notably
 *              for radices that are not powers of two).  A float32 output is
 *              its own workspace.  The contents need no initialisation;
 *              calls that share a workspace must not overlap in time.
 */
/*
 * Expand the learnable parameters of a mixed-radix side into the float32
 * blocks of harp_mixed_rotation.blocks (technical summary §2.2: each block
 * is B = Q(theta) G_b).  G_b is the fixed base mixer: H_b / sqrt(b) by
 * Sylvester's construction for powers of two, otherwise the orthogonal
 * factor Q of the QR factorisation of a fixed b x b Gaussian matrix, with
 * R's diagonal made positive (technical summary §2.1-2.2: QR of a fixed
 * Gaussian for radices that are no power of two).  Q(theta) is the Givens
 * rotation [[cos phi, -sin phi], [sin phi, cos phi]] for b = 2 and the
 * Cayley map (I - A)(I + A)^-1 of the skew-symmetric A for b > 2, so zero
 * parameters give B = G_b.  Offline, host memory: float64 arithmetic
 * (Householder QR, Gaussian elimination with partial pivoting), float32
 * output rounded to nearest.  Synchronous; launches nothing.
 *   n_stages, radix  as in harp_mixed_rotation (dim = prod radix)
 *   params     host float64, the stages one after the other; stage t holds
 *              [dim/b_t][b_t (b_t - 1) / 2]: per group the angle phi
 *              (b_t = 2) or A's upper triangle A[r][c], r < c, row by row.
 *   gaussians  host float64: one b_t x b_t row-major matrix for every stage
 *              whose radix is not a power of two, in stage order (pass the
 *              same matrix again for a repeated radix to share its mixer);
 *              NULL allowed when every radix is a power of two.
 *   blocks     host float32 out, 4 * dim * sum_t b_t bytes, in the layout of
 *              harp_mixed_rotation.blocks.
 * Errors: HARP_ERR_NULL (radix, params or blocks NULL; gaussians NULL while
 * needed), HARP_ERR_SHAPE / HARP_ERR_UNSUPPORTED for the schedule as in the
 * mixed-radix rotations, HARP_ERR_SHAPE for a non-finite parameter or
 * Gaussian entry or a rank-deficient Gaussian.  blocks is written only on
 * success.
 */
harp_status harp_mixed_expand(int32_t n_stages, const int32_t *radix, const double *params,
                              const double *gaussians, float *blocks);

harp_status harp_rotate_in_mixed(const harp_mixed_rotation *R, const void *x,
                                 harp_dtype x_dt, void *xt, harp_dtype xt_dt,
                                 int32_t M, void *workspace, size_t ws_bytes,
                                 harp_stream stream);
harp_status harp_rotate_out_mixed(const harp_mixed_rotation *R, const float *yt,
                                  void *y, harp_dtype y_dt, int32_t M,
                                  void *workspace, size_t ws_bytes, harp_stream stream);
/* Workspace bytes for M rows of dim with output dtype out_dt (0 for float32;
 * 0 for arguments out of range). */
size_t harp_rotate_mixed_workspace_bytes(int32_t dim, int32_t M, harp_dtype out_dt);

/*
 * y'[m][n] = sum_k w_hat[n][k] x~[m][k]: the quantized matmul between the
 * two rotations (technical summary §2.4: HARP wraps the backend's quantized
 * linear without changing it; the backend's codebook is not on the pages,
 * so w_hat is the stand-in per-group uniform grid described at the top of
 * this header).  float32 throughout: w_hat is exact in float32 and x~ is
 * not rounded.  One or two rows (and 3-bit codes up to 8 rows) on the
 * vector ALUs; 3..8 rows of 2- and 4-bit codes on the bf16 matrix cores
 * with x~ split into exact bf16 planes; from 9 rows on in 16-row tiles on
 * the float32 matrix cores (same products, float32 accumulation in a
 * different order).  Meant for decode batches; any M is accepted.
 *   xt  [M][W->K] float32;  yt  [M][W->N] float32.
 */
harp_status harp_deq_gemv(const harp_qweight *W, const float *xt, float *yt,
                          int32_t M, harp_stream stream);

/*
 * harp_deq_gemv with an optional workspace (the same product, reading
 * and contract: float32, x~ not rounded).  With a workspace, one row
 * (M = 1) of 2-bit codes on a layer of at least 2^27 weights (N a multiple
 * of 16, K of 256) runs on the FP4 x FP8 matrix cores: the codes enter as
 * exact FP4 values and x~ as eight FP8 planes of base-16 digits per
 * quantization group (x~ carried to 2^-28 of its group maximum, every
 * matrix-core sum exact), K split into slices summed in a fixed order
 * (bitwise reproducible).  Other calls, and NULL, run harp_deq_gemv.
 *   xt  [M][W->K] float32;  yt  [M][W->N] float32.
 *   workspace  optional: NULL, or at least harp_deq_gemv_workspace_bytes(M,
 *              N, K) bytes, 256-byte aligned, zero-filled before its first
 *              use (its first 2048 bytes are arrival counters that every
 *              call leaves at zero; the rest needs no initialisation).
 *              Calls that share a workspace must not overlap in time.
 */
harp_status harp_deq_gemv_ws(const harp_qweight *W, const float *xt, float *yt,
                             int32_t M, void *workspace, size_t ws_bytes,
                             harp_stream stream);

/* Workspace bytes harp_deq_gemv_ws uses for M rows of a K -> N product (0:
 * it uses none for this shape); 0 for out-of-range sizes. */
size_t harp_deq_gemv_workspace_bytes(int32_t M, int32_t N, int32_t K);

/*
 * y' = w_hat (F_V x) for small batches in one launch: every workgroup applies
 * the input rotation (technical summary §2.1-2.2, as harp_rotate_in with a
 * float32 x~) to the whole input row in its local memory while its weights
 * load, then forms its rows of the float32 product as harp_deq_gemv does.
 * Supported shapes: 1 <= M <= 4, W->K <= 4096, V->block >= 8; other shapes
 * return HARP_ERR_UNSUPPORTED (use harp_rotate_in + harp_deq_gemv).
 * Requires V->dim == W->K.
 *   x  [M][K] of x_dt;  yt  [M][W->N] float32.
 */
harp_status harp_rotate_in_deq_gemv(const harp_rotation *V,
                                    const harp_qweight *W, const void *x,
                                    harp_dtype x_dt, float *yt, int32_t M,
                                    harp_stream stream);

/*
 * y'[m][n] = sum_k w_hat[n][k] x~[m][k] for batched (prefill) rows on the
 * bf16 matrix cores with float32 accumulation: the same quantized matmul as
 * harp_deq_gemv (technical summary §2.4; w_hat the stand-in per-group
 * uniform grid described at the top of this header), with x~ given in bf16.
 * Any M >= 0.
 * M <= 64: one workgroup per 16 output features; the integer codes enter
 * the matrix cores exactly and scale and zero are applied per group, so
 * w_hat is not rounded; no workspace (a given workspace is not used).
 * M > 64: 128 x 128 output tiles on bf16(w_hat) (nearest even).
 *   xt_bf16    [M][W->K] bf16;  yt  [M][W->N] float32.
 *   workspace  optional (M > 64).  NULL runs the product as one K slice.
 *              Otherwise at least harp_deq_gemm_workspace_bytes(M, N, K)
 *              bytes, 256-byte aligned: the K dimension is split into slices
 *              that run concurrently and are summed in a fixed slice order
 *              (bitwise reproducible).  Its first 2048 bytes hold per-tile
 *              arrival counters at the same offset for every shape: zero-fill
 *              the workspace once before its first use; every call leaves the
 *              counters at zero, so one workspace serves any sequence of
 *              shapes it is large enough for (the partial tiles need no
 *              initialisation).  Calls that share a workspace must not
 *              overlap in time.
 */
harp_status harp_deq_gemm(const harp_qweight *W, const uint16_t *xt_bf16,
                          float *yt, int32_t M, void *workspace,
                          size_t ws_bytes, harp_stream stream);

/* Workspace bytes harp_deq_gemm uses for M rows of a K -> N product (0: the
 * product needs none: M <= 64, or one K slice); 0 for out-of-range sizes. */
size_t harp_deq_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K);

/* Workspace bytes harp_linear_fused needs for M rows of a K -> N linear;
 * 0 for M == 0 and when an argument is out of range. */
size_t harp_linear_workspace_bytes(int32_t M, int32_t N, int32_t K);

/*
 * The whole linear with mixed-radix sides, y = F_U^T deq(W) F_V x
 * (technical summary §2.4 with the stages of §2.1-2.2), for dimensions that
 * are no power of two (e.g. 5120 = 8*8*8*5*2).  Requires V->dim == W->K and
 * U->dim == W->N.  The same batch ranges and rounding points as
 * harp_linear_fused: float32 x~ below 64 rows (the product of harp_deq_gemv
 * below 16, the small-batch matrix-core product on the two-plane bf16 split
 * of x~ from 16), bf16 x~ from 64 rows (the small-batch product at 64, the
 * matrix-core GEMM with split K above).
 *   x  [M][K] of x_dt;  y  [M][N] of y_dt.
 *   workspace  at least harp_linear_mixed_workspace_bytes(M, N, K) bytes,
 *              256-byte aligned, zero-filled before its first use (its first
 *              2048 bytes are the split-K counters, at the same offset for
 *              every shape; every call leaves them at zero).  Calls that
 *              share a workspace must not overlap in time.
 */
harp_status harp_linear_fused_mixed(const harp_mixed_rotation *V, const harp_qweight *W,
                                    const harp_mixed_rotation *U, const void *x,
                                    harp_dtype x_dt, void *y, harp_dtype y_dt,
                                    int32_t M, void *workspace, size_t ws_bytes,
                                    harp_stream stream);
/* Workspace bytes of harp_linear_fused_mixed; 0 for M == 0 and for arguments
 * out of range. */
size_t harp_linear_mixed_workspace_bytes(int32_t M, int32_t N, int32_t K);

/*
 * y = F_U^T deq(W) F_V x, the whole linear (technical summary §2.4 and §5).
 * Requires V->dim == W->K and U->dim == W->N.  Batch ranges:
 *   M < 16: rotate-in to a float32 x~, the float32 product of
 *     harp_deq_gemv, rotate-out; the first two in one launch for M <= 2 and
 *     N <= 4096 where harp_rotate_in_deq_gemv supports the shape.
 *     M == 1 with 2- or 4-bit codes on a layer of at least 2^27 weights
 *     (N a multiple of 16, K of 256): the block-scaled matrix-core product
 *     (2-bit codes as FP4, 4-bit codes as FP8 values, x~ as FP8 digit planes
 *     exact to 2^-28 of each group's largest value, written by the input
 *     rotation's last launch for b_V = 256 / 4096 / 8192), K cut into
 *     slices summed in slice order; with a b_U = 256 output side and one K
 *     slice the output rotation runs inside the product's launch.
 *   16 <= M < 64: rotate-in to a float32 x~, the small-batch matrix-core
 *     product on x~ split exactly into two bf16 planes hi + lo
 *     (|x~ - hi - lo| <= 2^-16 |x~|; w_hat exact), rotate-out.  Where K is
 *     a multiple of 4096 and N at least 8192 the product may split K into
 *     slices whose partials, summed in slice order, use the workspace.
 *   M >= 64: rotate-in to a bf16 x~, the matrix-core product of
 *     harp_deq_gemm (w_hat exact at 64 rows, bf16 above), rotate-out.
 *   x  [M][K] of x_dt;  y  [M][N] of y_dt;
 *   workspace  at least harp_linear_workspace_bytes(M, N, K) bytes, 256-byte
 *              aligned, owned by the caller.  Zero-filled before its first
 *              use: its first 2048 bytes hold the split-K arrival counters,
 *              at the same offset for every shape, and every call leaves them
 *              at zero, so one workspace serves any sequence of shapes it is
 *              large enough for; the rest is clobbered.  Calls that share a
 *              workspace must not overlap in time.
 */
harp_status harp_linear_fused(const harp_rotation *V, const harp_qweight *W,
                              const harp_rotation *U, const void *x,
                              harp_dtype x_dt, void *y, harp_dtype y_dt,
                              int32_t M, void *workspace, size_t ws_bytes,
                              harp_stream stream);

/*
 * Offline preparation (technical summary §2.4: the processor rotates the
 * weight before the quantization backend; §5: an exact change of basis).
 *
 * W' = F_U W F_V^T for a dense float32 weight W [N][K] (out x in): each row
 * w_n becomes F_V w_n (the input-side rotation of harp_rotate_in, rows as
 * the batch), then each column is rotated by F_U (the rows of the
 * transpose).  float32 throughout.  Requires V->dim == K, U->dim == N,
 * N, K <= HARP_MAX_M.
 *   W, Wp      [N][K] float32, device, 16-byte aligned; Wp may not alias W.
 *   workspace  at least harp_rotate_weight_workspace_bytes(N, K) bytes,
 *              256-byte aligned, clobbered.
 */
harp_status harp_rotate_weight(const harp_rotation *V, const harp_rotation *U,
                               const float *W, float *Wp, int32_t N, int32_t K,
                               void *workspace, size_t ws_bytes, harp_stream stream);
size_t harp_rotate_weight_workspace_bytes(int32_t N, int32_t K);

/*
 * Quantize and pack a float32 weight Wp [N][K] into the harp_qweight layout
 * (qweight [N][K*bits/32], scale and zero [N][K/64] fp16 bit patterns):
 * per row and group of 64 inputs, lo = min(min w, 0), hi = max(max w, 0)
 * (-1 and 1 when both are 0), s = fp16((hi - lo) / (2^bits - 1)) at least
 * 2^-14, z = clamp(rint(-lo / s), 0, 2^bits - 1) (+0 when 0),
 * q = clamp(rint(w / s) + z, 0, 2^bits - 1); rint rounds half to even and
 * every step is one IEEE float32 operation, so the result is reproducible
 * bit for bit.  Wp finite.  bits 2, 3 or 4; K % 64 == 0.
 */
harp_status harp_quantize_pack(const float *Wp, int32_t N, int32_t K, int32_t bits,
                               uint32_t *qweight, uint16_t *scale, uint16_t *zero,
                               harp_stream stream);

/*
 * A stack of dependent decode linears in one launch (technical summary §2.4:
 * the rotated linear; §2.1-2.2: the stride stages of each side), the way a
 * decoder runs them layer after layer:
 *     y_l = F_{U,l}^T deq(W_l) F_{V,l} y_{l-1}   for l = 0 .. n_layers-1,
 * with y_{-1} = x.  Each layer's product is the float32 product of
 * harp_deq_gemv (x~ not rounded), so every y_l equals harp_linear_fused on
 * the stored y_{l-1} within its float32 bar; the next layer reads y_l as
 * stored (rounded to bf16 when y_dt is HARP_BF16).  The weights of layer
 * l + 1 are fetched while layer l still runs, and the steps between layers
 * are workgroup-to-workgroup handoffs on the device, not launches.
 * Supported shapes (else HARP_ERR_UNSUPPORTED): every layer square with
 * K = N = dim = V->block = U->block, dim 4096 or 8192; one bit width for the
 * whole stack; angles as float32 (cos, sin) pairs; 1 <= M <= 4 for dim 4096,
 * 1 <= M <= 2 for dim 8192 (M == 0 does nothing).
 *   layers     host array of n_layers layers (n_layers >= 0); y of each
 *              layer is device memory [M][dim] of y_dt.  Output buffers may
 *              be shared between layers (ping-pong) and with x: nothing in
 *              the stack reads a layer output back.
 *   x          [M][dim] of x_dt, device.
 *   workspace  at least harp_linear_chain_workspace_bytes(dim) bytes,
 *              256-byte aligned, zero-filled once before its first use; every
 *              call leaves it ready for the next.  Calls that share a
 *              workspace must not overlap in time.
 * Stacks longer than 48 layers run as one launch per 48 layers.  Every wait
 * inside a launch is bounded; a wait that runs out (which needs a stalled
 * device) leaves the outputs undefined and a nonzero second workspace word.
 */
typedef struct harp_chain_layer {
  harp_rotation V;
  harp_qweight W;
  harp_rotation U;
  void *y;
} harp_chain_layer;
size_t harp_linear_chain_workspace_bytes(int32_t dim);
harp_status harp_linear_chain(const harp_chain_layer *layers, int32_t n_layers, const void *x,
                              harp_dtype x_dt, harp_dtype y_dt, int32_t M, void *workspace,
                              size_t ws_bytes, harp_stream stream);

/*
 * harp_linear_fused for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, checks, results (within the path's float32 or
 * bf16 bar) and batch ranges as harp_linear_fused, minus the workspace:
 * x~ and y' live in a fixed device array of HARP_NOALLOC_SCRATCH_BYTES that
 * the library holds on each GPU it runs on until the process ends.  The call
 * allocates nothing (no hipMalloc/hipFree, no allocating library routine);
 * its first call on a device looks up that device's array address.
 * M > 64 runs the GEMM as one K slice (no split K), so nothing in the array
 * needs initialisation.  Size limit: 2048 + align256(M K e) + align256(4 M N)
 * bytes at most HARP_NOALLOC_SCRATCH_BYTES, with e = 4 for M < 64 and 2 from
 * 64 on (align256 rounds up to a multiple of 256); larger calls return
 * HARP_ERR_WORKSPACE and launch nothing.  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (other streams, other
 * threads) race and must be serialised by the caller.
 */
#define HARP_NOALLOC_SCRATCH_BYTES (32u << 20)
harp_status harp_linear_fused_noalloc(const harp_rotation *V, const harp_qweight *W,
                                      const harp_rotation *U, const void *x,
                                      harp_dtype x_dt, void *y, harp_dtype y_dt,
                                      int32_t M, harp_stream stream);

/*
 * Test hook, not on the hot path: writes the dense w_hat [N][K] as float32
 * (exact) or bf16 (nearest even), through the same device unpack and
 * dequant code the products use (the stand-in per-group uniform grid
 * described at the top of this header; technical summary §2.4 leaves the
 * backend's codebook open).
 *   out  [W->N][W->K] of out_dt, device, 16-byte aligned.
 */
harp_status harp_dequant(const harp_qweight *W, void *out, harp_dtype out_dt,
                         harp_stream stream);

/* Static string naming a status. */
const char *harp_status_string(harp_status status);

/* hipError_t of this thread's last failed launch (0 if none). */
int32_t harp_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HARP_H */
