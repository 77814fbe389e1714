"""Plain float64 CPU oracle for the HARP rotated low-bit linear.

TEST INFRASTRUCTURE ONLY.  This module exists to check the HIP library.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The library under ``rotated_bit_amd/`` never
imports, links or calls anything here, and nothing here imports the library.

What it computes, and where each step comes from
------------------------------------------------
Source page: "HARP: Hadamard-Preconditioned Adaptive Rotation Processor for
Extreme LLM Quantization" (gist.science technical summary of arXiv 2605.29843).

* Technical summary §2.1: the orthogonal map is a product of sparse stages,
  each a block-diagonal orthogonal matrix acting on coordinates that are a
  stride apart ("separated by stride permutations").  With every radix equal
  to 2 there are L = log2(b) stages, each made of b/2 independent 2x2 blocks.
* Technical summary §2.2: each block is B = Q(phi) G_2, where G_2 is the
  normalised 2x2 Sylvester Hadamard and Q a Givens rotation; at phi = 0 the
  whole map is the fixed randomized Hadamard transform (RHT).
* Technical summary §1 and §2.4: RHT costs O(d log d); the stages are applied
  in place, without materialising the permutation.
* Technical summary §5: the processor is an exact change of basis: the model
  y = U (U^T W V) V^T x is unchanged before quantization.

Readings taken where the page is silent (all listed with reasons in the
repository's design notes):

* Block form.  Q(phi) G_2 = [[cos t, sin t], [sin t, -cos t]] with
  t = pi/4 + phi (``paper_block`` and ``block``).  The library takes the block
  as the float32 pair (cos t, sin t).
* Pairing.  Stage s pairs coordinate i (bit s clear) with i + 2^s; the block
  index of that pair is i with bit s deleted.  Stages run s = 0, 1, ..., L-1.
* Signs.  One random +-1 diagonal per side, applied before the stages:
  F = B_{L-1} ... B_0 D.  The input side computes x~ = F_V x, the output side
  y = F_U^T y'.  Offline, W' = F_U W F_V^T.
* Dimensions that are not one power of two are block-diagonal: independent
  butterflies of size b, each with its own angles and sign slice.
* Quantizer stand-in (the page leaves the codebook to QuIP#/QTIP): per row
  and per group of 64 consecutive inputs, asymmetric min-max with zero forced
  into the range, fp16 scale s, integer zero z stored in fp16, round half to
  even, codes clamped to [0, 2^B - 1]; dequantized weight (q - z) s.
* Packing: 2- and 4-bit codes least-significant-bits first, 32/B per uint32
  word; 3-bit codes as a 96-bit little-endian bit stream per 32 weights
  (three words).
* Rounding points of the batched (bf16 matrix-core) path: the rotated input
  and the dequantized weight are rounded to bf16, round to nearest even; a
  matrix-core product that multiplies the integer codes and applies scale
  and zero per group afterwards rounds only the rotated input.
* Mixed radix (technical summary §2.1-2.2, ``mixed_forward``): stage t acts
  on mixed-radix digit t (stride prod_{s<t} b_s); blocks Q(theta) G_b with
  Q the Cayley map (I - A)(I + A)^-1 for b > 2 and the QR factor of a fixed
  Gaussian (positive R diagonal; the Gaussian itself is an input, drawn once
  per radix by the seeded generators) as G_b for radices that are not
  powers of two.
* int8 storage of the angles (technical summary §2.4 storage note, §4
  storage overhead; the pages give no encoding).  Each block's angle
  perturbation phi = t - pi/4 is stored as one signed 8-bit code c with one
  float32 step per side: phi = c * step (``decode_angle_codes``).  Code 0 is
  the Hadamard initialisation.

Every routine is written for clarity, not speed: numpy float64, one library
matrix product for the contraction, no blocking or fusion.
"""

from __future__ import annotations

import numpy as np

GROUP = 64


# ---------------------------------------------------------------------------
# Fixed base mixer (technical summary §2.2: normalised Sylvester Hadamard)
# ---------------------------------------------------------------------------

def sylvester_hadamard(b: int) -> np.ndarray:
    """Unnormalised Sylvester Hadamard matrix of order b (b a power of two).

    H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]].
    """
    if b < 1 or b & (b - 1):
        raise ValueError("b must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < b:
        h = np.block([[h, h], [h, -h]])
    return h


def paper_block(phi: float) -> np.ndarray:
    """The page's learnable 2x2 block Q(phi) G_2 (technical summary §2.2).

    Q is the Givens rotation [[cos, -sin], [sin, cos]] and G_2 the normalised
    2x2 Hadamard.  Built as a literal matrix product so that tests can pin the
    (cos t, sin t) form used everywhere else against it.
    """
    q = np.array([[np.cos(phi), -np.sin(phi)], [np.sin(phi), np.cos(phi)]])
    g2 = sylvester_hadamard(2) / np.sqrt(2.0)
    return q @ g2


def block(c: float, s: float) -> np.ndarray:
    """2x2 block for the pair (cos t, sin t): [[c, s], [s, -c]]."""
    return np.array([[c, s], [s, -c]], dtype=np.float64)


def decode_angle_codes(codes: np.ndarray, step) -> np.ndarray:
    """(cos t, sin t) pairs of int8-stored angles, t = pi/4 + code * step.

    codes: int8, any shape (the layout of the float32 pair array without its
    last axis); step: the side's float32 step, taken at its float32 value.
    Returns float64 (..., 2), ready for ``forward`` and ``transpose``.
    """
    c = np.asarray(codes)
    if c.dtype != np.int8:
        raise ValueError("angle codes must be int8")
    phi = c.astype(np.float64) * float(np.float32(step))
    t = np.pi / 4 + phi
    return np.stack([np.cos(t), np.sin(t)], axis=-1)


# ---------------------------------------------------------------------------
# Boundary formats (decoders only)
# ---------------------------------------------------------------------------

def decode_signs(sign_bits: np.ndarray, d: int) -> np.ndarray:
    """+-1 diagonal from the bitmask: bit i of word i//32 set means d_i = -1."""
    words = np.asarray(sign_bits, dtype=np.uint32)
    i = np.arange(d)
    bit = (words[i >> 5] >> (i & 31).astype(np.uint32)) & np.uint32(1)
    return 1.0 - 2.0 * bit.astype(np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64 values (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """fp16 bit patterns (uint16) to float64 values (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits.  Written with frexp so that the rounding is
    taken once, straight from float64 (no detour through float32).  Values
    here are normal numbers well inside the bf16 range.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


# ---------------------------------------------------------------------------
# Butterfly (technical summary §2.1-2.2)
# ---------------------------------------------------------------------------

def _log2(b: int) -> int:
    if b < 2 or b & (b - 1):
        raise ValueError("block size must be a power of two >= 2")
    return b.bit_length() - 1


def apply_stage(u: np.ndarray, cos_s: np.ndarray, sin_s: np.ndarray,
                s: int) -> np.ndarray:
    """One stage on the last axis of u (length b); returns a new array.

    Pairs (i, i + 2^s) for every i with bit s clear.  Writing
    i = hi * 2^(s+1) + lo with lo < 2^s, the pair's block index is
    hi * 2^s + lo (i with bit s deleted).  cos_s and sin_s have shape
    (..., b/2) and broadcast against the leading axes of u.
    """
    b = u.shape[-1]
    h = 1 << s
    v = u.reshape(u.shape[:-1] + (b // (2 * h), 2, h))
    a = v[..., 0, :]                     # coordinate i
    p = v[..., 1, :]                     # coordinate i + 2^s
    c = cos_s.reshape(cos_s.shape[:-1] + (b // (2 * h), h))
    sn = sin_s.reshape(sin_s.shape[:-1] + (b // (2 * h), h))
    out = np.empty_like(v)
    out[..., 0, :] = c * a + sn * p
    out[..., 1, :] = sn * a - c * p
    return out.reshape(u.shape)


def _as_blocks(cs: np.ndarray, d: int, b: int):
    cs = np.asarray(cs, dtype=np.float64)
    L = _log2(b)
    if d % b:
        raise ValueError("dimension must be a multiple of the block size")
    if cs.shape != (d // b, L, b // 2, 2):
        raise ValueError(f"cs must have shape {(d // b, L, b // 2, 2)}")
    return cs, L


def forward(x: np.ndarray, cs: np.ndarray, sign_bits: np.ndarray,
            b: int) -> np.ndarray:
    """F x = blockdiag_j(B^(j)_{L-1} ... B^(j)_0) D x, on the last axis of x.

    x: (..., d).  cs: (d/b, L, b/2, 2) holding (cos t, sin t) per stage and
    block.  sign_bits: bitmask of D.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    cs, L = _as_blocks(cs, d, b)
    u = x * decode_signs(sign_bits, d)
    u = u.reshape(x.shape[:-1] + (d // b, b))
    for s in range(L):
        u = apply_stage(u, cs[:, s, :, 0], cs[:, s, :, 1], s)
    return u.reshape(x.shape)


def transpose(y: np.ndarray, cs: np.ndarray, sign_bits: np.ndarray,
              b: int) -> np.ndarray:
    """F^T y: stages L-1 down to 0 (each stage is symmetric), then D."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    cs, L = _as_blocks(cs, d, b)
    u = y.reshape(y.shape[:-1] + (d // b, b))
    for s in reversed(range(L)):
        u = apply_stage(u, cs[:, s, :, 0], cs[:, s, :, 1], s)
    return u.reshape(y.shape) * decode_signs(sign_bits, d)


def rotation_matrix(cs: np.ndarray, sign_bits: np.ndarray, d: int,
                    b: int) -> np.ndarray:
    """Dense F (d x d): column j is F e_j."""
    return forward(np.eye(d), cs, sign_bits, b).T


# ---------------------------------------------------------------------------
# Mixed-radix stages (technical summary §2.1-2.2)
# ---------------------------------------------------------------------------
# Schedule b = (b_0, ..., b_{m-1}) with prod b_t = d.  Index i is written in
# mixed-radix digits, i = sum_t i_t * stride_t with stride_t = prod_{s<t} b_s
# and 0 <= i_t < b_t.  Stage t applies one b_t x b_t block to each group of
# coordinates that differ only in digit t; the group index c is i with digit
# t deleted: c = (i mod stride_t) + stride_t * (i div (stride_t * b_t)).
# Each block is B_{t,c} = Q_{t,c}(theta) G_{b_t}: G the fixed base mixer
# (normalised Sylvester Hadamard for powers of two, else the Q factor of a
# fixed Gaussian matrix), Q the Givens rotation for b_t = 2 and the Cayley
# map of a skew-symmetric parameter for b_t > 2, so theta = 0 gives B = G.
# F = B_{m-1} ... B_0 D, and the all-2 schedule is the radix-2 butterfly
# above.  Blocks are stored row-major: output r = sum_j B[r][j] input j.


def strides(radices) -> list:
    out, acc = [], 1
    for b in radices:
        out.append(acc)
        acc *= b
    return out


def cayley(A: np.ndarray) -> np.ndarray:
    """Q = (I - A)(I + A)^-1 for a skew-symmetric A (orthogonal, Q(0) = I)."""
    A = np.asarray(A, dtype=np.float64)
    if not np.allclose(A, -A.T, atol=0, rtol=0):
        raise ValueError("A must be skew-symmetric")
    I = np.eye(A.shape[0])
    return (I - A) @ np.linalg.inv(I + A)


def skew_from_params(p: np.ndarray, b: int) -> np.ndarray:
    """Skew-symmetric b x b matrix from its b(b-1)/2 upper-triangle entries
    (row-major order): A[r][c] = p_k for r < c, A[c][r] = -p_k."""
    p = np.asarray(p, dtype=np.float64)
    if p.shape != (b * (b - 1) // 2,):
        raise ValueError("need b(b-1)/2 parameters")
    A = np.zeros((b, b))
    iu = np.triu_indices(b, 1)
    A[iu] = p
    return A - A.T


def qr_mixer(g: np.ndarray) -> np.ndarray:
    """Q factor of the fixed b x b Gaussian g (an input: the random matrix the
    method draws once), with the sign of each column chosen so that R has a
    positive diagonal (the unique QR factorisation)."""
    g = np.asarray(g, dtype=np.float64)
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def base_mixer(b: int, g=None) -> np.ndarray:
    """G_b: normalised Sylvester Hadamard for powers of two, else the QR
    factor of the fixed Gaussian g (b x b)."""
    if b & (b - 1) == 0:
        return sylvester_hadamard(b) / np.sqrt(b)
    if g is None:
        raise ValueError(f"radix {b} is not a power of two: its fixed Gaussian is needed")
    return qr_mixer(g)


def mixed_blocks(radices, params, gaussians=None) -> list:
    """Expand the learnable parameters into blocks, one array per stage.

    params[t]: shape (d / b_t, b_t (b_t - 1) / 2): per group, the Givens
    angle phi (b_t = 2) or the upper triangle of the Cayley parameter
    (b_t > 2).  gaussians[t]: the fixed b_t x b_t Gaussian whose QR factor
    is stage t's mixer when b_t is not a power of two (None otherwise; the
    whole list may be None when every radix is a power of two).  Returns
    [t] -> (d / b_t, b_t, b_t) float64 blocks B = Q(theta) G_{b_t}.
    """
    d = int(np.prod(radices))
    out = []
    for t, b in enumerate(radices):
        G = base_mixer(b, None if gaussians is None else gaussians[t])
        P = np.asarray(params[t], dtype=np.float64)
        if P.shape != (d // b, b * (b - 1) // 2):
            raise ValueError(f"stage {t}: params must have shape {(d // b, b * (b - 1) // 2)}")
        blocks = np.empty((d // b, b, b))
        for c in range(d // b):
            if b == 2:
                phi = P[c, 0]
                Q = np.array([[np.cos(phi), -np.sin(phi)], [np.sin(phi), np.cos(phi)]])
            else:
                Q = cayley(skew_from_params(P[c], b))
            blocks[c] = Q @ G
        out.append(blocks)
    return out


def _mixed_stage(u: np.ndarray, blocks: np.ndarray, stride: int, b: int,
                 transpose: bool) -> np.ndarray:
    """Apply stage blocks (d/b, b, b) along the digit of stride `stride`."""
    d = u.shape[-1]
    lead = u.shape[:-1]
    # view: [hi][digit][lo] with lo < stride; group c = lo + stride * hi
    v = u.reshape(lead + (d // (stride * b), b, stride))
    Bm = blocks.reshape(d // (stride * b), stride, b, b)     # [hi][lo][r][j]
    if transpose:
        Bm = np.swapaxes(Bm, -1, -2)
    out = np.einsum("hlrj,...hjl->...hrl", Bm, v)
    return out.reshape(u.shape)


def mixed_forward(x: np.ndarray, radices, blocks, sign_bits) -> np.ndarray:
    """F x = B_{m-1} ... B_0 D x on the last axis (length prod radices)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if int(np.prod(radices)) != d:
        raise ValueError("radices must multiply to the dimension")
    u = x * decode_signs(sign_bits, d)
    for t, (b, st) in enumerate(zip(radices, strides(radices))):
        u = _mixed_stage(u, np.asarray(blocks[t], dtype=np.float64), st, b, False)
    return u


def mixed_transpose(y: np.ndarray, radices, blocks, sign_bits) -> np.ndarray:
    """F^T y = D B_0^T ... B_{m-1}^T y (blocks transposed, stages reversed)."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    if int(np.prod(radices)) != d:
        raise ValueError("radices must multiply to the dimension")
    u = y
    for t in reversed(range(len(radices))):
        u = _mixed_stage(u, np.asarray(blocks[t], dtype=np.float64),
                         strides(radices)[t], radices[t], True)
    return u * decode_signs(sign_bits, d)


# ---------------------------------------------------------------------------
# Offline preparation (technical summary §2.4: rotate, then quantize)
# ---------------------------------------------------------------------------

def rotate_weight(W: np.ndarray, cs_u, signs_u, b_u, cs_v, signs_v,
                  b_v) -> np.ndarray:
    """W' = F_U W F_V^T for W stored as [N][K] (out x in)."""
    W = np.asarray(W, dtype=np.float64)
    rows = forward(W, cs_v, signs_v, b_v)          # each row: F_V w_n
    return forward(rows.T, cs_u, signs_u, b_u).T   # each column: F_U


def quantize(Wp: np.ndarray, bits: int, group: int = GROUP, arith: str = "f64"):
    """Per-row, per-group uniform asymmetric quantizer (stand-in reading).

    Returns (q uint8 [N][K], scale fp16 [N][K/group], zero fp16 [N][K/group]).
    For one group w: lo = min(min w, 0), hi = max(max w, 0) (lo = -1, hi = 1
    when both are 0); s = fp16((hi - lo) / (2^B - 1)), at least 2^-14;
    z = clamp(rint(-lo / s), 0, 2^B - 1) (a zero-point of 0 stored as +0);
    q = clamp(rint(w / s) + z, 0, 2^B - 1).  rint rounds half to even.

    arith: the precision each step is evaluated in.  "f64" evaluates in
    float64 (the offline reference).  "f32" takes every step as one IEEE
    float32 operation rounded to nearest even (hi - lo, the division by
    2^B - 1, each w / s and -lo / s), as a float32 implementation does;
    float decides the integer codes, so a check of such an implementation
    takes the decisions in its precision.  The input is then float32.
    """
    if arith not in ("f64", "f32"):
        raise ValueError("arith must be 'f64' or 'f32'")
    ft = np.float64 if arith == "f64" else np.float32
    Wp = np.asarray(Wp, dtype=ft)
    n, k = Wp.shape
    if k % group:
        raise ValueError("K must be a multiple of the group size")
    qmax = (1 << bits) - 1
    g = Wp.reshape(n, k // group, group)
    zero = ft(0.0)
    lo = np.minimum(g.min(axis=2), zero)
    hi = np.maximum(g.max(axis=2), zero)
    flat = hi == lo
    lo = np.where(flat, ft(-1.0), lo).astype(ft)
    hi = np.where(flat, ft(1.0), hi).astype(ft)
    s16 = ((hi - lo) / ft(qmax)).astype(np.float16)
    s16 = np.maximum(s16, np.float16(2.0 ** -14))
    s = s16.astype(ft)
    # + 0: a zero-point of 0 is stored as +0 (a group whose minimum is -0.0
    # would otherwise give -0)
    z = (np.clip(np.rint(-lo / s), 0, qmax) + ft(0.0)).astype(ft)
    q = np.clip(np.rint(g / s[..., None]) + z[..., None], 0, qmax)
    return (q.reshape(n, k).astype(np.uint8), s16,
            z.astype(np.float16))


def pack(q: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes [N][K] into uint32 words [N][K*bits/32] (LSB first)."""
    q = np.asarray(q, dtype=np.uint64)
    n, k = q.shape
    if bits in (2, 4):
        per = 32 // bits
        if k % per:
            raise ValueError("K must fill whole words")
        f = q.reshape(n, k // per, per)
        shifts = (np.arange(per, dtype=np.uint64) * np.uint64(bits))
        return (f << shifts).sum(axis=2).astype(np.uint32)
    if bits == 3:
        if k % 32:
            raise ValueError("3-bit rows pack 32 codes into 3 words")
        f = q.reshape(n, k // 32, 32)
        words = np.zeros((n, k // 32, 3), dtype=np.uint64)
        for j in range(32):
            pos = 3 * j                          # bit position in the 96-bit run
            w, off = divmod(pos, 32)
            words[:, :, w] |= (f[:, :, j] << np.uint64(off)) & np.uint64(0xFFFFFFFF)
            if off > 29:                         # field straddles two words
                words[:, :, w + 1] |= f[:, :, j] >> np.uint64(32 - off)
        return words.reshape(n, k // 32 * 3).astype(np.uint32)
    raise ValueError("bits must be 2, 3 or 4")


def unpack(words: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Codes [N][K] from packed words [N][K*bits/32]; inverse of ``pack``."""
    w = np.asarray(words, dtype=np.uint64)
    n = w.shape[0]
    if w.shape[1] * 32 != K * bits:
        raise ValueError("word count does not match K and bits")
    mask = np.uint64((1 << bits) - 1)
    if bits in (2, 4):
        per = 32 // bits
        shifts = np.arange(per, dtype=np.uint64) * np.uint64(bits)
        q = (w[:, :, None] >> shifts) & mask
        return q.reshape(n, K).astype(np.uint8)
    if bits == 3:
        t = w.reshape(n, K // 32, 3)
        run = t[:, :, 0] | (t[:, :, 1] << np.uint64(32))   # low 64 bits
        high = t[:, :, 2]                                    # bits 64..95
        q = np.empty((n, K // 32, 32), dtype=np.uint64)
        for j in range(32):
            pos = 3 * j
            if pos + 3 <= 64:
                q[:, :, j] = (run >> np.uint64(pos)) & mask
            elif pos >= 64:
                q[:, :, j] = (high >> np.uint64(pos - 64)) & mask
            else:                                            # bits 63..65
                lo_bits = 64 - pos
                q[:, :, j] = ((run >> np.uint64(pos)) |
                              (high << np.uint64(lo_bits))) & mask
        return q.reshape(n, K).astype(np.uint8)
    raise ValueError("bits must be 2, 3 or 4")


def dequant(q: np.ndarray, scale: np.ndarray, zero: np.ndarray,
            group: int = GROUP) -> np.ndarray:
    """w_hat[n][k] = (q[n][k] - z[n][k/64]) * s[n][k/64], in float64.

    scale and zero are fp16 values (float16 arrays or already-decoded
    floats).  |q - z| <= 15 and s has 11 significant bits, so the product is
    exact in float64 and in float32.
    """
    q = np.asarray(q, dtype=np.float64)
    s = np.repeat(np.asarray(scale, dtype=np.float64), group, axis=1)
    z = np.repeat(np.asarray(zero, dtype=np.float64), group, axis=1)
    return (q - z) * s


# ---------------------------------------------------------------------------
# The online linear (technical summary §2.4 and §5): y = U W_hat V^T x
# ---------------------------------------------------------------------------

def linear(x: np.ndarray, words: np.ndarray, scale: np.ndarray,
           zero: np.ndarray, bits: int, cs_v, signs_v, b_v, cs_u, signs_u,
           b_u, mfma_contract: bool = False, weights_exact: bool = False) -> np.ndarray:
    """y = F_U^T (W_hat (F_V x)) for x of shape (M, K); returns (M, N).

    x holds the values the device received (decoded to float64).  With
    ``mfma_contract`` the rounding points of a bf16 matrix-core product are
    modelled: x~ is rounded to bf16 (round to nearest even) and, unless
    ``weights_exact``, so is w_hat, before the float64 contraction.  (A
    product that feeds the integer codes to the matrix cores and applies
    scale and zero afterwards uses w_hat exactly: ``weights_exact``.)
    Everything else is float64.
    """
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    w_hat = dequant(unpack(words, bits, K), scale, zero)
    xt = forward(x, cs_v, signs_v, b_v)
    if mfma_contract:
        xt = bf16_round(xt)
        if not weights_exact:
            w_hat = bf16_round(w_hat)
    yp = xt @ w_hat.T
    return transpose(yp, cs_u, signs_u, b_u)


def linear_mixed(x: np.ndarray, words: np.ndarray, scale: np.ndarray,
                 zero: np.ndarray, bits: int, radices_v, blocks_v, signs_v,
                 radices_u, blocks_u, signs_u, mfma_contract: bool = False,
                 weights_exact: bool = False) -> np.ndarray:
    """y = F_U^T (W_hat (F_V x)) with mixed-radix sides (technical summary
    §2.1-§2.2 for F, §2.4 for the linear); x (M, K) -> (M, N).

    The same steps as ``linear``: dequantize, rotate the input with
    ``mixed_forward``, model the matrix-core rounding points when asked,
    contract in float64, rotate the output with ``mixed_transpose``.
    """
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    w_hat = dequant(unpack(words, bits, K), scale, zero)
    xt = mixed_forward(x, radices_v, blocks_v, signs_v)
    if mfma_contract:
        xt = bf16_round(xt)
        if not weights_exact:
            w_hat = bf16_round(w_hat)
    yp = xt @ w_hat.T
    return mixed_transpose(yp, radices_u, blocks_u, signs_u)


def rel_l2(a: np.ndarray, ref: np.ndarray) -> float:
    """||a - ref||_2 / ||ref||_2 over the whole array."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(a - ref) / np.linalg.norm(ref))
