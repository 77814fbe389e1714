"""GPU parity: every entry point of include/harp.h against the float64 oracle.

Bars (each derived from the rounding points of its path):
* unpack / dequant (harp_dequant): bit-exact, float32 and bf16;
* butterfly alone, float32 in and out: relative L2 <= 1e-5;
* linear outputs: relative L2 <= 1e-3 over the whole output (the contract),
  and, because every rounding point of the path is modelled, also within
  FP32_PATH_TOL = 2e-5 (float32 accumulation error for K <= 28672).
All inputs come from the seeded generators in synth/.  Shapes run from tiny
ragged cases through the Llama/Qwen layer shapes at their real sizes;
where the oracle cannot finish a full layer quickly it computes sampled
output blocks or row chunks.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import harp_oracle as O
from synth import workloads as S

pytestmark = pytest.mark.gpu

CONTRACT_TOL = 1e-3
BUTTERFLY_TOL = 1e-5
FP32_PATH_TOL = 2e-5
# bf16 matrix-core path: the device rounds a float32 x~ to bf16, the oracle
# the float64 x~; values within the float32 error (<= 1e-5 relative, the
# butterfly bar) of a rounding boundary round one ulp apart.  Flip rate
# p <= 2e-5 / 2^-8 ~ 5e-3, each flip one ulp (2^-8 relative), so the
# output error is <= sqrt(p) 2^-8 ~ 2.8e-4.
MFMA_PATH_TOL = 3e-4
# The fused linear keeps x~ in float32 below BF16_MIN_M rows (the contract
# of the decode batches): the float32 product below 16 rows, then the
# small-batch matrix-core product on the exact two-plane bf16 split of x~
# (x~ kept to ~16 significant bits), both within the float32 bar of the
# unrounded oracle.  From BF16_MIN_M rows on x~ is rounded to bf16; up to
# SKINNY_MAX_M rows that product feeds the integer codes to the matrix cores
# and applies scale and zero per group (w_hat exact, only x~ rounded), above
# it rounds both x~ and w_hat to bf16.
BF16_MIN_M = 64
SKINNY_MAX_M = 64


def path_tol(M):
    return FP32_PATH_TOL if M < BF16_MIN_M else MFMA_PATH_TOL


def mode_for(M):
    """Rounding points of the product the fused linear runs at batch M."""
    if M < BF16_MIN_M:
        return "f32"
    return "mfma_exact_w" if M <= SKINNY_MAX_M else "mfma"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotated_bit_amd  # noqa: F401  (raises if libharp.so is missing)
    yield


def H():
    import rotated_bit_amd
    return rotated_bit_amd


def D():
    import devbuf
    return devbuf


def rng(*k):
    return np.random.default_rng(np.random.SeedSequence([977, *k]))


def assert_bf16_rounding_close(got, ref, fp32_tol):
    """got = bf16(float32 result), ref = float64 result.

    |bf16(a) - bf16(r)| <= ulp + |a - r| for a float32 value a of the float64
    value r, and |a - r| is bounded by the float32 bar of the path
    (fp32_tol of the RMS).  Rounding ties may flip in a few elements.
    """
    refb = O.bf16_round(ref)
    ulp = np.ldexp(1.0, np.frexp(np.abs(refb))[1] - 8)
    delta = fp32_tol * np.sqrt(np.mean(ref ** 2))
    assert np.all(np.abs(got - refb) <= ulp + delta)
    assert np.mean(got != refb) < 0.01


def report(name, got, ref):
    r = O.rel_l2(got, ref)
    rows = np.linalg.norm(got - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-300)
    print(f"[{name}] rel_l2={r:.3e} max_row={rows.max():.3e}", flush=True)
    return r


# ---------------------------------------------------------------------------
# a2: unpack + dequant, bit-exact
# ---------------------------------------------------------------------------

# "wide" weights: zero-points over the whole grid (0 and 2^B - 1 included)
# and fp16 scales from the smallest subnormal up
@pytest.mark.parametrize("bits,N,K,spread", [
    (2, 100, 320, "mid"), (3, 100, 320, "mid"), (4, 100, 320, "mid"),
    (2, 4096, 4096, "mid"), (3, 512, 8192, "mid"), (4, 512, 8192, "mid"),
    (2, 64, 28672, "mid"), (2, 100, 320, "wide"), (3, 512, 8192, "wide"),
    (4, 64, 28672, "wide"),
])
def test_dequant_bit_exact(bits, N, K, spread):
    w = S.qweight(N, K, bits, rng(1, bits, N, K), spread=spread)
    d = D()
    Wd = d.dev_qweight(w)
    ref = O.dequant(O.unpack(w.words, bits, K), d.scale_f16(w), d.zero_f16(w))
    out = torch.empty((N, K), dtype=torch.float32, device="cuda")
    H().harp_dequant(Wd, out)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)
    outb = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    H().harp_dequant(Wd, outb)
    got_bits = outb.view(torch.int16).cpu().numpy().view(np.uint16)
    ref_b = O.bf16_round(ref)
    assert np.array_equal(O.bf16_bits_to_f64(got_bits), ref_b)


# ---------------------------------------------------------------------------
# a1 / a5: butterfly in and out
# ---------------------------------------------------------------------------

ROT_CASES = [
    (2, 2, 5, "f32"), (4, 4, 3, "f32"), (8, 8, 7, "f32"), (48, 16, 9, "f32"),
    (256, 256, 4, "f32"), (512, 32, 33, "bf16"), (4096, 4096, 1, "bf16"),
    (4096, 4096, 17, "bf16"), (8192, 8192, 2, "bf16"), (11008, 256, 16, "bf16"),
    (28672, 256, 3, "bf16"), (12288, 256, 512, "bf16"), (4096, 4096, 512, "bf16"),
    (8192, 8192, 32, "bf16"),
    # blocks of 64..512 (one wave per block row, pairs staged in LDS), 1024
    # (workgroup barriers), and a ragged batch with four rows per slot
    (192, 64, 70, "f32"), (640, 128, 21, "bf16"), (1024, 512, 37, "f32"),
    (2048, 1024, 9, "bf16"), (28672, 256, 300, "f32"),
    # input rotation of up to 64 rows at b = 4096 / 8192 into float32: two
    # launches (sub-blocks, then the last three stages); 65 rows: one
    (8192, 4096, 3, "f32"), (4096, 4096, 64, "bf16"), (4096, 4096, 65, "f32"),
    (16384, 8192, 5, "bf16"),
]


@pytest.mark.parametrize("dim,b,M,xdt", ROT_CASES)
def test_rotate_in_out(dim, b, M, xdt):
    d = D()
    rot = S.rotation(dim, b, rng(2, dim, b))
    R = d.dev_rotation(rot)
    out_idx = S.outlier_channels(dim, rng(3, dim)) if dim >= 100 else None
    x = S.activations(M, dim, rng(4, dim, M), xdt, out_idx)
    xd = d.dev_x(x, xdt)
    x64 = d.x_f64(x, xdt)
    xt = torch.empty((M, dim), dtype=torch.float32, device="cuda")
    H().harp_rotate_in(R, xd, xt)
    ref = O.forward(x64, rot.cs, rot.sign_bits, b)
    assert report(f"rotate_in {dim}/{b} M={M}", d.host(xt), ref) <= BUTTERFLY_TOL
    # bf16 output: rounding of the float32 result; ties may flip vs float64
    xtb = torch.empty((M, dim), dtype=torch.bfloat16, device="cuda")
    H().harp_rotate_in(R, xd, xtb)
    assert_bf16_rounding_close(d.host(xtb), ref, BUTTERFLY_TOL)
    # transpose on a float32 y'
    yp = rng(5, dim, M).normal(size=(M, dim)).astype(np.float32)
    ypd = d.dev(yp)
    y = torch.empty((M, dim), dtype=torch.float32, device="cuda")
    H().harp_rotate_out(R, ypd, y)
    reft = O.transpose(yp.astype(np.float64), rot.cs, rot.sign_bits, b)
    assert report(f"rotate_out {dim}/{b} M={M}", d.host(y), reft) <= BUTTERFLY_TOL


ROT8_CASES = [
    (2, 2, 5, "f32"), (8, 8, 7, "f32"), (48, 16, 9, "f32"), (256, 256, 4, "f32"),
    (512, 32, 33, "bf16"), (4096, 4096, 1, "bf16"), (4096, 4096, 17, "bf16"),
    (8192, 8192, 1, "bf16"), (8192, 8192, 32, "bf16"), (11008, 256, 16, "bf16"),
    (12288, 256, 512, "bf16"), (4096, 4096, 512, "bf16"),
]


@pytest.mark.parametrize("dim,b,M,xdt", ROT8_CASES)
def test_rotate_int8_angles(dim, b, M, xdt):
    """int8-stored angles: the kernel's float32 table against the oracle's
    float64 decode of the same codes, both directions."""
    d = D()
    rot = S.rotation_q8(dim, b, rng(30, dim, b))
    R = d.dev_rotation(rot)
    cs = d.cs64(rot)
    x = S.activations(M, dim, rng(31, dim, M), xdt)
    xt = torch.empty((M, dim), dtype=torch.float32, device="cuda")
    H().harp_rotate_in(R, d.dev_x(x, xdt), xt)
    ref = O.forward(d.x_f64(x, xdt), cs, rot.sign_bits, b)
    assert report(f"rotate_in int8 {dim}/{b} M={M}", d.host(xt), ref) <= BUTTERFLY_TOL
    yp = rng(32, dim, M).normal(size=(M, dim)).astype(np.float32)
    y = torch.empty((M, dim), dtype=torch.float32, device="cuda")
    H().harp_rotate_out(R, d.dev(yp), y)
    reft = O.transpose(yp.astype(np.float64), cs, rot.sign_bits, b)
    assert report(f"rotate_out int8 {dim}/{b} M={M}", d.host(y), reft) <= BUTTERFLY_TOL


# Output rotations of up to 64 rows at b = 4096 / 8192 run split over eight
# workgroups per block; M = 65 is the first batch of the one-workgroup form.
SPLIT_CASES = [
    (4096, 4096, 1, "f32"), (4096, 4096, 8, "f32"), (4096, 4096, 9, "f32"),
    (8192, 8192, 3, "int8"), (8192, 4096, 5, "f32"), (16384, 8192, 2, "int8"),
    (4096, 4096, 4, "int8"), (4096, 4096, 64, "f32"), (4096, 4096, 65, "f32"),
    (8192, 8192, 33, "int8"),
]


@pytest.mark.parametrize("dim,b,M,angles", SPLIT_CASES)
def test_rotate_out_few_rows(dim, b, M, angles):
    """F^T y' for a few rows, float32 and bf16 outputs, both angle formats,
    block-diagonal sides included."""
    d = D()
    rot = (S.rotation if angles == "f32" else S.rotation_q8)(dim, b, rng(36, dim, b))
    R = d.dev_rotation(rot)
    cs = rot.cs if angles == "f32" else d.cs64(rot)
    yp = rng(37, dim, M).normal(size=(M, dim)).astype(np.float32)
    reft = O.transpose(yp.astype(np.float64), cs, rot.sign_bits, b)
    y = torch.empty((M, dim), dtype=torch.float32, device="cuda")
    H().harp_rotate_out(R, d.dev(yp), y)
    assert report(f"rotate_out {angles} {dim}/{b} M={M}", d.host(y), reft) <= BUTTERFLY_TOL
    yb = torch.empty((M, dim), dtype=torch.bfloat16, device="cuda")
    H().harp_rotate_out(R, d.dev(yp), yb)
    assert_bf16_rounding_close(d.host(yb), reft, BUTTERFLY_TOL)


@pytest.mark.parametrize("b", [16, 4096])
def test_rotate_int8_extreme_codes(b):
    """Codes 0 (Hadamard initialisation) and +-127 at step pi/508 (pair swap
    and pair negation), and the int8 extremes -128 / 127 at a large step."""
    d = D()
    L = b.bit_length() - 1
    x = rng(33, b).normal(size=(2, b)).astype(np.float32)
    for code, step in ((0, 0.3), (127, math.pi / 508), (-127, math.pi / 508),
                       (-128, 0.05), (127, 0.05)):
        rot = S.rotation_q8(b, b, rng(34, b, code + 128),
                            codes=np.full((1, L, b // 2), code), step=step)
        xt = torch.empty((2, b), dtype=torch.float32, device="cuda")
        H().harp_rotate_in(d.dev_rotation(rot), d.dev(x), xt)
        ref = O.forward(x.astype(np.float64), d.cs64(rot), rot.sign_bits, b)
        assert report(f"int8 code {code} b={b}", d.host(xt), ref) <= BUTTERFLY_TOL
        if code == 0:
            Hm = scipy.linalg.hadamard(b) / math.sqrt(b)
            rht = (x.astype(np.float64) * O.decode_signs(rot.sign_bits, b)) @ Hm.T
            assert O.rel_l2(d.host(xt), rht) <= BUTTERFLY_TOL


@pytest.mark.parametrize("b", [256, 4096, 8192])
def test_rotate_in_at_init_is_randomized_hadamard(b):
    """Zero-initialised angles: the kernel computes H D x / sqrt(b) (scipy H)."""
    d = D()
    L = b.bit_length() - 1
    rot = S.rotation(b, b, rng(6, b), theta=np.full((1, L, b // 2), math.pi / 4))
    x = rng(7, b).normal(size=(3, b)).astype(np.float32)
    xt = torch.empty((3, b), dtype=torch.float32, device="cuda")
    H().harp_rotate_in(d.dev_rotation(rot), d.dev(x), xt)
    Hm = scipy.linalg.hadamard(b).astype(np.float64)
    ref = (x.astype(np.float64) * O.decode_signs(rot.sign_bits, b)) @ Hm.T / math.sqrt(b)
    assert report(f"rht {b}", d.host(xt), ref) <= BUTTERFLY_TOL


def test_rotate_max_batch_sampled():
    """M = 65536 rows (the ABI maximum) on a 256-wide side; sampled rows."""
    d = D()
    dim, b, M = 256, 256, 65536
    rot = S.rotation(dim, b, rng(8))
    x = S.activations(M, dim, rng(9), "bf16")
    xt = torch.empty((M, dim), dtype=torch.float32, device="cuda")
    H().harp_rotate_in(d.dev_rotation(rot), d.dev_x(x, "bf16"), xt)
    rows = np.unique(np.concatenate([rng(10).integers(0, M, 64), [0, M - 1]]))
    got = xt[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    ref = O.forward(O.bf16_bits_to_f64(x[rows]), rot.cs, rot.sign_bits, b)
    assert report("rotate max M", got, ref) <= BUTTERFLY_TOL


# ---------------------------------------------------------------------------
# a3: GEMV (float32), a4: GEMM (bf16 matrix cores)
# ---------------------------------------------------------------------------

GEMV_CASES = [(100, 320, b, m, "mid") for b in (2, 3, 4) for m in (1, 2, 3, 5, 8, 9, 13)] + [
    (4096, 4096, 2, 1, "mid"), (11008, 4096, 2, 16, "mid"), (4096, 11008, 2, 16, "mid"),
    (8192, 8192, 3, 1, "mid"), (2048, 8192, 4, 32, "mid"), (1000, 28672, 2, 1, "mid"),
    (64, 256, 2, 63, "mid"),
    (4096, 4096, 2, 1, "wide"), (100, 320, 3, 9, "wide"), (2048, 8192, 4, 5, "wide"),
]


@pytest.mark.parametrize("N,K,bits,M,spread", GEMV_CASES)
def test_gemv(N, K, bits, M, spread):
    d = D()
    w = S.qweight(N, K, bits, rng(11, N, K, bits), spread=spread)
    xt = rng(12, K, M).normal(size=(M, K)).astype(np.float32)
    yt = torch.empty((M, N), dtype=torch.float32, device="cuda")
    H().harp_deq_gemv(d.dev_qweight(w), d.dev(xt), yt)
    w_hat = O.dequant(O.unpack(w.words, bits, K), d.scale_f16(w), d.zero_f16(w))
    ref = xt.astype(np.float64) @ w_hat.T
    r = report(f"gemv {N}x{K} b{bits} M={M} {spread}", d.host(yt), ref)
    assert r <= CONTRACT_TOL and r <= FP32_PATH_TOL


# Full-width decode products checked on sampled output features: strips of
# two 16-feature tiles (N >= 16384) with a ragged last strip, several
# four-group blocks per wave, uneven wave ranges (K / 64 not a multiple of
# 8), both product kernels (M = 1, 2 and 3-bit: vector ALU; M = 3..8 at 2
# and 4 bits: matrix cores on the bf16 planes of x~).
WIDE_GEMV_CASES = [(16400, 8192, 2, 3), (16400, 8192, 4, 5), (16400, 8192, 4, 8),
                   (16400, 4160, 2, 6), (16400, 8192, 2, 1), (16400, 8192, 4, 2),
                   (4100, 8192, 4, 4), (16400, 4160, 3, 5), (16400, 8192, 2, 7),
                   # one row over more than 1024 row blocks: a persistent grid
                   # of 512 workgroups, each taking several blocks (ragged
                   # last block, a partial second chunk, odd item counts)
                   (16420, 4160, 3, 1), (28680, 4096, 4, 1)]


@pytest.mark.parametrize("N,K,bits,M", WIDE_GEMV_CASES)
def test_gemv_wide_sampled(N, K, bits, M):
    d = D()
    w = S.qweight(N, K, bits, rng(13, N, K, bits, M))
    xt = rng(14, K, M).normal(size=(M, K)).astype(np.float32)
    yt = torch.empty((M, N), dtype=torch.float32, device="cuda")
    H().harp_deq_gemv(d.dev_qweight(w), d.dev(xt), yt)
    edges = [0, 1, 15, 16, 31, 32, 33, 63, 64, N // 2, N - 17, N - 16, N - 2, N - 1]
    rows = np.unique(np.concatenate([edges, rng(15, N).integers(0, N, 96)]))
    w_hat = O.dequant(O.unpack(w.words[rows], bits, K), d.scale_f16(w)[rows],
                      d.zero_f16(w)[rows])
    ref = xt.astype(np.float64) @ w_hat.T
    r = report(f"gemv wide {N}x{K} b{bits} M={M}", d.host(yt)[:, rows], ref)
    assert r <= CONTRACT_TOL and r <= FP32_PATH_TOL


ROTGEMV_CASES = [
    (256, 256, 8, 2, 1, "f32", "f32"), (300, 256, 16, 3, 3, "int8", "bf16"),
    (4096, 4096, 4096, 2, 1, "f32", "bf16"), (4096, 4096, 4096, 2, 1, "int8", "bf16"),
    (11008, 4096, 4096, 4, 2, "int8", "bf16"), (100, 1024, 64, 2, 4, "f32", "f32"),
    (513, 2048, 2048, 3, 4, "int8", "bf16"), (64, 64, 64, 4, 1, "f32", "bf16"),
]


@pytest.mark.parametrize("N,K,b,bits,M,angles,xdt", ROTGEMV_CASES)
def test_rotate_in_deq_gemv(N, K, b, bits, M, angles, xdt):
    """y' = w_hat (F_V x) in one launch against the oracle's two steps."""
    d = D()
    draw = S.rotation if angles == "f32" else S.rotation_q8
    rot = draw(K, b, rng(40, K, b))
    w = S.qweight(N, K, bits, rng(41, N, K, bits))
    x = S.activations(M, K, rng(42, K, M), xdt)
    yt = torch.empty((M, N), dtype=torch.float32, device="cuda")
    H().harp_rotate_in_deq_gemv(d.dev_rotation(rot), d.dev_qweight(w), d.dev_x(x, xdt), yt)
    xt = O.forward(d.x_f64(x, xdt), d.cs64(rot), rot.sign_bits, b)
    w_hat = O.dequant(O.unpack(w.words, bits, K), d.scale_f16(w), d.zero_f16(w))
    ref = xt @ w_hat.T
    r = report(f"rotate_in_deq_gemv {N}x{K} b={b} bits={bits} M={M} {angles}", d.host(yt), ref)
    assert r <= CONTRACT_TOL and r <= FP32_PATH_TOL


GEMM_CASES = [
    # M <= 64: the small-batch kernel (16 features per workgroup)
    (100, 320, 2, 16, "mid"), (300, 256, 3, 33, "mid"), (257, 128, 4, 1, "mid"),
    (4096, 4096, 2, 16, "mid"), (4096, 4096, 2, 32, "mid"), (11008, 4096, 2, 16, "mid"),
    (4096, 11008, 4, 48, "mid"), (1024, 28672, 3, 32, "mid"), (2000, 8192, 2, 5, "mid"),
    (1000, 1088, 4, 64, "mid"), (64, 64, 2, 17, "mid"),
    # M <= 64 on wide strips (K a multiple of 4096, N >= 8192): 32 and 64
    # features per wave, ragged row tiles
    (8192, 4096, 2, 64, "mid"), (16384, 4096, 3, 33, "wide"), (16384, 4096, 4, 1, "mid"),
    (8200, 8192, 2, 17, "wide"),
    # M > 64: 128 x 128 tiles, optionally split K
    (300, 256, 3, 65, "mid"), (128, 64, 2, 200, "mid"),
    (4096, 4096, 2, 512, "mid"), (12288, 4096, 4, 512, "mid"), (4096, 12288, 2, 512, "mid"),
    (4096, 4096, 3, 129, "mid"), (1000, 1088, 2, 300, "mid"), (384, 2048, 4, 64, "mid"),
    # zero-points at 0 and 2^B - 1, subnormal fp16 scales
    (4096, 4096, 2, 16, "wide"), (300, 256, 3, 33, "wide"), (1000, 1088, 4, 64, "wide"),
    (4096, 4096, 4, 512, "wide"), (1000, 1088, 3, 300, "wide"),
]


@pytest.mark.parametrize("N,K,bits,M,spread", GEMM_CASES)
def test_gemm(N, K, bits, M, spread):
    """One K slice (no workspace) and split K (workspace) against the oracle;
    the split result is bitwise reproducible and its counters return to 0."""
    d = D()
    w = S.qweight(N, K, bits, rng(13, N, K, bits), spread=spread)
    xt = S.activations(M, K, rng(14, K, M), "bf16")
    Wd, xd = d.dev_qweight(w), d.dev(xt)
    w_hat = O.dequant(O.unpack(w.words, bits, K), d.scale_f16(w), d.zero_f16(w))
    if M > SKINNY_MAX_M:      # the tiled product rounds w_hat to bf16
        w_hat = O.bf16_round(w_hat)
    ref = O.bf16_bits_to_f64(xt) @ w_hat.T
    yt = torch.empty((M, N), dtype=torch.float32, device="cuda")
    H().harp_deq_gemm(Wd, xd, yt)
    y_again = torch.empty_like(yt)
    H().harp_deq_gemm(Wd, xd, y_again)
    torch.cuda.synchronize()
    assert torch.equal(yt, y_again)
    r = report(f"gemm {N}x{K} b{bits} M={M} {spread}", d.host(yt), ref)
    assert r <= CONTRACT_TOL and r <= FP32_PATH_TOL
    ws = d.gemm_workspace(M, N, K)
    if ws is not None:
        y1 = torch.empty_like(yt)
        y2 = torch.empty_like(yt)
        H().harp_deq_gemm(Wd, xd, y1, ws)
        H().harp_deq_gemm(Wd, xd, y2, ws)
        r = report(f"gemm split-K {N}x{K} b{bits} M={M}", d.host(y1), ref)
        assert r <= CONTRACT_TOL and r <= FP32_PATH_TOL
        torch.cuda.synchronize()
        assert torch.equal(y1, y2)
        counters = ws[:2048].view(torch.int32)   # fixed front area, left at zero
        assert int(counters.abs().sum().item()) == 0


# ---------------------------------------------------------------------------
# a6: the whole linear
# ---------------------------------------------------------------------------

def oracle_linear_rows(li, x64, mode, blocks=None, chunk=2048):
    """Oracle linear composed from oracle steps; output-side blocks optional.

    mode: "f32" (no rounding), "mfma" (x~ and w_hat rounded to bf16) or
    "mfma_exact_w" (only x~ rounded).  y' rows are produced in chunks so that
    large layers fit in memory.  When ``blocks`` is given, only those output
    blocks (of size b_U; independent because U is block-diagonal) are
    produced.  Returns (y, output columns).
    """
    assert mode in ("f32", "mfma", "mfma_exact_w")
    lin, w = li.lin, li.W
    xt = O.forward(x64, D().cs64(li.V), li.V.sign_bits, lin.b_v)
    if mode != "f32":
        xt = O.bf16_round(xt)
    bu = lin.b_u
    full = blocks is None
    blocks = list(range(lin.N // bu)) if full else list(blocks)
    rows = np.concatenate([np.arange(j * bu, (j + 1) * bu) for j in blocks])
    yp = np.empty((x64.shape[0], len(rows)))
    s16, z16 = w.scale.view(np.float16), w.zero.view(np.float16)
    for c0 in range(0, len(rows), chunk):
        rr = rows[c0:c0 + chunk]
        wh = O.dequant(O.unpack(w.words[rr], w.bits, lin.K), s16[rr], z16[rr])
        if mode == "mfma":
            wh = O.bf16_round(wh)
        yp[:, c0:c0 + len(rr)] = xt @ wh.T
    cs_u = D().cs64(li.U)
    if full:
        return O.transpose(yp, cs_u, li.U.sign_bits, bu), rows
    assert bu % 32 == 0
    wpb = bu // 32
    y = np.empty_like(yp)
    for i, j in enumerate(blocks):
        sl = slice(i * bu, (i + 1) * bu)
        sb = li.U.sign_bits[j * wpb:(j + 1) * wpb]
        y[:, sl] = O.transpose(yp[:, sl], cs_u[j:j + 1], sb, bu)
    return y, rows


def run_fused(li, y_dtype=torch.float32):
    d = D()
    lin = li.lin
    V, U, W = d.dev_rotation(li.V), d.dev_rotation(li.U), d.dev_qweight(li.W)
    x = d.dev_x(li.x, li.x_dtype)
    y = torch.empty((li.M, lin.N), dtype=y_dtype, device="cuda")
    ws = d.workspace(li.M, lin.N, lin.K)
    H().harp_linear_fused(V, W, U, x, y, ws)
    return y


FUSED_CASES = [("tiny", 0, 2, 4), ("l7b_decode", 0, 2, 1), ("l7b_decode", 0, 2, 16),
               ("l7b_decode", 0, 2, 33), ("l7b_decode", 0, 3, 48), ("l7b_decode", 0, 4, 63),
               ("l7b_decode", 0, 2, 64)]
FUSED_CASES += [("l7b_mlp", i, 2, m) for i in (0, 1) for m in (1, 16)]
FUSED_CASES += [("q8b_prefill", i, b, 512) for i in (0, 1, 2) for b in (2, 4)]


@pytest.mark.parametrize("cfg,lin,bits,M", FUSED_CASES)
def test_fused_configs(cfg, lin, bits, M):
    c = S.CONFIGS[cfg]
    li = S.layer_inputs(c, lin, bits, M)
    y = D().host(run_fused(li))
    ref, _ = oracle_linear_rows(li, D().x_f64(li.x, li.x_dtype), mode_for(M))
    r = report(f"fused {cfg}[{lin}] b{bits} M={M}", y, ref)
    assert r <= CONTRACT_TOL
    assert r <= path_tol(M)


L70B_CASES = [(0, 2), (0, 3), (0, 4), (1, 2), (1, 3), (1, 4), (2, 2), (2, 3), (2, 4)]


FUSED8_CASES = [("tiny", 0, 2, 4), ("l7b_decode", 0, 2, 1), ("l7b_mlp", 1, 2, 16),
                ("l7b_mlp", 0, 2, 1), ("q8b_prefill", 0, 2, 512), ("q8b_prefill", 2, 4, 512)]


@pytest.mark.parametrize("cfg,lin,bits,M", FUSED8_CASES)
def test_fused_int8_angles(cfg, lin, bits, M):
    li = S.layer_inputs(S.CONFIGS[cfg], lin, bits, M, angles="int8")
    y = D().host(run_fused(li))
    ref, _ = oracle_linear_rows(li, D().x_f64(li.x, li.x_dtype), mode_for(M))
    r = report(f"fused int8 angles {cfg}[{lin}] b{bits} M={M}", y, ref)
    assert r <= CONTRACT_TOL
    assert r <= path_tol(M)


@pytest.mark.parametrize("lin,bits", L70B_CASES)
def test_fused_l70b_slice(lin, bits):
    """Llama-70B slice at M = 1 and 32, 2/3/4 bits.  8192 -> 28672 checks 13
    sampled 256-wide output blocks; 28672 -> 8192 (b = 8192 output side, so
    every output needs all 8192 rows) is checked in full."""
    c = S.CONFIGS["l70b_slice"]
    lis = [S.layer_inputs(c, lin, bits, M) for M in c.Ms]
    ys = [D().host(run_fused(li)) for li in lis]
    L0 = lis[0].lin
    blocks = None
    if L0.N // L0.b_u > 16:
        nb = L0.N // L0.b_u
        blocks = sorted(set(rng(20, lin, bits).integers(0, nb, 12).tolist()) | {nb - 1})
    # one oracle pass per batch: M = 1 takes the float32 product, M = 32 the
    # matrix-core product on the two-plane split of the float32 x~; both
    # against the unrounded oracle
    for li, y in zip(lis, ys):
        ref, rows = oracle_linear_rows(li, D().x_f64(li.x, li.x_dtype), mode_for(li.M),
                                       blocks)
        r = report(f"fused l70b[{lin}] b{bits} M={li.M}", y[:, rows], ref)
        assert r <= CONTRACT_TOL and r <= path_tol(li.M)


@pytest.mark.parametrize("b_v,M,angles,xdt", [
    (4, 1, "f32", "bf16"), (8, 1, "f32", "bf16"), (8, 3, "int8", "f32"),
    (64, 2, "int8", "bf16"), (512, 4, "f32", "f32"), (4096, 1, "int8", "bf16"),
    (4096, 4, "f32", "bf16"), (2048, 2, "f32", "bf16"),
])
def test_fused_decode_input_blocks(b_v, M, angles, xdt):
    """Small batches over the input-side block sizes: b >= 8 takes the
    single-launch input rotation, b = 4 the separate rotation kernel."""
    cfg = S.Config(10, "dec", (S.Linear("d", 4096, 768, b_v, 256),), (2,), (M,), x_dtype=xdt)
    li = S.layer_inputs(cfg, 0, 2, M, angles=angles)
    ref, _ = oracle_linear_rows(li, D().x_f64(li.x, xdt), "f32")
    y = D().host(run_fused(li))
    r = report(f"decode b_v={b_v} M={M} {angles} {xdt}", y, ref)
    assert r <= CONTRACT_TOL and r <= FP32_PATH_TOL


@pytest.mark.parametrize("M,angles_v,angles_u", [
    (1, "f32", "f32"), (3, "int8", "int8"), (4, "f32", "f32"),
    (1, "int8", "f32"), (2, "f32", "int8"),
])
def test_fused_decode_mixed_angle_formats(M, angles_v, angles_u):
    """Decode linear with each side's angles in either format: oracle parity
    and two calls on one workspace bitwise equal."""
    cfg = S.Config(11, "mix", (S.Linear("t", 2048, 4096, 2048, 4096),), (2,), (M,))
    base = S.layer_inputs(cfg, 0, 2, M, angles=angles_v)
    other = S.layer_inputs(cfg, 0, 2, M, angles=angles_u)
    li = S.LayerInputs(base.lin, 2, M, base.x, base.x_dtype, base.V, other.U, base.W)
    d = D()
    V, U, W = d.dev_rotation(li.V), d.dev_rotation(li.U), d.dev_qweight(li.W)
    x = d.dev_x(li.x, li.x_dtype)
    ws = d.workspace(M, 4096, 2048)
    y1 = torch.empty((M, 4096), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y1)
    H().harp_linear_fused(V, W, U, x, y1, ws)
    H().harp_linear_fused(V, W, U, x, y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    ref, _ = oracle_linear_rows(li, d.x_f64(li.x, li.x_dtype), "f32")
    r = report(f"decode M={M} V {angles_v} U {angles_u}", d.host(y1), ref)
    assert r <= CONTRACT_TOL and r <= FP32_PATH_TOL


@pytest.mark.parametrize("M", [0, 1, 2, 3, 4, 5, 7, 63, 64, 65, 100])
def test_fused_batch_edges_and_bf16_out(M):
    """Ragged batches around the GEMV/GEMM switch, bf16 output, empty input."""
    cfg = S.Config(9, "edge", (S.Linear("e", 256, 512, 16, 256),), (3,), (M,))
    li = S.layer_inputs(cfg, 0, 3, M)
    if M == 0:
        d = D()
        y = torch.full((1, 512), 7.0, device="cuda")
        H().harp_linear_fused(d.dev_rotation(li.V), d.dev_qweight(li.W),
                              d.dev_rotation(li.U), d.dev_x(li.x, "bf16"), y,
                              d.workspace(1, 512, 256), M=0)
        assert torch.all(y == 7.0)
        return
    ref, _ = oracle_linear_rows(li, D().x_f64(li.x, "bf16"), mode_for(M))
    y = D().host(run_fused(li))
    r = report(f"edge M={M}", y, ref)
    assert r <= CONTRACT_TOL and r <= path_tol(M)
    assert_bf16_rounding_close(D().host(run_fused(li, torch.bfloat16)), ref,
                               path_tol(M))


@pytest.mark.parametrize("M,bits", [(1, 2), (3, 4), (9, 3), (16, 2), (40, 4), (63, 3),
                                    (64, 2), (100, 4)])
def test_fused_wide_weights(M, bits):
    """Zero-points at 0 and 2^B - 1 and subnormal fp16 scales through every
    product of the fused linear (2048 -> 4096, b = 2048 / 4096)."""
    cfg = S.Config(12, "wide", (S.Linear("w", 2048, 4096, 2048, 4096),), (bits,), (M,))
    li = S.layer_inputs(cfg, 0, bits, M)
    w = S.qweight(4096, 2048, bits, rng(50, M, bits), spread="wide")
    li = S.LayerInputs(li.lin, bits, M, li.x, li.x_dtype, li.V, li.U, w)
    ref, _ = oracle_linear_rows(li, D().x_f64(li.x, li.x_dtype), mode_for(M))
    y = D().host(run_fused(li))
    r = report(f"fused wide weights M={M} b{bits}", y, ref)
    assert r <= CONTRACT_TOL and r <= path_tol(M)


def test_fused_workspace_reused_across_shapes():
    """One workspace, sized for the largest call and zero-filled once, serves
    M = 512, then 128, then 512 and 16 on the same 4096 x 4096 layer: the split-K
    counters sit at a fixed offset, so no call sees another's leftovers."""
    c = S.CONFIGS["q8b_prefill"]
    Ms = (512, 128, 512, 16, 128)
    lis = {M: S.layer_inputs(c, 0, 2, M) for M in set(Ms)}
    d = D()
    nbytes = max(H().harp_linear_workspace_bytes(M, 4096, 4096) for M in Ms)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    base = lis[512]
    V, U, W = d.dev_rotation(base.V), d.dev_rotation(base.U), d.dev_qweight(base.W)
    refs = {}
    for M in Ms:
        li = lis[M]
        li = S.LayerInputs(base.lin, 2, M, li.x, li.x_dtype, base.V, base.U, base.W)
        y = torch.empty((M, 4096), dtype=torch.float32, device="cuda")
        H().harp_linear_fused(V, W, U, d.dev_x(li.x, li.x_dtype), y, ws)
        if M not in refs:
            refs[M] = oracle_linear_rows(li, d.x_f64(li.x, li.x_dtype), mode_for(M))[0]
        r = report(f"reused workspace M={M}", d.host(y), refs[M])
        assert r <= CONTRACT_TOL and r <= path_tol(M)
    torch.cuda.synchronize()
    assert int(ws[:2048].view(torch.int32).abs().sum().item()) == 0


@pytest.mark.parametrize("M", [1, 16, 512])
def test_fused_deterministic(M):
    c = S.CONFIGS["q8b_prefill"] if M == 512 else S.CONFIGS["l7b_mlp"]
    li = S.layer_inputs(c, 1 if M == 512 else 0, 2, M)
    a = run_fused(li)
    b = run_fused(li)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
