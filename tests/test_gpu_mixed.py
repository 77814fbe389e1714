"""GPU parity of the mixed-radix rotation (HARP technical summary §2.1-2.2)
against the float64 oracle: the pages' 5120 = 8*8*8*5*2 schedule, the
layer dimensions of the workloads as mixed-radix products (11008, 12288,
28672), power-of-two and tiny odd schedules, both directions, float32 and
bf16.  The device blocks are the library's own expansion of seeded
parameters and fixed Gaussians (harp_mixed_expand: Cayley map, QR mixers,
float32); the oracle expands the same inputs itself in float64, so the bars
also cover the float32 rounding of the blocks.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import harp_oracle as O
from synth import workloads as S

pytestmark = pytest.mark.gpu

BUTTERFLY_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotated_bit_amd  # noqa: F401
    yield


def H():
    import rotated_bit_amd
    return rotated_bit_amd


def D():
    import devbuf
    return devbuf


def rng(*k):
    return np.random.default_rng(np.random.SeedSequence([3131, *k]))


def device_side(radices, seed, zero=False):
    """The device side: the library expands the seeded parameters and fixed
    Gaussians itself (harp_mixed_expand); the oracle expands the same inputs
    on its own, in float64, for the reference."""
    side = S.mixed_rotation(radices, rng(1, seed), mixer_seed=seed)
    params = [np.zeros_like(p) for p in side.params] if zero else side.params
    flat = H().harp_mixed_expand(radices, params, side.gaussians)
    R = H().MixedRotation(D().dev(flat), D().dev(side.sign_bits), radices)
    blocks64 = O.mixed_blocks(radices, params, side.gaussians)
    return R, blocks64, side.sign_bits


CASES = [
    ((8, 8, 8, 5, 2), 1, "bf16"), ((8, 8, 8, 5, 2), 17, "f32"), ((8, 8, 4, 43), 2, "bf16"),
    ((16, 16, 16, 3), 3, "bf16"), ((64, 64, 7), 2, "bf16"), ((2,) * 12, 5, "f32"),
    ((5, 3), 9, "f32"), ((3,), 4, "f32"), ((7, 2, 5, 3), 64, "bf16"), ((43, 4, 64), 1, "bf16"),
]


@pytest.mark.parametrize("radices,M,xdt", CASES)
def test_rotate_mixed_in_out(radices, M, xdt):
    d = D()
    R, blocks, signs = device_side(radices, 7)
    dim = R.dim
    x = S.activations(M, dim, rng(2, dim, M), xdt)
    xt = torch.empty((M, dim), dtype=torch.float32, device="cuda")
    H().harp_rotate_in_mixed(R, d.dev_x(x, xdt), xt)
    ref = O.mixed_forward(d.x_f64(x, xdt), radices, blocks, signs)
    r = O.rel_l2(d.host(xt), ref)
    print(f"[mixed in {radices} M={M}] rel_l2={r:.3e}", flush=True)
    assert r <= BUTTERFLY_TOL
    yp = rng(3, dim, M).normal(size=(M, dim)).astype(np.float32)
    y = torch.empty((M, dim), dtype=torch.float32, device="cuda")
    H().harp_rotate_out_mixed(R, d.dev(yp), y)
    reft = O.mixed_transpose(yp.astype(np.float64), radices, blocks, signs)
    r = O.rel_l2(d.host(y), reft)
    print(f"[mixed out {radices} M={M}] rel_l2={r:.3e}", flush=True)
    assert r <= BUTTERFLY_TOL
    # bf16 output rounds the float32 result
    yb = torch.empty((M, dim), dtype=torch.bfloat16, device="cuda")
    H().harp_rotate_out_mixed(R, d.dev(yp), yb)
    refb = O.bf16_round(reft)
    ulp = np.ldexp(1.0, np.frexp(np.abs(refb))[1] - 8)
    delta = BUTTERFLY_TOL * np.sqrt(np.mean(reft ** 2))
    assert np.all(np.abs(d.host(yb) - refb) <= ulp + delta)


def assert_bf16_of(got, ref64):
    """got = bf16 of a float32 result within the butterfly bar of ref64."""
    refb = O.bf16_round(ref64)
    ulp = np.ldexp(1.0, np.frexp(np.abs(refb))[1] - 8)
    delta = BUTTERFLY_TOL * np.sqrt(np.mean(ref64 ** 2))
    assert np.all(np.abs(got - refb) <= ulp + delta)
    assert np.mean(got != refb) < 0.01


WS_CASES = [((8, 8, 8, 5, 2), 1), ((8, 8, 4, 43), 3), ((64, 64, 7), 70), ((43, 4, 64), 2),
            ((5, 3), 9), ((3,), 4), ((8, 8, 8, 8, 7), 2)]


@pytest.mark.parametrize("radices,M", WS_CASES)
def test_rotate_mixed_bf16_workspace(radices, M):
    """bf16 outputs with a workspace (one launch per stage in float32, the
    last writing bf16) against the oracle and against the one-workgroup-per-
    row path without a workspace: both apply every block in the same float32
    order, so the bf16 outputs are equal."""
    d = D()
    R, blocks, signs = device_side(radices, 9)
    dim = R.dim
    ws = torch.empty(H().harp_rotate_mixed_workspace_bytes(dim, M, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    x = S.activations(M, dim, rng(5, dim, M), "bf16")
    xd = d.dev_x(x, "bf16")
    ref = O.mixed_forward(d.x_f64(x, "bf16"), radices, blocks, signs)
    a = torch.empty((M, dim), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((M, dim), dtype=torch.bfloat16, device="cuda")
    H().harp_rotate_in_mixed(R, xd, a, workspace=ws)
    H().harp_rotate_in_mixed(R, xd, b)
    assert_bf16_of(d.host(a), ref)
    assert torch.equal(a, b)
    yp = rng(6, dim, M).normal(size=(M, dim)).astype(np.float32)
    reft = O.mixed_transpose(yp.astype(np.float64), radices, blocks, signs)
    H().harp_rotate_out_mixed(R, d.dev(yp), a, workspace=ws)
    H().harp_rotate_out_mixed(R, d.dev(yp), b)
    assert_bf16_of(d.host(a), reft)
    assert torch.equal(a, b)


@pytest.mark.parametrize("radices", [(4, 4, 4, 4, 4, 4), (16, 8, 32)])
def test_rotate_mixed_zero_parameters_is_hadamard(radices):
    """theta = 0 with power-of-two radices: F x = H_d D x / sqrt(d) (scipy)."""
    d = D()
    R, _, signs = device_side(radices, 11, zero=True)
    dim = R.dim
    x = rng(4, dim).normal(size=(2, dim)).astype(np.float32)
    xt = torch.empty((2, dim), dtype=torch.float32, device="cuda")
    H().harp_rotate_in_mixed(R, d.dev(x), xt)
    Hd = scipy.linalg.hadamard(dim) / math.sqrt(dim)
    ref = (x.astype(np.float64) * O.decode_signs(signs, dim)) @ Hd.T
    assert O.rel_l2(d.host(xt), ref) <= BUTTERFLY_TOL


# The fused linear over mixed-radix sides.  Product paths and their rounding
# points follow the batch size as for the radix-2 fused linear: below 16 rows
# float32 throughout; up to 64 the codes enter the matrix cores exactly and
# only x~ is rounded to bf16; above, x~ and w_hat are both rounded.
FP32_PATH_TOL = 2e-5
MFMA_PATH_TOL = 3e-4
LINEAR_MIXED_CASES = [
    ((8, 8, 8, 5, 2), (8, 8, 8, 5, 2), 2, 1, "f32"),
    ((8, 8, 8, 5, 2), (8, 8, 8, 5, 2), 2, 5, "bf16"),
    ((8, 8, 8, 8), (8, 8, 4, 43), 4, 16, "f32"),     # 4096 -> 11008
    ((8, 8, 4, 43), (8, 8, 8, 8), 3, 40, "bf16"),    # 11008 -> 4096
    ((8, 8, 8, 5, 2), (16, 16, 20), 2, 100, "f32"),  # 5120 -> 5120, GEMM with split K
    ((64, 5), (40, 8), 2, 3, "bf16"),                # 320 -> 320, ragged tiles
    # decode batches: the workloads' schedules, a radix-43 stage, no
    # leading segment (64 x 64), twelve radix-2 stages
    ((8, 8, 8, 8), (8, 8, 4, 43), 2, 2, "bf16"),     # 4096 -> 11008
    ((8, 8, 4, 43), (8, 8, 8, 8), 4, 4, "f32"),      # 11008 -> 4096
    ((8, 8, 8, 8, 3), (8, 8, 8, 5, 2), 3, 1, "bf16"),  # 12288 -> 5120
    ((64, 64), (2,) * 12, 2, 3, "f32"),             # 4096 -> 4096
]


@pytest.mark.parametrize("rv,ru,bits,M,ydt", LINEAR_MIXED_CASES)
def test_linear_fused_mixed(rv, ru, bits, M, ydt):
    d = D()
    V, bv, sv = device_side(rv, 21)
    U, bu, su = device_side(ru, 22)
    K, N = V.dim, U.dim
    w = S.qweight(N, K, bits, rng(7, N, K, bits))
    W = d.dev_qweight(w)
    x = S.activations(M, K, rng(8, K, M), "bf16", S.outlier_channels(K, rng(9, K)))
    ws = torch.zeros(H().harp_linear_mixed_workspace_bytes(M, N, K), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    H().harp_linear_fused_mixed(V, W, U, d.dev_x(x, "bf16"), y, ws)
    # float32 x~ below 64 rows (the two-plane split from 16 on), bf16 x~ from
    # 64 on (w_hat exact up to 64 rows, bf16 above)
    contract = M >= 64
    ref = O.linear_mixed(d.x_f64(x, "bf16"), w.words, w.scale.view(np.float16),
                         w.zero.view(np.float16), bits, rv, bv, sv, ru, bu, su,
                         mfma_contract=contract, weights_exact=M <= 64)
    tol = MFMA_PATH_TOL if contract else FP32_PATH_TOL
    r = O.rel_l2(d.host(y), ref)
    print(f"[linear mixed {rv}->{ru} {bits}-bit M={M}] rel_l2={r:.3e}", flush=True)
    assert r <= tol
    # a second call on the same workspace (split-K counters left at zero)
    y2 = torch.empty_like(y)
    H().harp_linear_fused_mixed(V, W, U, d.dev_x(x, "bf16"), y2, ws)
    assert torch.equal(y, y2)
    if ydt == "bf16":
        # the bf16 output is the float32 result rounded to nearest even
        yb = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        H().harp_linear_fused_mixed(V, W, U, d.dev_x(x, "bf16"), yb, ws)
        assert torch.equal(yb, y.to(torch.bfloat16))


@pytest.mark.parametrize("M", [1, 2, 64])
def test_rotate_mixed_maximum_dim(M):
    """d = 32768 = 64 * 64 * 8, the largest mixed-radix side: float32 outputs
    (stage launches), bf16 with a workspace and bf16 without one (a whole row
    of 128 KB in LDS)."""
    radices = (64, 64, 8)
    d = D()
    R, blocks, signs = device_side(radices, 13)
    dim = R.dim
    x = S.activations(M, dim, rng(11, dim, M), "bf16")
    xd = d.dev_x(x, "bf16")
    ref = O.mixed_forward(d.x_f64(x, "bf16"), radices, blocks, signs)
    xt = torch.empty((M, dim), dtype=torch.float32, device="cuda")
    H().harp_rotate_in_mixed(R, xd, xt)
    assert O.rel_l2(d.host(xt), ref) <= BUTTERFLY_TOL
    ws = torch.empty(H().harp_rotate_mixed_workspace_bytes(dim, M, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    a = torch.empty((M, dim), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((M, dim), dtype=torch.bfloat16, device="cuda")
    H().harp_rotate_in_mixed(R, xd, a, workspace=ws)
    H().harp_rotate_in_mixed(R, xd, b)
    assert torch.equal(a, xt.to(torch.bfloat16))
    assert torch.equal(b, a)
    yp = rng(12, dim, M).normal(size=(M, dim)).astype(np.float32)
    reft = O.mixed_transpose(yp.astype(np.float64), radices, blocks, signs)
    y = torch.empty((M, dim), dtype=torch.float32, device="cuda")
    H().harp_rotate_out_mixed(R, d.dev(yp), y)
    assert O.rel_l2(d.host(y), reft) <= BUTTERFLY_TOL
