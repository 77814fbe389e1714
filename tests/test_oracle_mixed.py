"""Pins for the oracle's mixed-radix stages (HARP technical summary §2.1-2.2).

Each check ties the oracle to something other than itself: the Cayley map's
2x2 closed form and orthogonality, the QR factorisation's defining
properties, scipy's Sylvester Hadamard at zero parameters, the pinned
radix-2 butterfly for the all-2 schedule, and a dense matrix built by
enumerating mixed-radix digits with divmod.
"""
import math

import numpy as np
import pytest
import scipy.linalg

from oracle import harp_oracle as O
from synth import workloads as S

rng0 = np.random.default_rng(777)


def random_signs(d, rng):
    bits = rng.integers(0, 2 ** 32, size=(d + 31) // 32, dtype=np.uint64).astype(np.uint32)
    if d % 32:
        bits[-1] &= np.uint32((1 << (d % 32)) - 1)
    return bits


def zero_params(radices):
    d = int(np.prod(radices))
    return [np.zeros((d // b, b * (b - 1) // 2)) for b in radices]


def random_params(radices, rng, scale=0.3):
    d = int(np.prod(radices))
    return [rng.normal(0, scale, size=(d // b, b * (b - 1) // 2)) for b in radices]


def test_cayley_closed_form_2x2():
    for a in (0.0, 0.3, -1.7, 5.0):
        A = np.array([[0.0, a], [-a, 0.0]])
        Q = O.cayley(A)
        ref = np.array([[1 - a * a, -2 * a], [2 * a, 1 - a * a]]) / (1 + a * a)
        assert np.allclose(Q, ref, atol=1e-14, rtol=0)


@pytest.mark.parametrize("b", [3, 5, 8, 16])
def test_cayley_orthogonal_and_identity_at_zero(b):
    A = O.skew_from_params(rng0.normal(size=b * (b - 1) // 2), b)
    Q = O.cayley(A)
    assert np.allclose(Q @ Q.T, np.eye(b), atol=1e-12)
    assert abs(np.linalg.det(Q) - 1.0) < 1e-10
    assert np.array_equal(O.cayley(np.zeros((b, b))), np.eye(b))


def test_skew_from_params_layout():
    A = O.skew_from_params(np.array([1.0, 2.0, 3.0]), 3)
    assert np.array_equal(A, np.array([[0, 1, 2], [-1, 0, 3], [-2, -3, 0.0]]))
    with pytest.raises(ValueError):
        O.cayley(np.array([[0.0, 1.0], [1.0, 0.0]]))


@pytest.mark.parametrize("b", [3, 5, 7, 43])
def test_qr_mixer_is_the_unique_qr_factor(b):
    g = S.mixer_gaussian(b, 11)
    G = O.qr_mixer(g)
    R = G.T @ g
    assert np.allclose(G @ G.T, np.eye(b), atol=1e-12)
    assert np.allclose(np.tril(R, -1), 0.0, atol=1e-12)      # upper triangular
    assert np.all(np.diag(R) > 0)                             # positive diagonal
    assert np.array_equal(G, O.qr_mixer(S.mixer_gaussian(b, 11)))   # fixed
    with pytest.raises(ValueError):
        O.base_mixer(b)                                       # needs its Gaussian


@pytest.mark.parametrize("b", [2, 4, 8, 64])
def test_base_mixer_power_of_two_is_sylvester(b):
    assert np.allclose(O.base_mixer(b), scipy.linalg.hadamard(b) / math.sqrt(b),
                       atol=1e-15, rtol=0)


@pytest.mark.parametrize("radices", [(4, 4), (2, 8), (8, 2, 4), (16, 16), (4, 2, 2, 8)])
def test_zero_parameters_give_sylvester_hadamard(radices):
    """theta = 0, power-of-two radices: F = H_d D / sqrt(d) exactly."""
    d = int(np.prod(radices))
    signs = random_signs(d, rng0)
    blocks = O.mixed_blocks(radices, zero_params(radices))
    x = rng0.normal(size=(3, d))
    Hd = scipy.linalg.hadamard(d) / math.sqrt(d)
    ref = (x * O.decode_signs(signs, d)) @ Hd.T
    assert np.allclose(O.mixed_forward(x, radices, blocks, signs), ref, atol=1e-12, rtol=0)


def test_all_two_schedule_is_the_radix2_butterfly():
    L, d = 6, 64
    radices = (2,) * L
    params = random_params(radices, rng0)
    blocks = O.mixed_blocks(radices, params)
    signs = random_signs(d, rng0)
    # the radix-2 format: (cos t, sin t) with t = pi/4 + phi, [1][L][d/2]
    t = math.pi / 4 + np.stack([params[s][:, 0] for s in range(L)])[None]
    cs = np.stack([np.cos(t), np.sin(t)], axis=-1)
    x = rng0.normal(size=(2, d))
    assert np.allclose(O.mixed_forward(x, radices, blocks, signs), O.forward(x, cs, signs, d),
                       atol=1e-13, rtol=0)


def dense_by_enumeration(radices, blocks, signs):
    """F as an explicit product of d x d stage matrices, built index by index."""
    d = int(np.prod(radices))
    F = np.diag(O.decode_signs(signs, d))
    stride = 1
    for t, b in enumerate(radices):
        S = np.zeros((d, d))
        for i in range(d):
            lo = i % stride
            digit = (i // stride) % b
            hi = i // (stride * b)
            c = lo + stride * hi
            for j in range(b):
                src = lo + stride * j + stride * b * hi
                S[i, src] = blocks[t][c][digit][j]
        F = S @ F
        stride *= b
    return F


@pytest.mark.parametrize("radices", [(3, 2, 5), (5, 3), (2, 7, 2), (4, 3)])
def test_dense_brute_force_and_transpose(radices):
    d = int(np.prod(radices))
    params = random_params(radices, rng0)
    blocks = O.mixed_blocks(radices, params, S.mixer_gaussians(radices, 5))
    signs = random_signs(d, rng0)
    F = dense_by_enumeration(radices, blocks, signs)
    x = rng0.normal(size=(4, d))
    assert np.allclose(O.mixed_forward(x, radices, blocks, signs), x @ F.T, atol=1e-12, rtol=0)
    assert np.allclose(O.mixed_transpose(x, radices, blocks, signs), x @ F, atol=1e-12, rtol=0)
    assert np.allclose(F @ F.T, np.eye(d), atol=1e-12)


def test_paper_schedule_5120_orthogonal():
    """The pages' example 5120 = 8 * 8 * 8 * 5 * 2: norm preserved, the
    transpose inverts the forward map."""
    radices = (8, 8, 8, 5, 2)
    params = random_params(radices, rng0, 0.1)
    blocks = O.mixed_blocks(radices, params, S.mixer_gaussians(radices))
    signs = random_signs(5120, rng0)
    x = rng0.normal(size=(2, 5120))
    y = O.mixed_forward(x, radices, blocks, signs)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    assert np.allclose(O.mixed_transpose(y, radices, blocks, signs), x, atol=1e-12)


def packed_weight(N, K, bits, rng):
    """Random codes, scales and zeros in the packed format (the packer is
    pinned to hand-derived layout fixtures elsewhere)."""
    qmax = (1 << bits) - 1
    q = rng.integers(0, qmax + 1, size=(N, K))
    scale = (rng.uniform(0.5, 1.5, size=(N, K // 64)) * 0.01).astype(np.float16)
    zero = rng.integers(0, qmax + 1, size=(N, K // 64)).astype(np.float16)
    return O.pack(q, bits), scale, zero, q


def test_linear_mixed_all_two_is_linear():
    """Radix-2 schedules on both sides reproduce the radix-2 linear exactly."""
    K, N, bits = 64, 128, 3
    rv, ru = (2,) * 6, (2,) * 7
    pv, pu = random_params(rv, rng0), random_params(ru, rng0)
    sv, su = random_signs(K, rng0), random_signs(N, rng0)
    words, scale, zero, _ = packed_weight(N, K, bits, rng0)
    cs = []
    for radices, params in ((rv, pv), (ru, pu)):
        t = math.pi / 4 + np.stack([params[s][:, 0] for s in range(len(radices))])[None]
        cs.append(np.stack([np.cos(t), np.sin(t)], axis=-1))
    x = rng0.normal(size=(3, K))
    for contract in (False, True):
        got = O.linear_mixed(x, words, scale, zero, bits, rv,
                             O.mixed_blocks(rv, pv, S.mixer_gaussians(rv)), sv,
                             ru, O.mixed_blocks(ru, pu, S.mixer_gaussians(ru)), su,
                             mfma_contract=contract)
        ref = O.linear(x, words, scale, zero, bits, cs[0], sv, K, cs[1], su, N,
                       mfma_contract=contract)
        assert np.allclose(got, ref, atol=1e-12, rtol=0)


def test_linear_mixed_dense_composition():
    """y = F_U^T W_hat F_V x with F built by digit enumeration and W_hat
    decoded code by code (q - z) s."""
    rv, ru = (4, 4, 4), (5, 2, 3, 4)                # K = 64 (one quantization group)
    K, N, bits = 64, int(np.prod(ru)), 4
    pv, pu = random_params(rv, rng0), random_params(ru, rng0)
    bv = O.mixed_blocks(rv, pv, S.mixer_gaussians(rv, 3))
    bu = O.mixed_blocks(ru, pu, S.mixer_gaussians(ru, 3))
    sv, su = random_signs(K, rng0), random_signs(N, rng0)
    words, scale, zero, q = packed_weight(N, K, bits, rng0)
    Fv = dense_by_enumeration(rv, bv, sv)
    Fu = dense_by_enumeration(ru, bu, su)
    g = np.arange(K) // 64
    w_hat = (q - zero.astype(np.float64)[:, g]) * scale.astype(np.float64)[:, g]
    x = rng0.normal(size=(5, K))
    ref = x @ Fv.T @ w_hat.T @ Fu
    got = O.linear_mixed(x, words, scale, zero, bits, rv, bv, sv, ru, bu, su)
    assert np.allclose(got, ref, atol=1e-12, rtol=0)


def test_linear_mixed_contract_rounds_operands():
    """Contract mode equals the float64 product of bf16-rounded x~ and w_hat
    (both rounded by the pinned bf16 rounding), weights_exact keeps w_hat."""
    rv, ru = (8, 8), (5, 8)
    K, N, bits = 64, 40, 2
    bv = O.mixed_blocks(rv, random_params(rv, rng0), S.mixer_gaussians(rv))
    bu = O.mixed_blocks(ru, random_params(ru, rng0), S.mixer_gaussians(ru))
    sv, su = random_signs(K, rng0), random_signs(N, rng0)
    words, scale, zero, q = packed_weight(N, K, bits, rng0)
    x = rng0.normal(size=(2, K))
    xt = O.mixed_forward(x, rv, bv, sv)
    w_hat = O.dequant(O.unpack(words, bits, K), scale, zero)
    for exact in (False, True):
        w = w_hat if exact else O.bf16_round(w_hat)
        ref = O.mixed_transpose(O.bf16_round(xt) @ w.T, ru, bu, su)
        got = O.linear_mixed(x, words, scale, zero, bits, rv, bv, sv, ru, bu, su,
                             mfma_contract=True, weights_exact=exact)
        assert np.allclose(got, ref, atol=1e-12, rtol=0)
