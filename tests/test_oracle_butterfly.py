"""Pins for the oracle's butterfly (HARP technical summary §2.1-2.2).

Each check ties the oracle to something other than itself: scipy's Sylvester
Hadamard, the page's own block definition Q(phi) G_2, closed forms at special
angles, a dense product built by enumeration, and orthogonality.
"""
import math

import numpy as np
import pytest
import scipy.linalg

from oracle import harp_oracle as O

rng0 = np.random.default_rng(1234)


def cs_from_theta(theta):
    theta = np.asarray(theta, dtype=np.float64)
    return np.stack([np.cos(theta), np.sin(theta)], axis=-1)


def const_cs(d, b, t):
    L = b.bit_length() - 1
    return cs_from_theta(np.full((d // b, L, b // 2), t))


def random_signs(d, rng):
    bits = rng.integers(0, 2 ** 32, size=(d + 31) // 32, dtype=np.uint64)
    bits = bits.astype(np.uint32)
    if d % 32:
        bits[-1] &= np.uint32((1 << (d % 32)) - 1)
    return bits


def signs_pm1(bits, d):
    # independent decode: string of bits per word, least significant first
    out = []
    for i in range(d):
        w = int(bits[i // 32])
        out.append(-1.0 if (w >> (i % 32)) & 1 else 1.0)
    return np.array(out)


@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 64, 256, 512])
def test_sylvester_matches_scipy(b):
    assert np.array_equal(O.sylvester_hadamard(b), scipy.linalg.hadamard(b))


def test_sign_decode_against_bitstring():
    bits = random_signs(100, rng0)
    assert np.array_equal(O.decode_signs(bits, 100), signs_pm1(bits, 100))


@pytest.mark.parametrize("phi", [0.0, 0.3, -1.1, 2.5])
def test_paper_block_is_reflection_form(phi):
    """Q(phi) G_2 (page, §2.2) equals [[cos t, sin t], [sin t, -cos t]], t = pi/4 + phi."""
    t = math.pi / 4 + phi
    assert np.allclose(O.paper_block(phi), O.block(math.cos(t), math.sin(t)),
                       atol=1e-15, rtol=0)


@pytest.mark.parametrize("b", [2, 4, 8, 16, 32, 64, 128, 256])
def test_init_is_randomized_hadamard(b):
    """Zero-initialised angles give F = H_b D / sqrt(b) exactly (§2.2)."""
    d = b
    bits = random_signs(d, rng0)
    F = O.rotation_matrix(const_cs(d, b, math.pi / 4), bits, d, b)
    ref = scipy.linalg.hadamard(b) @ np.diag(signs_pm1(bits, d)) / math.sqrt(b)
    assert np.max(np.abs(F - ref)) < 1e-12


def test_init_block_diagonal_is_rht_per_block():
    b, nblk = 16, 3
    d = b * nblk
    bits = random_signs(d, rng0)
    F = O.rotation_matrix(const_cs(d, b, math.pi / 4), bits, d, b)
    ref = scipy.linalg.block_diag(*[scipy.linalg.hadamard(b)] * nblk)
    ref = ref @ np.diag(signs_pm1(bits, d)) / math.sqrt(b)
    assert np.max(np.abs(F - ref)) < 1e-12


@pytest.mark.parametrize("b", [2, 4, 8, 16, 64])
def test_theta_zero_is_popcount_sign(b):
    """t = 0: every block is diag(1, -1), so B = diag((-1)^popcount(i))."""
    F = O.rotation_matrix(const_cs(b, b, 0.0), np.zeros((b + 31) // 32, np.uint32), b, b)
    ref = np.diag([(-1.0) ** bin(i).count("1") for i in range(b)])
    assert np.max(np.abs(F - ref)) < 1e-15


@pytest.mark.parametrize("b", [2, 4, 8, 16, 64])
def test_theta_half_pi_reverses(b):
    """t = pi/2: every block swaps its pair, so B maps e_i to e_{b-1-i}."""
    F = O.rotation_matrix(const_cs(b, b, math.pi / 2), np.zeros((b + 31) // 32, np.uint32), b, b)
    ref = np.eye(b)[::-1]
    assert np.max(np.abs(F - ref)) < 1e-15


def dense_stage_by_enumeration(b, s, cos_s, sin_s):
    """Stage s as a dense matrix; block c is the c-th pair in increasing i."""
    S = np.zeros((b, b))
    heads = [i for i in range(b) if not (i >> s) & 1]
    for c, i in enumerate(heads):
        j = i + (1 << s)
        S[i, i], S[i, j] = cos_s[c], sin_s[c]
        S[j, i], S[j, j] = sin_s[c], -cos_s[c]
    return S


@pytest.mark.parametrize("b", [2, 4, 8, 16])
def test_brute_force_perturbed(b):
    """Perturbed angles: fast butterfly == dense product S_{L-1}..S_0 D."""
    L = b.bit_length() - 1
    theta = math.pi / 4 + rng0.normal(0, 0.5, size=(1, L, b // 2))
    cs = cs_from_theta(theta)
    bits = random_signs(b, rng0)
    P = np.diag(signs_pm1(bits, b))
    for s in range(L):
        P = dense_stage_by_enumeration(b, s, cs[0, s, :, 0], cs[0, s, :, 1]) @ P
    F = O.rotation_matrix(cs, bits, b, b)
    assert np.max(np.abs(F - P)) < 1e-12


@pytest.mark.parametrize("b,d", [(8, 8), (16, 48), (256, 256), (256, 768)])
def test_orthogonality_and_inverse(b, d):
    L = b.bit_length() - 1
    theta = math.pi / 4 + rng0.normal(0, math.sqrt(0.05), size=(d // b, L, b // 2))
    cs = cs_from_theta(theta)
    bits = random_signs(d, rng0)
    F = O.rotation_matrix(cs, bits, d, b)
    assert np.max(np.abs(F @ F.T - np.eye(d))) < 1e-12
    x = rng0.normal(size=(3, d))
    fx = O.forward(x, cs, bits, b)
    assert np.allclose(np.linalg.norm(fx, axis=1), np.linalg.norm(x, axis=1),
                       rtol=1e-13, atol=0)
    assert np.max(np.abs(O.transpose(fx, cs, bits, b) - x)) < 1e-12
    # the transpose routine applies the matrix transpose
    T = O.transpose(np.eye(d), cs, bits, b).T
    assert np.max(np.abs(T - F.T)) < 1e-12


def test_each_stage_orthogonal():
    b = 32
    L = 5
    theta = rng0.uniform(-3, 3, size=(1, L, b // 2))
    cs = cs_from_theta(theta)
    for s in range(L):
        S = O.apply_stage(np.eye(b), cs[0, s, :, 0], cs[0, s, :, 1], s).T
        assert np.max(np.abs(S @ S.T - np.eye(b))) < 1e-15


def test_block_diagonal_independent_blocks():
    """Off-diagonal blocks are zero; block j is the b-sized butterfly of slice j."""
    b, nblk = 8, 4
    d = b * nblk
    L = 3
    theta = rng0.uniform(-3, 3, size=(nblk, L, b // 2))
    cs = cs_from_theta(theta)
    bits = random_signs(d, rng0)
    F = O.rotation_matrix(cs, bits, d, b)
    pm = signs_pm1(bits, d)
    for j in range(nblk):
        for k in range(nblk):
            blk = F[j * b:(j + 1) * b, k * b:(k + 1) * b]
            if j != k:
                assert np.all(blk == 0)
            else:
                P = np.diag(pm[j * b:(j + 1) * b])
                for s in range(L):
                    P = dense_stage_by_enumeration(b, s, cs[j, s, :, 0], cs[j, s, :, 1]) @ P
                assert np.max(np.abs(blk - P)) < 1e-12


def test_large_init_matches_hadamard_on_vectors():
    """b = 4096 at init: F x == H (D x) / 64 with scipy's Hadamard."""
    b = 4096
    bits = random_signs(b, rng0)
    x = rng0.normal(size=(2, b))
    got = O.forward(x, const_cs(b, b, math.pi / 4), bits, b)
    H = scipy.linalg.hadamard(b).astype(np.float64)
    ref = (x * signs_pm1(bits, b)) @ H.T / 64.0
    assert np.max(np.abs(got - ref)) < 1e-12


# ---------------------------------------------------------------------------
# int8-stored angles: t = pi/4 + code * step (technical summary §2.4 storage
# note).  Pinned by the page's block definition and by closed forms at the
# codes that give quarter turns (a swap) and zero turns (a diagonal).
# ---------------------------------------------------------------------------

QUARTER = np.float32(math.pi / 508)      # 127 * step = pi/4 up to float32


def _code_block(d, b, code):
    L = b.bit_length() - 1
    return np.full((d // b, L, b // 2), code, dtype=np.int8)


def test_angle_codes_match_page_block():
    """block(decoded pair) equals Q(code * step) G_2 as the page defines it."""
    r = np.random.default_rng(40)
    codes = r.integers(-128, 128, size=50).astype(np.int8)
    step = np.float32(0.0123)
    cs = O.decode_angle_codes(codes, step)
    for c, pair in zip(codes, cs):
        phi = int(c) * float(step)
        assert np.allclose(O.block(pair[0], pair[1]), O.paper_block(phi),
                           atol=1e-15, rtol=0)


@pytest.mark.parametrize("b", [2, 16, 256])
def test_angle_code_zero_is_randomized_hadamard(b):
    """Code 0 is the Hadamard initialisation whatever the step."""
    r = np.random.default_rng(41 + b)
    signs = random_signs(2 * b, r)
    x = r.normal(size=(3, 2 * b))
    cs = O.decode_angle_codes(_code_block(2 * b, b, 0), np.float32(0.37))
    Hb = scipy.linalg.hadamard(b) / math.sqrt(b)
    xd = x * signs_pm1(signs, 2 * b)
    ref = np.concatenate([xd[:, :b] @ Hb.T, xd[:, b:] @ Hb.T], axis=1)
    assert np.allclose(O.forward(x, cs, signs, b), ref, atol=1e-13, rtol=0)


@pytest.mark.parametrize("b", [4, 32, 512])
def test_angle_code_quarter_turn_reverses(b):
    """Code +127 at step pi/508: every stage swaps its pairs, so F x [i] is
    (D x)[b - 1 - i] (index complement over all L bits)."""
    r = np.random.default_rng(50 + b)
    signs = random_signs(b, r)
    x = r.normal(size=(2, b))
    cs = O.decode_angle_codes(_code_block(b, b, 127), QUARTER)
    ref = (x * signs_pm1(signs, b))[:, ::-1]
    assert np.allclose(O.forward(x, cs, signs, b), ref, atol=1e-6, rtol=0)


@pytest.mark.parametrize("b", [4, 32, 512])
def test_angle_code_negative_quarter_is_parity_sign(b):
    """Code -127 at step pi/508: t = 0, every stage negates the partner
    coordinate, so F x [i] = (-1)^popcount(i) (D x)[i]."""
    r = np.random.default_rng(60 + b)
    signs = random_signs(b, r)
    x = r.normal(size=(2, b))
    cs = O.decode_angle_codes(_code_block(b, b, -127), QUARTER)
    par = np.array([(-1.0) ** bin(i).count("1") for i in range(b)])
    ref = x * signs_pm1(signs, b) * par
    assert np.allclose(O.forward(x, cs, signs, b), ref, atol=1e-6, rtol=0)


def test_angle_codes_stage_and_pair_layout():
    """Codes vary by stage (b = 8) and by pair (b = 4): closed forms.

    b = 8, stages 0 and 2 swap (+127) and stage 1 is diagonal (-127):
    F x [j] = (-1)^bit1(j) (D x)[j xor 5].
    b = 4, stage 0 pair 0 swaps, pair 1 is diagonal; stage 1 diagonal:
    F x = (x1, x0, -x2, x3) after D.
    """
    r = np.random.default_rng(70)
    signs = random_signs(8, r)
    x = r.normal(size=(2, 8))
    codes = np.array([[[127] * 4, [-127] * 4, [127] * 4]], dtype=np.int8)
    got = O.forward(x, O.decode_angle_codes(codes, QUARTER), signs, 8)
    xd = x * signs_pm1(signs, 8)
    ref = np.stack([(-1.0) ** ((j >> 1) & 1) * xd[:, j ^ 5] for j in range(8)], axis=1)
    assert np.allclose(got, ref, atol=1e-6, rtol=0)

    signs4 = random_signs(4, r)
    x4 = r.normal(size=(2, 4))
    codes4 = np.array([[[127, -127], [-127, -127]]], dtype=np.int8)
    got4 = O.forward(x4, O.decode_angle_codes(codes4, QUARTER), signs4, 4)
    u = x4 * signs_pm1(signs4, 4)
    ref4 = np.stack([u[:, 1], u[:, 0], -u[:, 2], u[:, 3]], axis=1)
    assert np.allclose(got4, ref4, atol=1e-6, rtol=0)


def test_angle_codes_reject_other_dtypes():
    with pytest.raises(ValueError):
        O.decode_angle_codes(np.zeros(4, dtype=np.int16), 0.1)
