"""harp_mixed_expand (host C++ in libharp) against the oracle's expansion of
the same learnable parameters and the same fixed Gaussians (HARP technical
summary §2.1-2.2: B = Q(theta) G_b, Givens for b = 2, Cayley map for b > 2,
Sylvester Hadamard or the QR factor of a fixed Gaussian as G_b).  Host
logic only: no GPU involved."""
import math

import numpy as np
import pytest
import scipy.linalg

import rotated_bit_amd as H
from oracle import harp_oracle as O
from synth import workloads as S

SCHEDULES = [(8, 8, 8, 5, 2), (3,), (5, 3), (7, 2, 5, 3), (43, 4, 64), (64, 64, 7),
             (2,) * 6, (16, 16, 20), (8, 8, 4, 43)]


def split_stages(flat, radices):
    d = int(np.prod(radices))
    out, off = [], 0
    for b in radices:
        n = d * b
        out.append(flat[off:off + n].reshape(d // b, b, b))
        off += n
    assert off == flat.size
    return out


@pytest.mark.parametrize("radices", SCHEDULES)
def test_expand_matches_oracle(radices):
    side = S.mixed_rotation(radices, np.random.default_rng(sum(radices)), scale=0.3,
                            mixer_seed=7)
    got = split_stages(H.harp_mixed_expand(radices, side.params, side.gaussians), radices)
    ref = O.mixed_blocks(radices, side.params, side.gaussians)
    for g, r in zip(got, ref):
        # float32 rounding of entries of magnitude <= 1 (half an ulp <= 6e-8)
        assert np.max(np.abs(g.astype(np.float64) - r)) <= 1.2e-7
        eye = np.eye(g.shape[-1])
        gg = g.astype(np.float64)
        assert np.max(np.abs(gg @ np.swapaxes(gg, -1, -2) - eye)) <= 2e-6


@pytest.mark.parametrize("radices", [(4, 8), (2, 2, 16), (64,)])
def test_zero_parameters_give_the_sylvester_mixer(radices):
    params = [np.zeros((int(np.prod(radices)) // b, b * (b - 1) // 2)) for b in radices]
    got = split_stages(H.harp_mixed_expand(radices, params), radices)
    for b, g in zip(radices, got):
        Hb = scipy.linalg.hadamard(b) / math.sqrt(b)
        assert np.allclose(g, Hb[None].astype(np.float32), atol=0, rtol=0)


def test_expand_error_paths():
    L = H._lib
    radices = (5, 2)
    side = S.mixed_rotation(radices, np.random.default_rng(0))
    out = np.full(10 * 7, 7.0, dtype=np.float32)
    rad = np.array(radices, dtype=np.int32)
    p = np.concatenate([a.ravel() for a in side.params]).astype(np.float64)
    g = side.gaussians[0].astype(np.float64).ravel().copy()
    f = L.lib.harp_mixed_expand
    assert f(2, rad.ctypes.data, p.ctypes.data, g.ctypes.data, out.ctypes.data) == L.HARP_OK
    good = out.copy()
    out[:] = 7.0
    assert f(2, None, p.ctypes.data, g.ctypes.data, out.ctypes.data) == L.HARP_ERR_NULL
    assert f(2, rad.ctypes.data, None, g.ctypes.data, out.ctypes.data) == L.HARP_ERR_NULL
    assert f(2, rad.ctypes.data, p.ctypes.data, None, out.ctypes.data) == L.HARP_ERR_NULL
    assert f(2, rad.ctypes.data, p.ctypes.data, g.ctypes.data, None) == L.HARP_ERR_NULL
    assert f(0, rad.ctypes.data, p.ctypes.data, g.ctypes.data, out.ctypes.data) == L.HARP_ERR_SHAPE
    bad = np.array([1, 10], dtype=np.int32)
    assert f(2, bad.ctypes.data, p.ctypes.data, g.ctypes.data, out.ctypes.data) == L.HARP_ERR_SHAPE
    bad = np.array([65, 2], dtype=np.int32)
    assert f(2, bad.ctypes.data, p.ctypes.data, g.ctypes.data,
             out.ctypes.data) == L.HARP_ERR_UNSUPPORTED
    big = np.array([64, 64, 64], dtype=np.int32)          # 262144 > the mixed maximum
    assert f(3, big.ctypes.data, p.ctypes.data, g.ctypes.data,
             out.ctypes.data) == L.HARP_ERR_UNSUPPORTED
    pn = p.copy()
    pn[3] = np.nan
    assert f(2, rad.ctypes.data, pn.ctypes.data, g.ctypes.data, out.ctypes.data) == L.HARP_ERR_SHAPE
    g0 = np.zeros_like(g)                                  # rank-deficient Gaussian
    assert f(2, rad.ctypes.data, p.ctypes.data, g0.ctypes.data, out.ctypes.data) == L.HARP_ERR_SHAPE
    out[:] = 7.0
    assert f(2, rad.ctypes.data, pn.ctypes.data, g.ctypes.data, out.ctypes.data) == L.HARP_ERR_SHAPE
    assert np.all(out == 7.0)                              # untouched on error
    assert f(2, rad.ctypes.data, p.ctypes.data, g.ctypes.data, out.ctypes.data) == L.HARP_OK
    assert np.array_equal(out, good)
