"""The seeded input generators: determinism, boundary shapes and ranges."""
import numpy as np
import pytest

from synth import workloads as S


def test_deterministic_and_shapes():
    cfg = S.CONFIGS["l7b_mlp"]
    a = S.layer_inputs(cfg, 1, 2, 16)
    b = S.layer_inputs(cfg, 1, 2, 16)
    for f in ("words", "scale", "zero"):
        assert np.array_equal(getattr(a.W, f), getattr(b.W, f))
    assert np.array_equal(a.x, b.x) and np.array_equal(a.V.cs, b.V.cs)
    assert a.W.words.shape == (4096, 11008 * 2 // 32)
    assert a.W.scale.shape == (4096, 11008 // 64) and a.W.scale.dtype == np.uint16
    assert a.V.cs.shape == (43, 8, 128, 2) and a.V.cs.dtype == np.float32
    assert a.U.cs.shape == (1, 12, 2048, 2)
    assert a.x.shape == (16, 11008) and a.x.dtype == np.uint16


def test_outliers_and_signs():
    out = S.outlier_channels(4096, np.random.default_rng(0))
    assert len(out) == 41 and len(set(out.tolist())) == 41
    r = S.rotation(11008, 256, np.random.default_rng(1))
    assert r.sign_bits.shape == (344,)
    r = S.rotation(48, 16, np.random.default_rng(2))
    assert r.sign_bits[-1] >> 16 == 0          # bits beyond dim are clear
    c, s = r.cs[..., 0].astype(np.float64), r.cs[..., 1].astype(np.float64)
    assert np.allclose(c * c + s * s, 1.0, atol=1e-6)


def test_qweight_zero_and_scale_ranges():
    for bits in (2, 3, 4):
        w = S.qweight(32, 256, bits, np.random.default_rng(bits))
        z = w.zero.view(np.float16).astype(np.float64)
        qmax = (1 << bits) - 1
        assert set(np.unique(z)) <= {qmax // 2, qmax // 2 + 1}
        s = w.scale.view(np.float16).astype(np.float64)
        assert s.min() > 0 and s.max() < 0.2


def test_qweight_wide_spread_covers_the_format_edges():
    for bits in (2, 3, 4):
        qmax = (1 << bits) - 1
        w = S.qweight(64, 1024, bits, np.random.default_rng(bits), spread="wide")
        z = w.zero.view(np.float16).astype(np.float64)
        s = w.scale.view(np.float16).astype(np.float64)
        assert z.min() == 0 and z.max() == qmax and np.all(z == np.round(z))
        assert np.all(z[:, 0] == 0) and np.all(z[:, -1] == qmax)
        assert s.min() == 2.0 ** -24                       # smallest fp16 subnormal
        assert np.any(s == 1023 * 2.0 ** -24)              # largest subnormal
        assert (s < 2.0 ** -14).mean() > 0.2 and s.max() > 4.0
        assert np.all(s > 0) and np.all(np.isfinite(s))
    with pytest.raises(ValueError):
        S.qweight(4, 64, 2, np.random.default_rng(0), spread="bogus")


def test_bf16_activations_carry_outliers():
    out = np.array([3, 17])
    x = S.activations(64, 32, np.random.default_rng(3), "bf16", out)
    v = (x.astype(np.uint32) << 16).view(np.float32)
    big = np.abs(v[:, out]).mean()
    small = np.abs(np.delete(v, out, axis=1)).mean()
    assert big > 10 * small


def test_int8_angle_codes():
    cfg = S.CONFIGS["l7b_mlp"]
    a = S.layer_inputs(cfg, 0, 2, 1, angles="int8")
    b = S.layer_inputs(cfg, 0, 2, 1, angles="int8")
    assert a.V.cs is None and a.V.phi_codes.dtype == np.int8
    assert a.V.phi_codes.shape == (1, 12, 2048) and a.U.phi_codes.shape == (43, 8, 128)
    assert np.array_equal(a.V.phi_codes, b.V.phi_codes)
    assert np.array_equal(a.U.sign_bits, b.U.sign_bits)
    c = a.V.phi_codes.astype(np.float64)
    assert c.min() >= -127 and c.max() <= 127
    # spread: std of code * step near sqrt(0.05)
    std = (c * a.V.phi_step).std()
    assert abs(std - np.sqrt(S.THETA_VAR)) < 0.02
    assert np.float32(a.V.phi_step) == a.V.phi_step


def test_mixed_rotation_parameters():
    a = S.mixed_rotation((8, 8, 8, 5, 2), np.random.default_rng(5))
    b = S.mixed_rotation((8, 8, 8, 5, 2), np.random.default_rng(5))
    assert a.dim == 5120 and len(a.params) == 5
    assert a.params[0].shape == (640, 28) and a.params[3].shape == (1024, 10)
    assert a.params[4].shape == (2560, 1)
    assert all(np.array_equal(p, q) for p, q in zip(a.params, b.params))
    assert a.sign_bits.shape == (160,)
