"""Pins for the oracle's quantizer, packing, dequantization and bf16 rounding.

The pages leave the codebook open; the stand-in grid, its packing and its
dequantization are fixed by the stated reading and pinned here by hand-derived
layout fixtures (tests/golden/pack_layout.txt), exact-recovery constructions,
error bounds and library conversions (numpy fp16, torch bf16).
"""
import os

import numpy as np
import pytest
import torch

from oracle import harp_oracle as O

rng0 = np.random.default_rng(99)


def load_layout_fixtures(golden_dir):
    cases = []
    with open(os.path.join(golden_dir, "pack_layout.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            bits, K, spec = int(parts[0]), int(parts[1]), parts[2]
            words = [int(w, 16) for w in parts[3:]]
            if spec.startswith("mod:"):
                P = int(spec[4:])
                codes = [k % P for k in range(K)]
            else:
                pos, val = spec[4:].split("=")
                codes = [0] * K
                codes[int(pos)] = int(val)
            cases.append((bits, K, codes, words))
    return cases


def test_pack_layout_fixtures(golden_dir):
    cases = load_layout_fixtures(golden_dir)
    assert len(cases) >= 8
    for bits, K, codes, words in cases:
        q = np.array([codes], dtype=np.uint8)
        got = O.pack(q, bits)
        assert got.shape == (1, K * bits // 32)
        assert [int(w) for w in got[0]] == words, (bits, codes)
        assert np.array_equal(O.unpack(got, bits, K), q)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_unpack_roundtrip(bits):
    q = rng0.integers(0, 1 << bits, size=(5, 256)).astype(np.uint8)
    w = O.pack(q, bits)
    assert w.dtype == np.uint32 and w.shape == (5, 256 * bits // 32)
    assert np.array_equal(O.unpack(w, bits, 256), q)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_unpack_random_words_in_range(bits):
    w = rng0.integers(0, 2 ** 32, size=(3, 64 * bits // 32 * 4), dtype=np.uint64)
    w = w.astype(np.uint32)
    q = O.unpack(w, bits, 256)
    assert q.max() <= (1 << bits) - 1
    # every bit of every word is used exactly once: repacking reproduces it
    assert np.array_equal(O.pack(q, bits), w)


@pytest.mark.parametrize("arith", ["f64", "f32"])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantizer_bounds(bits, arith):
    qmax = (1 << bits) - 1
    W = rng0.normal(0, 0.02, size=(16, 512))
    W[:, 7] *= 20
    if arith == "f32":
        W = W.astype(np.float32).astype(np.float64)
    q, s16, z16 = O.quantize(W, bits, arith=arith)
    assert q.max() <= qmax
    s = s16.astype(np.float64)
    z = z16.astype(np.float64)
    assert np.all(z == np.rint(z)) and z.min() >= 0 and z.max() <= qmax
    w_hat = O.dequant(q, s16, z16)
    sr = np.repeat(s, 64, axis=1)
    zr = np.repeat(z, 64, axis=1)
    lo_grid = -zr * sr
    hi_grid = (qmax - zr) * sr
    inside = (W >= lo_grid) & (W <= hi_grid)
    err = np.abs(W - w_hat)
    rel = 1e-12 if arith == "f64" else 1e-6     # w / s rounded to float32
    assert np.all(err[inside] <= sr[inside] / 2 * (1 + rel))
    # outside the grid, the clamp costs at most one more half step
    # (z rounding) plus fp16 rounding of s over qmax steps
    assert np.all(err <= sr * (1.0 + qmax * 2.0 ** -11) + 1e-15)
    # zero is on the grid: codes equal to z dequantize to exactly 0
    assert np.all(w_hat[q == zr] == 0.0)


@pytest.mark.parametrize("arith", ["f64", "f32"])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantizer_exact_recovery(bits, arith):
    """A group that lies on a grid spanning its own min and max is recovered."""
    qmax = (1 << bits) - 1
    n, G = 6, 4
    s0 = (rng0.integers(600, 1400, size=(n, G)) * 2.0 ** -16)  # fp16-exact
    z0 = rng0.integers(0, qmax + 1, size=(n, G)).astype(np.float64)
    q0 = rng0.integers(0, qmax + 1, size=(n, G, 64))
    q0[..., 0] = 0
    q0[..., 1] = qmax
    W = (q0 - z0[..., None]) * s0[..., None]      # exact in float32 too
    q, s16, z16 = O.quantize(W.reshape(n, G * 64), bits, arith=arith)
    assert np.array_equal(s16.astype(np.float64), s0)
    assert np.array_equal(z16.astype(np.float64), z0)
    assert np.array_equal(q, q0.reshape(n, G * 64))


def load_tie_fixtures(golden_dir):
    """Exact-tie groups (tests/golden/quantize_ties.txt): (bits, scale,
    zero, values[64], codes[64]); unlisted positions hold 0.0 whose code is
    the zero-point."""
    cases = []
    with open(os.path.join(golden_dir, "quantize_ties.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            bits, scale, zero = int(parts[0]), float(parts[1]), int(parts[2])
            vals = np.zeros(64)
            codes = np.full(64, zero, dtype=np.uint8)
            for i, vc in enumerate(parts[3:]):
                v, c = vc.split(":")
                vals[i] = float(v)
                codes[i] = int(c)
            cases.append((bits, scale, zero, vals, codes))
    return cases


@pytest.mark.parametrize("arith", ["f64", "f32"])
def test_quantizer_tie_rule_golden(golden_dir, arith):
    """Round half to even for both the zero-point and the codes: hand-derived
    exact-tie groups, each of which rounding half up would change."""
    cases = load_tie_fixtures(golden_dir)
    assert len(cases) >= 7
    for bits, scale, zero, vals, codes in cases:
        q, s16, z16 = O.quantize(vals[None, :], bits, arith=arith)
        assert float(s16[0, 0]) == scale, (bits, vals[:4])
        assert float(z16[0, 0]) == zero, (bits, vals[:4])
        assert np.array_equal(q[0], codes), (bits, vals[:6], q[0][:6], codes[:6])
    # the same groups side by side in one row: each group decides alone
    for bits in (2, 3, 4):
        sub = [c for c in cases if c[0] == bits]
        row = np.concatenate([c[3] for c in sub])[None, :]
        q, s16, z16 = O.quantize(row, bits, arith=arith)
        assert np.array_equal(q[0], np.concatenate([c[4] for c in sub]))
        assert [float(z) for z in z16[0]] == [c[2] for c in sub]


@pytest.mark.parametrize("arith", ["f64", "f32"])
def test_quantizer_degenerate_group(arith):
    W = np.zeros((2, 128))
    W[1, 64:] = 0.5
    q, s16, z16 = O.quantize(W, 2, arith=arith)
    assert float(s16[0, 0]) == float(np.float16(2.0 / 3.0))
    assert np.all(O.dequant(q, s16, z16)[0] == 0.0)
    # all-positive group: lo forced to 0 -> z = 0, top code hits max exactly
    assert float(z16[1, 1]) == 0.0 and np.all(q[1, 64:] == 3)


@pytest.mark.parametrize("arith", ["f64", "f32"])
def test_quantizer_scale_floor(arith):
    W = np.full((1, 64), 1e-9)
    _, s16, _ = O.quantize(W, 2, arith=arith)
    assert float(s16[0, 0]) == 2.0 ** -14


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantizer_f32_decisions_differ_only_at_boundaries(bits):
    """The float32 mode takes the float64 decisions except where a value
    lies within float32 rounding of a decision boundary: rarely, and then
    by one code."""
    W = (rng0.normal(0, 0.02, size=(256, 1024))).astype(np.float32).astype(np.float64)
    q64, s64, z64 = O.quantize(W, bits)
    q32, s32, z32 = O.quantize(W, bits, arith="f32")
    same_s = s64 == s32
    assert same_s.mean() > 0.99
    rows = np.repeat(same_s & (z64 == z32), 64, axis=1)
    d = np.abs(q64.astype(int) - q32.astype(int))[rows]
    assert d.max() <= 1 and (d > 0).mean() < 1e-3


@pytest.mark.parametrize("arith", ["f64", "f32"])
def test_quantizer_zero_point_is_positive_zero(arith):
    W = np.full((2, 64), 0.3)
    W[0, 0] = -0.0               # minimum -0.0: lo = -0.0, z = +0
    W[1, :] = -0.0               # all -0.0: the flat-group case
    _, _, z16 = O.quantize(W, 2, arith=arith)
    assert not np.any(z16.view(np.uint16) & 0x8000)


def test_quantizer_rejects_unknown_arith():
    with pytest.raises(ValueError):
        O.quantize(np.zeros((1, 64)), 2, arith="f16")


def test_dequant_exact_in_float32():
    """(q - z) s is exact in float32 for every code, zero and fp16 scale."""
    s_bits = rng0.integers(0x0400, 0x7BFF, size=(64, 8)).astype(np.uint16)
    s16 = s_bits.view(np.float16)
    for bits in (2, 3, 4):
        qmax = (1 << bits) - 1
        q = rng0.integers(0, qmax + 1, size=(64, 512)).astype(np.uint8)
        z16 = rng0.integers(0, qmax + 1, size=(64, 8)).astype(np.float16)
        ref = O.dequant(q, s16, z16)
        q32 = q.astype(np.float32)
        s32 = np.repeat(s16.astype(np.float32), 64, axis=1)
        z32 = np.repeat(z16.astype(np.float32), 64, axis=1)
        f32 = (q32 - z32) * s32
        assert np.array_equal(f32.astype(np.float64), ref)


def test_bf16_round_matches_torch():
    x = rng0.normal(0, 3, size=4096).astype(np.float32)
    # add exact ties: low 16 bits = 0x8000, with even and odd upper halves
    u = x.view(np.uint32).copy()
    u[:64] = (u[:64] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    u[64:128] = (u[64:128] & np.uint32(0xFFFE0000)) | np.uint32(0x18000)
    x = u.view(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_f16_and_bf16_decoders():
    v = rng0.normal(size=100).astype(np.float16)
    assert np.array_equal(O.f16_bits_to_f64(v.view(np.uint16)), v.astype(np.float64))
    t = torch.from_numpy(rng0.normal(size=100).astype(np.float32)).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_bits_to_f64(bits), t.to(torch.float64).numpy())
