"""Pins for the oracle's two-sided linear (HARP technical summary §2.4, §5).

* exact change of basis: with the rotated weight unquantized, the composed
  map equals W x (page: the full-precision model is preserved);
* at the Hadamard initialisation the linear has a closed form with scipy's
  Hadamard matrix;
* dense composition with explicit rotation matrices on the tiny layer;
* the offline pipeline (rotate, quantize, pack) reproduces W x up to the
  quantization error, and rotation lowers the output error when inputs and
  weights carry outlier channels (qualitative incoherence claim, technical
  summary §1; not a parity gate).
"""
import math

import numpy as np
import scipy.linalg

from oracle import harp_oracle as O
from synth import workloads as S

rng0 = np.random.default_rng(7)


def side(d, b, var=0.05, seed=0, theta=None):
    return S.rotation(d, b, np.random.default_rng(seed), theta_var=var, theta=theta)


def f64cs(rot):
    # float64 (cos, sin) of the float64 angles, for exact-orthogonality pins
    return np.stack([np.cos(rot.theta), np.sin(rot.theta)], axis=-1)


def test_exact_change_of_basis():
    N, K = 48, 64
    V = side(K, 16, seed=1)
    U = side(N, 16, seed=2)
    W = rng0.normal(size=(N, K))
    x = rng0.normal(size=(3, K))
    Wp = O.rotate_weight(W, f64cs(U), U.sign_bits, 16, f64cs(V), V.sign_bits, 16)
    FU = O.rotation_matrix(f64cs(U), U.sign_bits, N, 16)
    FV = O.rotation_matrix(f64cs(V), V.sign_bits, K, 16)
    assert np.max(np.abs(Wp - FU @ W @ FV.T)) < 1e-12
    xt = O.forward(x, f64cs(V), V.sign_bits, 16)
    y = O.transpose(xt @ Wp.T, f64cs(U), U.sign_bits, 16)
    assert np.max(np.abs(y - x @ W.T)) < 1e-12


def test_linear_at_init_closed_form():
    """t = pi/4 everywhere: y = D_U H W_hat H D_V x / b (scipy Hadamard)."""
    b = 256
    t = np.full((1, 8, 128), math.pi / 4)
    V = side(b, b, theta=t, seed=3)
    U = side(b, b, theta=t, seed=4)
    Wq = S.qweight(b, b, 2, np.random.default_rng(5))
    x = rng0.normal(size=(4, b))
    y = O.linear(x, Wq.words, Wq.scale.view(np.float16), Wq.zero.view(np.float16),
                 2, f64cs(V), V.sign_bits, b, f64cs(U), U.sign_bits, b)
    H = scipy.linalg.hadamard(b).astype(np.float64)
    dv = O.decode_signs(V.sign_bits, b)
    du = O.decode_signs(U.sign_bits, b)
    w_hat = O.dequant(O.unpack(Wq.words, 2, b), Wq.scale.view(np.float16),
                      Wq.zero.view(np.float16))
    ref = ((x * dv) @ H.T @ w_hat.T @ H) * du / b
    assert np.max(np.abs(y - ref)) < 1e-12 * np.max(np.abs(ref))


def test_linear_dense_composition_tiny():
    """Tiny layer with float32 boundary coefficients: fast == dense matrices."""
    li = S.layer_inputs(S.CONFIGS["tiny"], 0, 2, 4)
    x = li.x.astype(np.float64)
    y = O.linear(x, li.W.words, li.W.scale.view(np.float16), li.W.zero.view(np.float16),
                 2, li.V.cs, li.V.sign_bits, 256, li.U.cs, li.U.sign_bits, 256)
    FV = O.rotation_matrix(li.V.cs, li.V.sign_bits, 256, 256)
    FU = O.rotation_matrix(li.U.cs, li.U.sign_bits, 256, 256)
    w_hat = O.dequant(O.unpack(li.W.words, 2, 256), li.W.scale.view(np.float16),
                      li.W.zero.view(np.float16))
    ref = (FU.T @ w_hat @ FV @ x.T).T
    assert np.max(np.abs(y - ref)) < 1e-12 * np.max(np.abs(ref))


def test_mfma_contract_rounds_both_operands():
    """Contract mode equals the f64 linear of bf16-rounded x~ and w_hat."""
    li = S.layer_inputs(S.CONFIGS["tiny"], 0, 2, 4)
    x = li.x.astype(np.float64)
    args = (li.W.words, li.W.scale.view(np.float16), li.W.zero.view(np.float16), 2,
            li.V.cs, li.V.sign_bits, 256, li.U.cs, li.U.sign_bits, 256)
    y0 = O.linear(x, *args)
    y1 = O.linear(x, *args, mfma_contract=True)
    # bf16 keeps 8 significant bits: relative error ~ 2^-9 / sqrt(3) per term
    r = O.rel_l2(y1, y0)
    assert 1e-4 < r < 5e-3


def test_mfma_contract_with_exact_weights_rounds_only_x():
    """weights_exact: the dense composition with only x~ rounded to bf16."""
    li = S.layer_inputs(S.CONFIGS["tiny"], 0, 2, 4)
    x = li.x.astype(np.float64)
    s16, z16 = li.W.scale.view(np.float16), li.W.zero.view(np.float16)
    args = (li.W.words, s16, z16, 2, li.V.cs, li.V.sign_bits, 256, li.U.cs,
            li.U.sign_bits, 256)
    y = O.linear(x, *args, mfma_contract=True, weights_exact=True)
    FV = O.rotation_matrix(li.V.cs, li.V.sign_bits, 256, 256)
    FU = O.rotation_matrix(li.U.cs, li.U.sign_bits, 256, 256)
    w_hat = O.dequant(O.unpack(li.W.words, 2, 256), s16, z16)
    xt = O.bf16_round((FV @ x.T).T)
    ref = (FU.T @ (w_hat @ xt.T)).T
    assert np.max(np.abs(y - ref)) < 1e-12 * np.max(np.abs(ref))
    # one rounding point instead of two: closer to the float64 linear
    y0 = O.linear(x, *args)
    y2 = O.linear(x, *args, mfma_contract=True)
    assert 0 < O.rel_l2(y, y0) < O.rel_l2(y2, y0)


def test_offline_pipeline_and_incoherence():
    """Rotate -> quantize -> pack, then the online linear approximates W x;
    with outlier channels, rotation lowers the 2-bit output error."""
    N, K, b = 256, 512, 256
    out = S.outlier_channels(K, np.random.default_rng(11))
    W = S.dense_weight(N, K, np.random.default_rng(12), 0.02, out)
    V = side(K, b, seed=13)
    U = side(N, b, seed=14)
    Wp = O.rotate_weight(W, U.cs, U.sign_bits, b, V.cs, V.sign_bits, b)
    q, s16, z16 = O.quantize(Wp, 2)
    words = O.pack(q, 2)
    x = S.activations(8, K, np.random.default_rng(15), "f32", out).astype(np.float64)
    y = O.linear(x, words, s16, z16, 2, V.cs, V.sign_bits, b, U.cs, U.sign_bits, b)
    y_ref = x @ W.T
    err_rot = O.rel_l2(y, y_ref)
    # plain (unrotated) quantization of the same W
    q0, s0, z0 = O.quantize(W, 2)
    err_plain = O.rel_l2(x @ O.dequant(q0, s0, z0).T, y_ref)
    # 2-bit output error: ~0.06 rotated vs ~0.11-0.16 plain on this recipe
    assert err_rot < 0.1
    assert err_rot < 0.75 * err_plain
