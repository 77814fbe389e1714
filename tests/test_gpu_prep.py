"""GPU parity of the offline preparation: W' = F_U W F_V^T (float32 butterfly
bar against the float64 oracle) and quantize + pack (bit-exact against the
oracle quantizer taking its decisions in float32, the kernel's precision).
Inputs are seeded (synth/); special groups exercise ties, flat and signed-
zero groups.
"""
import numpy as np
import pytest
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
    return np.random.default_rng(np.random.SeedSequence([4242, *k]))


ROTW_CASES = [
    (256, 256, 256, 256, "f32"), (512, 2048, 32, 2048, "f32"), (1024, 4096, 1024, 4096, "int8"),
    (768, 256, 256, 16, "int8"), (64, 8192, 64, 8192, "f32"), (11008, 256, 256, 256, "f32"),
]


@pytest.mark.parametrize("N,K,bu,bv,angles", ROTW_CASES)
def test_rotate_weight(N, K, bu, bv, angles):
    d = D()
    draw = S.rotation if angles == "f32" else S.rotation_q8
    V = draw(K, bv, rng(1, K, bv))
    U = draw(N, bu, rng(2, N, bu))
    out = S.outlier_channels(K, rng(3, K))
    W = S.dense_weight(N, K, rng(4, N, K), 0.02, out).astype(np.float32)
    Wd = d.dev(W)
    Wp = torch.empty_like(Wd)
    ws = torch.empty(H().harp_rotate_weight_workspace_bytes(N, K), dtype=torch.uint8,
                     device="cuda")
    H().harp_rotate_weight(d.dev_rotation(V), d.dev_rotation(U), Wd, Wp, ws)
    ref = O.rotate_weight(W.astype(np.float64), d.cs64(U), U.sign_bits, bu,
                          d.cs64(V), V.sign_bits, bv)
    r = O.rel_l2(Wp.cpu().numpy().astype(np.float64), ref)
    print(f"[rotate_weight {N}x{K} bu={bu} bv={bv} {angles}] rel_l2={r:.3e}", flush=True)
    assert r <= BUTTERFLY_TOL


def salted_weight(N, K, seed):
    """Seeded float32 weight with special groups in the first rows."""
    W = S.dense_weight(N, K, rng(5, N, K, seed), 0.02).astype(np.float32)
    if N >= 6 and K >= 128:
        W[0, :64] = 0.0                               # flat group (lo = -1, hi = 1)
        W[1, :64] = np.float32(0.25)                  # constant positive group
        W[2, :64] = np.abs(W[2, :64])
        W[2, 0] = np.float32(-0.0)                    # minimum -0.0
        step = np.float32(2.0 ** -6)                  # exact ties: w / s = n + 1/2
        W[3, :64] = step * (np.arange(64) % 4 - np.float32(1.5))
        W[4, 64:128] = -np.abs(W[4, 64:128])          # all-negative group
        W[5, 64] = np.float32(3.0)                    # one large outlier
    return W


QP_CASES = [(64, 256, 2), (64, 256, 3), (64, 256, 4), (4096, 4096, 2), (1000, 11008, 3),
            (17, 64, 4), (512, 28672, 2)]


@pytest.mark.parametrize("N,K,bits", QP_CASES)
def test_quantize_pack_bit_exact(N, K, bits):
    d = D()
    W = salted_weight(N, K, bits)
    q_ref, s_ref, z_ref = O.quantize(W, bits, arith="f32")
    words_ref = O.pack(q_ref, bits)
    qw = torch.empty((N, K * bits // 32), dtype=torch.int32, device="cuda")
    sc = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
    zr = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
    H().harp_quantize_pack(d.dev(W), bits, qw, sc, zr)
    torch.cuda.synchronize()
    got_w = qw.cpu().numpy().view(np.uint32)
    got_s = sc.cpu().numpy().view(np.uint16)
    got_z = zr.cpu().numpy().view(np.uint16)
    assert np.array_equal(got_s, s_ref.view(np.uint16))
    assert np.array_equal(got_z, z_ref.view(np.uint16))
    assert np.array_equal(got_w, words_ref)


def test_prepare_then_linear():
    """GPU rotate -> quantize -> pack, then the fused linear: the codes match
    the oracle pipeline (float64 rotation, float32-precision decisions)
    except where the float32 rotation moves a weight across a decision
    boundary (rarely, by one code); the linear approximates W x."""
    d = D()
    N, K, b = 512, 1024, 256
    V = S.rotation(K, b, rng(6))
    U = S.rotation(N, b, rng(7))
    out = S.outlier_channels(K, rng(8))
    W = S.dense_weight(N, K, rng(9), 0.02, out).astype(np.float32)
    Vd, Ud = d.dev_rotation(V), d.dev_rotation(U)
    Wp = torch.empty((N, K), dtype=torch.float32, device="cuda")
    ws = torch.empty(H().harp_rotate_weight_workspace_bytes(N, K), dtype=torch.uint8,
                     device="cuda")
    H().harp_rotate_weight(Vd, Ud, d.dev(W), Wp, ws)
    qw = torch.empty((N, K * 2 // 32), dtype=torch.int32, device="cuda")
    sc = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
    zr = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
    H().harp_quantize_pack(Wp, 2, qw, sc, zr)
    Wp_ref = O.rotate_weight(W.astype(np.float64), U.cs, U.sign_bits, b, V.cs, V.sign_bits, b)
    q_ref, s_ref, z_ref = O.quantize(Wp_ref.astype(np.float32), 2, arith="f32")
    got_q = O.unpack(qw.cpu().numpy().view(np.uint32), 2, K)
    same_sz = (sc.cpu().numpy().view(np.uint16) == s_ref.view(np.uint16)) & \
              (zr.cpu().numpy().view(np.uint16) == z_ref.view(np.uint16))
    assert same_sz.mean() > 0.99
    rows = np.repeat(same_sz, 64, axis=1)
    diff = np.abs(got_q.astype(int) - q_ref.astype(int))[rows]
    assert diff.max() <= 1 and (diff > 0).mean() < 2e-3
    # the prepared layer in the hot path
    Wq = H().QWeight(qw, sc, zr, N, K, 2)
    x = S.activations(4, K, rng(10), "f32", out)
    y = torch.empty((4, N), dtype=torch.float32, device="cuda")
    wsl = d.workspace(4, N, K)
    H().harp_linear_fused(Vd, Wq, Ud, d.dev(x), y, wsl)
    got = y.cpu().numpy().astype(np.float64)
    # parity: the oracle's linear on the very buffers the GPU produced
    y_or = O.linear(x.astype(np.float64), qw.cpu().numpy().view(np.uint32),
                    sc.cpu().numpy().view(np.float16), zr.cpu().numpy().view(np.float16), 2,
                    V.cs, V.sign_bits, b, U.cs, U.sign_bits, b)
    r = O.rel_l2(got, y_or)
    print(f"[prepare+linear 2-bit] rel_l2 vs oracle on the same buffers = {r:.3e}", flush=True)
    assert r <= 2e-5
    # and the quantized layer approximates the dense one
    y_ref = x.astype(np.float64) @ W.astype(np.float64).T
    err = O.rel_l2(got, y_ref)
    print(f"[prepare+linear 2-bit] rel_l2 vs W x = {err:.3f}", flush=True)
    assert err < 0.5
