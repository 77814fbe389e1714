"""GPU parity of the one-row 2- and 4-bit decode product on the block-scaled
matrix cores (the fused linear at M = 1 on layers of at least 2^27 weights, HARP
technical summary §2.4 with the per-group uniform grid standing in for the
quantizer).  2-bit codes enter as FP4 values, 4-bit codes (fused linear
only) as FP8 values.

x~ is not rounded on this path (eight FP8 planes of base-16 digits per
quantization group carry it to 2^-28 of the group maximum, and every
matrix-core sum is exact), so every case meets the float32 bar of the
decode product against the unrounded oracle.  The cases
cover each way the K dimension is cut (one slice; split K over 4 and 8
slices, equal and ragged), planes written by the input rotation's last
launch (b_V = 256 / 4096 / 8192, both angle formats), the output rotation
applied by the product (b_U = 256, float32 and bf16 y), the product alone
through harp_deq_gemv_ws, x~
with zero, tiny, subnormal and outlier blocks, the edge
weight format (zero-points 0 and 2^B - 1, subnormal fp16 scales), a
workspace reused across shapes and products (the split-K counters end at
zero), repeatability, and the no-allocation entry point.
"""
import numpy as np
import pytest
import torch

from oracle import harp_oracle as O
from synth import workloads as S

pytestmark = pytest.mark.gpu

FP32_PATH_TOL = 2e-5


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
    return np.random.default_rng(np.random.SeedSequence([4417, *k]))


def oracle_yp(li, xt, chunk=2048):
    """Unrounded oracle product y' = w_hat x~, rows of w_hat in chunks."""
    lin, w = li.lin, li.W
    yp = np.empty((xt.shape[0], lin.N))
    s16, z16 = w.scale.view(np.float16), w.zero.view(np.float16)
    for r0 in range(0, lin.N, chunk):
        rr = slice(r0, min(r0 + chunk, lin.N))
        wh = O.dequant(O.unpack(w.words[rr], w.bits, lin.K), s16[rr], z16[rr])
        yp[:, rr] = xt @ wh.T
    return yp


def oracle_y(li, x64):
    """Unrounded oracle linear: x~ = F_V x, y' = w_hat x~, y = F_U^T y'."""
    lin = li.lin
    xt = O.forward(x64, D().cs64(li.V), li.V.sign_bits, lin.b_v)
    return O.transpose(oracle_yp(li, xt), D().cs64(li.U), li.U.sign_bits, lin.b_u)


def run(li, ws=None, noalloc=False):
    d = D()
    lin = li.lin
    V, U, W = d.dev_rotation(li.V), d.dev_rotation(li.U), d.dev_qweight(li.W)
    x = d.dev_x(li.x, li.x_dtype)
    y = torch.empty((li.M, lin.N), dtype=torch.float32, device="cuda")
    if noalloc:
        H().harp_linear_fused_noalloc(V, W, U, x, y)
    else:
        H().harp_linear_fused(V, W, U, x, y, d.workspace(li.M, lin.N, lin.K) if ws is None else ws)
    torch.cuda.synchronize()
    return y


def check(name, li, y):
    ref = oracle_y(li, D().x_f64(li.x, li.x_dtype))
    r = O.rel_l2(D().host(y), ref)
    print(f"[{name}] rel_l2={r:.3e}", flush=True)
    assert r <= FP32_PATH_TOL
    return r


def layer(K, N, b_v, b_u, seed, bits=2, xdt="bf16", angles="f32"):
    cfg = S.Config(60 + seed, "f4", (S.Linear("f", K, N, b_v, b_u),), (bits,), (1,),
                   x_dtype=xdt)
    return S.layer_inputs(cfg, 0, bits, 1, angles=angles)


# (K, N, b_v, b_u), all at least 2^27 weights: one slice of 64 steps (1024
# tiles); split K 4 ways (512 tiles, 32 steps each); 4 ragged slices of
# 16-17 step pairs; 8 ragged slices of 17 step pairs (256 tiles)
F4_SHAPES = [(8192, 16384, 8192, 256), (16384, 8192, 256, 8192), (16640, 8192, 256, 256),
             (34816, 4096, 256, 4096)]


@pytest.mark.parametrize("K,N,b_v,b_u", F4_SHAPES)
def test_f4_shapes(K, N, b_v, b_u):
    li = layer(K, N, b_v, b_u, seed=K % 97)
    check(f"f4 {K}->{N}", li, run(li))


# 4-bit codes on the same product as FP8 values: one slice with the output
# rotation in the launch (8192 -> 28672 shape family), split K 4 ways, 8
# ragged slices; wide zero-points (0 and 15) and subnormal fp16 scales
F4_SHAPES_4BIT = [(8192, 16384, 8192, 256, "f32"), (16384, 8192, 256, 8192, "int8"),
                  (34816, 4096, 256, 4096, "f32")]


@pytest.mark.parametrize("K,N,b_v,b_u,angles", F4_SHAPES_4BIT)
def test_f4_shapes_4bit(K, N, b_v, b_u, angles):
    li = layer(K, N, b_v, b_u, seed=K % 89 + 4, bits=4, angles=angles)
    check(f"f4 4-bit {K}->{N} {angles}", li, run(li))


def test_f4_wide_weights_4bit():
    li = layer(16384, 8192, 256, 8192, seed=7, bits=4)
    w = S.qweight(8192, 16384, 4, rng(5), spread="wide")
    li = S.LayerInputs(li.lin, 4, 1, li.x, li.x_dtype, li.V, li.U, w)
    check("f4 4-bit wide weights", li, run(li))


@pytest.mark.parametrize("K,N,b_v,angles,xdt", [
    (4096, 32768, 4096, "int8", "f32"), (4096, 32768, 4096, "f32", "bf16"),
    (16384, 8192, 8192, "int8", "bf16"), (8192, 16384, 8192, "f32", "f32"),
    (28672, 8192, 256, "int8", "f32"), (16384, 8192, 256, "f32", "bf16")])
def test_f4_planes_from_rotation(K, N, b_v, angles, xdt):
    """b_V = 256 / 4096 / 8192 input sides: the rotation's last launch writes
    the product's planes itself (float32 and int8-stored angles, bf16 and
    float32 x, one to 112 blocks)."""
    li = layer(K, N, b_v, 256, seed=b_v % 83 + K % 7, xdt=xdt, angles=angles)
    check(f"f4 planes from rotation {K}->{N} b_v={b_v} {angles} {xdt}", li, run(li))


@pytest.mark.parametrize("angles", ["f32", "int8"])
def test_f4_output_rotation_in_product(angles):
    """b_U = 256 with one K slice: the product's second workgroup of each
    256-output block applies F_U^T.  float32 output against the oracle; the
    bf16 output is the float32 output rounded to nearest even, bit for bit;
    repeated calls on one workspace agree and leave the counters at zero."""
    li = layer(8192, 16384, 8192, 256, seed=9, angles=angles)
    d = D()
    V, U, W = d.dev_rotation(li.V), d.dev_rotation(li.U), d.dev_qweight(li.W)
    x = d.dev_x(li.x, li.x_dtype)
    ws = d.workspace(1, 16384, 8192)
    y32 = torch.empty((1, 16384), dtype=torch.float32, device="cuda")
    y16 = torch.empty((1, 16384), dtype=torch.bfloat16, device="cuda")
    y32b = torch.empty_like(y32)
    H().harp_linear_fused(V, W, U, x, y32, ws)
    H().harp_linear_fused(V, W, U, x, y16, ws)
    H().harp_linear_fused(V, W, U, x, y32b, ws)
    torch.cuda.synchronize()
    assert torch.equal(y32, y32b)
    assert torch.equal(y16, y32.to(torch.bfloat16))
    assert int(ws[:2048].view(torch.int32).abs().sum().item()) == 0
    check(f"f4 output rotation in the product {angles}", li, y32)


@pytest.mark.parametrize("K,N,bits", [(8192, 28672, 2), (28672, 8192, 2), (34816, 4096, 2),
                                      (28672, 8192, 4)])
def test_f4_deq_gemv_ws(K, N, bits):
    """The product alone (harp_deq_gemv_ws with a workspace: one K slice at
    28672 rows, 4 and 8 slices below) against the oracle product on the
    same float32 x~ (random, with a zero group and an outlier); twice on one
    workspace, bitwise equal, counters left at zero; without a workspace the
    vector-ALU product, within the same bar.  4-bit codes take the vector
    product here even with a workspace (the matrix-core form is no faster
    alone; the fused linear uses it)."""
    li = layer(K, N, 256, 256, seed=N % 89, bits=bits)
    g = rng(3, K)
    xt = g.standard_normal((1, K)).astype(np.float32)
    xt[0, 128:192] = 0.0
    xt[0, 1000] = 500.0
    d = D()
    W = d.dev_qweight(li.W)
    ws = torch.zeros(H().harp_deq_gemv_workspace_bytes(1, N, K), dtype=torch.uint8,
                     device="cuda")
    x_d = d.dev(xt)
    outs = []
    for w in (ws, ws, None):
        yt = torch.empty((1, N), dtype=torch.float32, device="cuda")
        H().harp_deq_gemv_ws(W, x_d, yt, w)
        outs.append(yt)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    assert int(ws[:2048].view(torch.int32).abs().sum().item()) == 0
    ref = oracle_yp(li, xt.astype(np.float64))
    for name, y in (("with workspace", outs[0]), ("no workspace", outs[2])):
        r = O.rel_l2(d.host(y), ref)
        print(f"[f4 deq_gemv_ws {K}->{N} {bits}-bit {name}] rel_l2={r:.3e}", flush=True)
        assert r <= FP32_PATH_TOL


def test_f4_special_inputs():
    """x~ blocks of zeros, of tiny normal and subnormal float32 values, with
    a single large outlier, and of mixed magnitudes (b_V = 2, so each block
    of x reaches x~ mixed only within pairs)."""
    li = layer(8192, 16384, 2, 256, seed=3, xdt="f32")
    g = rng(1)
    x = g.standard_normal((1, 8192)).astype(np.float32)
    x[0, 0:64] = 0.0                                   # a whole group of zeros
    x[0, 64:96] = 1e-35 * g.standard_normal(32)        # tiny normals
    x[0, 96:128] = 3e-41 * np.sign(g.standard_normal(32))   # float32 subnormals
    x[0, 128:160] = 1e-3 * g.standard_normal(32)
    x[0, 140] = 3e4                                    # one outlier in that block
    x[0, 160:192] = np.ldexp(g.standard_normal(32), g.integers(-60, 40, 32))
    li = S.LayerInputs(li.lin, 2, 1, x, "f32", li.V, li.U, li.W)
    check("f4 special x", li, run(li))


def test_f4_wide_weights():
    """Zero-points at 0 and 3 and subnormal fp16 scales on the split path."""
    li = layer(16384, 8192, 256, 8192, seed=4)
    w = S.qweight(8192, 16384, 2, rng(2), spread="wide")
    li = S.LayerInputs(li.lin, 2, 1, li.x, li.x_dtype, li.V, li.U, w)
    check("f4 wide weights", li, run(li))


def test_f4_repeatable_and_counters_left_zero():
    """Two calls on one workspace are bitwise equal; a larger batch on the
    same workspace in between (its own split K) disturbs nothing; the
    counter area ends at zero."""
    li1 = layer(16384, 8192, 256, 8192, seed=5)
    cfg16 = S.Config(65, "f4", (li1.lin,), (2,), (16,))
    li16 = S.layer_inputs(cfg16, 0, 2, 16)
    li16 = S.LayerInputs(li1.lin, 2, 16, li16.x, li16.x_dtype, li1.V, li1.U, li1.W)
    nbytes = max(H().harp_linear_workspace_bytes(M, 8192, 16384) for M in (1, 16))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    a = run(li1, ws).clone()
    y16 = run(li16, ws)
    b = run(li1, ws)
    assert torch.equal(a, b)
    check("f4 after reuse", li1, b)
    ref16 = oracle_y(li16, D().x_f64(li16.x, li16.x_dtype))
    assert O.rel_l2(D().host(y16), ref16) <= FP32_PATH_TOL
    assert int(ws[:2048].view(torch.int32).abs().sum().item()) == 0


@pytest.mark.parametrize("K,N,b_v,b_u,bits", [(8192, 16384, 8192, 256, 2),
                                             (16384, 8192, 256, 8192, 2),
                                             (8192, 16384, 8192, 256, 4)])
def test_f4_noalloc(K, N, b_v, b_u, bits):
    """No-allocation entry point: one K slice (no counters) on the
    block-scaled path (8192 -> 16384, 2- and 4-bit codes); 16384 -> 8192
    needs split K, so it takes the vector-ALU product there."""
    li = layer(K, N, b_v, b_u, seed=6, bits=bits)
    check(f"f4 noalloc {K}->{N} {bits}-bit", li, run(li, noalloc=True))
