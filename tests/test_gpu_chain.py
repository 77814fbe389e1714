"""GPU parity of harp_linear_chain: stacks of dependent decode linears in one
launch (HARP technical summary §2.4 per layer, §2.1-2.2 for the sides).

Every checked layer is compared with the oracle's linear applied to the
GPU's own stored input of that layer (the previous layer's stored output),
so errors do not compound and each layer meets the float32 bar of the decode
product (x~ not rounded).  bf16 outputs: the oracle output rounded to bf16,
within one bf16 ulp plus the float32 bar.  Stacks longer than 48 layers run
as several launches; one workspace serves repeated calls.
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


def chain_inputs(dim, n_layers, bits, M, seed):
    cfg = S.Config(20 + seed, "chain", (S.Linear("c", dim, dim, dim, dim),), (bits,), (M,))
    lis = [S.layer_inputs(cfg, 0, bits, M, inst=i) for i in range(n_layers)]
    return lis


def run_chain(lis, ydt, ws=None):
    d = D()
    M, dim = lis[0].M, lis[0].lin.K
    layers = []
    for li in lis:
        y = torch.empty((M, dim), dtype=ydt, device="cuda")
        layers.append((d.dev_rotation(li.V), d.dev_qweight(li.W), d.dev_rotation(li.U), y))
    x = d.dev_x(lis[0].x, lis[0].x_dtype)
    if ws is None:
        ws = torch.zeros(H().harp_linear_chain_workspace_bytes(dim), dtype=torch.uint8,
                         device="cuda")
    H().harp_linear_chain(layers, x, ws)
    torch.cuda.synchronize()
    return [L[3] for L in layers], ws


def check_layers(lis, ys, check):
    d = D()
    x64 = d.x_f64(lis[0].x, lis[0].x_dtype)
    for l, (li, y) in enumerate(zip(lis, ys)):
        got = d.host(y)
        if l in check:
            ref = O.linear(x64, li.W.words, li.W.scale.view(np.float16),
                           li.W.zero.view(np.float16), li.bits, li.V.cs, li.V.sign_bits,
                           li.lin.b_v, li.U.cs, li.U.sign_bits, li.lin.b_u)
            if y.dtype == torch.bfloat16:
                refb = O.bf16_round(ref)
                ulp = np.ldexp(1.0, np.frexp(np.abs(refb))[1] - 8)
                delta = FP32_PATH_TOL * np.sqrt(np.mean(ref ** 2))
                assert np.all(np.abs(got - refb) <= ulp + delta), l
                assert np.mean(got != refb) < 0.01
                r = O.rel_l2(got, ref)
            else:
                r = O.rel_l2(got, ref)
                assert r <= FP32_PATH_TOL, (l, r)
            print(f"[chain layer {l}/{len(lis)} {y.dtype} M={li.M}] rel_l2={r:.3e}", flush=True)
        x64 = got            # the next layer's input is this layer's stored output


@pytest.mark.parametrize("dim,n_layers,bits,M,ydt", [
    (4096, 3, 2, 1, torch.bfloat16), (4096, 2, 4, 2, torch.float32),
    (4096, 2, 3, 4, torch.bfloat16), (4096, 2, 2, 3, torch.float32),
    (8192, 2, 2, 1, torch.bfloat16), (8192, 2, 4, 2, torch.float32),
])
def test_chain_parity(dim, n_layers, bits, M, ydt):
    lis = chain_inputs(dim, n_layers, bits, M, seed=dim // 4096 + bits)
    ys, ws = run_chain(lis, ydt)
    assert int(ws[4:8].view(torch.int32).item()) == 0      # no wait ran out
    check_layers(lis, ys, set(range(n_layers)))


def test_chain_longer_than_one_launch_and_reused_workspace():
    """50 layers (two launches of 48 and 2), twice on one workspace: bitwise
    equal results, and the layers around the launch boundary checked."""
    lis = chain_inputs(4096, 50, 2, 1, seed=7)
    ys1, ws = run_chain(lis, torch.bfloat16)
    ys1 = [y.clone() for y in ys1]
    ys2, ws = run_chain(lis, torch.bfloat16, ws)
    for a, b in zip(ys1, ys2):
        assert torch.equal(a, b)
    assert int(ws[4:8].view(torch.int32).item()) == 0
    check_layers(lis, ys2, {0, 1, 46, 47, 48, 49})
