"""harp_linear_fused_noalloc (no workspace, library-held device scratch)
against harp_linear_fused, both through the C ABI.

Two calls in a row on one GPU, the second smaller than the first, each
compared with harp_linear_fused on the same inputs: bitwise for M < 64 (the
same kernels in the same order), within the bf16 matrix-core bar at M = 512
(the workspace path may split K, the scratch path runs one K slice, so the
float32 accumulation order differs).  A call that needs more than the
scratch is rejected before anything is launched.
"""
import numpy as np
import pytest
import torch

from synth import workloads as S

pytestmark = pytest.mark.gpu

MFMA_PATH_TOL = 3e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotated_bit_amd  # noqa: F401  (raises if libharp.so is missing)
    yield


def rel_l2(a, r):
    a = a.double().cpu().numpy()
    r = r.double().cpu().numpy()
    return float(np.linalg.norm(a - r) / np.linalg.norm(r))


def run_both(cfg, lin, bits, M):
    import devbuf as d
    import rotated_bit_amd as H
    li = S.layer_inputs(S.CONFIGS[cfg], lin, bits, M)
    V, U, W = d.dev_rotation(li.V), d.dev_rotation(li.U), d.dev_qweight(li.W)
    x = d.dev_x(li.x, li.x_dtype)
    N = li.lin.N
    y_na = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    H.harp_linear_fused_noalloc(V, W, U, x, y_na)
    y_ref = torch.empty((M, N), dtype=torch.float32, device="cuda")
    H.harp_linear_fused(V, W, U, x, y_ref, d.workspace(M, N, li.lin.K))
    torch.cuda.synchronize()
    return y_na, y_ref


def test_noalloc_two_calls_second_smaller():
    # 4096 x 4096 at M = 512: 1 KB + 4 MiB bf16 x~ + 8 MiB y' of scratch
    y_na, y_ref = run_both("q8b_prefill", 0, 2, 512)
    r = rel_l2(y_na, y_ref)
    print(f"[noalloc 4096x4096 M=512] rel_l2 vs harp_linear_fused = {r:.3e}", flush=True)
    assert r <= MFMA_PATH_TOL
    # then 11008 -> 4096 at M = 16 on the same scratch (left holding the
    # first call's data): the same kernels as the workspace path
    y_na, y_ref = run_both("l7b_mlp", 1, 2, 16)
    print(f"[noalloc 11008x4096 M=16] max |diff| = "
          f"{(y_na - y_ref).abs().max().item():.3e}", flush=True)
    assert torch.equal(y_na, y_ref)
    # and a decode call (M = 1, two launches)
    y_na, y_ref = run_both("l7b_decode", 0, 2, 1)
    assert torch.equal(y_na, y_ref)


def test_noalloc_rejects_calls_beyond_the_scratch():
    import devbuf as d
    import rotated_bit_amd as H
    # 4096 -> 28672 at M = 512: y' alone is 56 MiB, beyond the 32 MiB scratch
    M, K, N = 512, 4096, 28672
    cfg = S.Config(13, "big", (S.Linear("b", K, N, 4096, 256),), (2,), (M,))
    li = S.layer_inputs(cfg, 0, 2, M)
    V, U, W = d.dev_rotation(li.V), d.dev_rotation(li.U), d.dev_qweight(li.W)
    x = d.dev_x(li.x, li.x_dtype)
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(H.HarpError) as e:
        H.harp_linear_fused_noalloc(V, W, U, x, y)
    assert e.value.status == H._lib.HARP_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0))
