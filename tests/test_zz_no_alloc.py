"""omm_gemm_noalloc (split-K partials in the library's static per-GPU scratch,
nothing allocated) against omm_gemm on the same inputs: the same kernels in
the same order, so the outputs must be identical, and both within the
tolerance of the oracle.  Two calls in a row, the second smaller, so the
second reads a scratch that still holds the first call's partials."""
import numpy as np
import pytest
import torch

import oracle
from onnx_matmul_family_amd import synth
from tests.gpu_util import check_close, dev, host_f64

pytestmark = pytest.mark.gpu

om = pytest.importorskip("onnx_matmul_family_amd._omm")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    om.lib()


def case(rng, dt, M, N, K, tB, cform):
    A = synth.store(synth.normal(rng, (M, K), 0.05), dt)
    B = synth.store(synth.normal(rng, (N, K) if tB else (K, N), 0.05), dt)
    C = None if cform is None else synth.store(synth.uniform(rng, cform, -0.1, 0.1), dt)
    return A, B, C


def run_both(A, B, C, dt, alpha, beta, tB):
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dt]
    dA, dB = dev(A, dt), dev(B, dt)
    dC = dev(C, dt) if C is not None else None
    M, N = A.shape[0], (B.shape[0] if tB else B.shape[1])
    Y0 = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
    Y1 = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
    om.gemm(dA, dB, dC, alpha, beta, 0, tB, Y0)
    om.gemm_noalloc(dA, dB, dC, alpha, beta, 0, tB, Y1)
    torch.cuda.synchronize()
    return Y0, Y1


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_noalloc_matches_gemm_twice(dt):
    rng = np.random.default_rng(77)
    # 1: few output tiles, long K -> 128x128 split-K (16 K ranges x 64 x 4096 fp32 partials, 16 MiB)
    A, B, C = case(rng, dt, 64, 4096, 8192, 0, (4096,))
    Y0, Y1 = run_both(A, B, C, dt, 0.5, -1.5, 0)
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))
    y, t = oracle.gemm(A, B, C, 0.5, -1.5, 0, 0, dt=dt)
    check_close(host_f64(Y1), y, 0.5 * t + 1.5 * np.abs(oracle.decode(C, dt))[None, :], dt, "noalloc split-K")
    # 2: smaller, decode-like (16 rows, B stored (N, K), few columns and K past
    # the single-pass kernel's range) -> the skinny split-K kernel (32 x 16 x 1000 fp32)
    A, B, C = case(rng, dt, 16, 1000, 20480, 1, (16, 1000))
    Y0, Y1 = run_both(A, B, C, dt, 1.0, 1.0, 1)
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))
    y, t = oracle.gemm(A, B, C, 1.0, 1.0, 0, 1, dt=dt)
    check_close(host_f64(Y1), y, t + np.abs(oracle.decode(C, dt)).reshape(16, 1000), dt, "noalloc skinny")


def test_noalloc_without_split_and_fp32():
    """Shapes that split nothing (256x256 tiles; fp32) take no scratch and match omm_gemm."""
    rng = np.random.default_rng(78)
    A, B, C = case(rng, "bf16", 1024, 1024, 512, 1, (1024,))
    Y0, Y1 = run_both(A, B, C, "bf16", 1.0, 1.0, 1)
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))
    A, B, C = case(rng, "f32", 70, 90, 300, 0, None)
    Y0, Y1 = run_both(A, B, C, "f32", 1.0, 0.0, 0)
    assert torch.equal(Y0, Y1)


def test_noalloc_rejects_oversized():
    """Partials beyond the 32 MiB scratch: OMM_ERR_SCRATCH, nothing launched (Y untouched)."""
    M, N, K = 16, 8176, 131328
    A = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    Y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(om.OmmError) as e:
        om.gemm_noalloc(A, B, None, 1.0, 0.0, 0, 1, Y)
    assert e.value.code == -8
    torch.cuda.synchronize()
    assert bool((Y == 3.0).all())
