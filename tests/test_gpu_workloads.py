"""GPU parity at the five benchmark workloads' full sizes, through the same
entry points and launch configuration the benchmark times.

The oracle computes a random sample of output elements one by one (plus the
first and last element); the rest of each output is checked through
properties that hold at any size (every element written and finite, int8
outputs inside the type's range)."""
import numpy as np
import pytest
import torch

import oracle
from onnx_matmul_family_amd import synth
from tests.gpu_util import check_close, dev, host_f64, sample_indices

pytestmark = pytest.mark.gpu

om = pytest.importorskip("onnx_matmul_family_amd._omm")


def pick(t, sel):
    """Sampled elements of a GPU tensor, gathered on the device, as float64."""
    return host_f64(t.reshape(-1)[torch.from_numpy(sel).cuda()])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    om.lib()


def test_gemm_f32_64x32x48_full():
    c = synth.gemm_f32_64x32x48()
    Y = om.gemm(dev(c["A"]), dev(c["B"]), dev(c["C"]), c["alpha"], c["beta"], c["transA"], c["transB"])
    torch.cuda.synchronize()
    y, t = oracle.gemm(c["A"], c["B"], c["C"], c["alpha"], c["beta"], c["transA"], c["transB"])
    # the beta*C term joins t in the tolerance scale (its own fp32 rounding)
    check_close(host_f64(Y), y, t + abs(c["beta"]) * np.abs(np.broadcast_to(c["C"], y.shape)), "f32",
                "Gemm fp32 64x32x48")


def test_matmul_bf16_bcast_sampled():
    c = synth.matmul_bf16_bcast()
    Y = torch.full((8, 16, 512, 768), float("nan"), dtype=torch.bfloat16, device="cuda")
    om.matmul(dev(c["A"], "bf16"), dev(c["B"], "bf16"), Y)
    torch.cuda.synchronize()
    assert torch.isfinite(Y.float()).all()
    sel = sample_indices(Y.numel(), 100000, 1)
    y, t = oracle.matmul(c["A"], c["B"], dt="bf16", sel=sel)
    check_close(pick(Y, sel), y, t, "bf16", "MatMul bf16 [8,1,512,1024]x[1,16,1024,768]")


def test_gemm_bf16_8192_sampled():
    c = synth.gemm_bf16_8192()
    Y = torch.full((8192, 8192), float("nan"), dtype=torch.bfloat16, device="cuda")
    om.gemm(dev(c["A"], "bf16"), dev(c["B"], "bf16"), dev(c["C"], "bf16"), 1.0, 1.0, 0, 1, Y)
    torch.cuda.synchronize()
    assert torch.isfinite(Y.float()).all()
    sel = sample_indices(Y.numel(), 50000, 2)
    y, t = oracle.gemm(c["A"], c["B"], c["C"], 1.0, 1.0, 0, 1, dt="bf16", sel=sel)
    check_close(pick(Y, sel), y, t, "bf16", "Gemm bf16 8192^3 transB")


def test_qlinear_i8_4096_sampled_exact():
    c = synth.qlinear_i8_4096()
    y = om.qlinear_matmul(*(dev(c[k]) for k in ("a", "a_scale", "a_zero_point", "b", "b_scale", "b_zero_point",
                                                 "y_scale", "y_zero_point")))
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    sel = sample_indices(got.size, 100000, 3)
    ref, _ = oracle.qlinear_matmul(*(c[k] for k in ("a", "a_scale", "a_zero_point", "b", "b_scale",
                                                    "b_zero_point", "y_scale", "y_zero_point")), sel=sel)
    assert np.array_equal(got.ravel()[sel], ref)
    # whole rows and columns exactly, so every tile position is covered
    rows = np.array([0, 255, 256, 2047, 4095])
    for r in rows:
        ref_r, _ = oracle.qlinear_matmul(*(c[k] for k in ("a", "a_scale", "a_zero_point", "b", "b_scale",
                                                          "b_zero_point", "y_scale", "y_zero_point")),
                                         sel=np.arange(r * 4096, (r + 1) * 4096))
        assert np.array_equal(got[r], ref_r), r


def test_grouped_bf16_moe_sampled():
    c = synth.grouped_bf16_moe()
    out = torch.full((16384, 8, 2048), float("nan"), dtype=torch.bfloat16, device="cuda")
    out, ws = om.grouped_matmul(dev(c["input"], "bf16"), dev(c["weights"], "bf16"), dev(c["group_indices"]),
                                dev(c["bias"], "bf16"), output=out)
    assert om.grouped_matmul_check(ws) == 0
    assert torch.isfinite(out.float()).all()
    sel = sample_indices(out.numel(), 50000, 4)
    y, t = oracle.grouped_matmul(c["input"], c["weights"], c["group_indices"], c["bias"], dt="bf16", sel=sel)
    check_close(pick(out, sel), y, t, "bf16", "GroupedMatMul bf16 16384x8 -> 2048, G=64")
