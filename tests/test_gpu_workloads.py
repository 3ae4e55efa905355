"""GPU parity at the five benchmark workloads' full sizes, through the same
entry points and launch configuration the benchmark times.

Every output element is compared with the oracle for the fp32 Gemm, the bf16
MatMul broadcast, the bf16 8192^3 Gemm (in four row ranges, one test each, so
that no single test runs the oracle for minutes) and the int8 QLinearMatMul
(bit for bit).  The GroupedMatMul output (268M elements, about 20 minutes of
oracle time) is compared on complete output rows: eight rows from every routed
256-row tile, at positions that cover every row slot of a tile across the
launch, plus a random sample of elements; the routing itself (tile table and
group-sorted pairs in the workspace) is checked to be a valid counting sort of
the indices.  Outputs start as NaN, so an element the kernels never write
fails the comparison."""
import numpy as np
import pytest
import torch

import oracle
from onnx_matmul_family_amd import synth
from tests.gpu_util import (check_close, check_routing, dev, host_f32, host_f64, routing_from_workspace,
                            sample_indices, tile_row_pairs)

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
    """The literal fp32 bound |err| <= 1e-5 t + 1e-6 with t = sum_k |a b| (alpha and beta*C not added)."""
    c = synth.gemm_f32_64x32x48()
    Y = torch.full((64, 32), float("nan"), dtype=torch.float32, device="cuda")
    om.gemm(dev(c["A"]), dev(c["B"]), dev(c["C"]), c["alpha"], c["beta"], c["transA"], c["transB"], Y)
    torch.cuda.synchronize()
    y, t = oracle.gemm(c["A"], c["B"], c["C"], c["alpha"], c["beta"], c["transA"], c["transB"])
    check_close(host_f64(Y), y, t, "f32", "Gemm fp32 64x32x48")


def test_matmul_bf16_bcast_full():
    c = synth.matmul_bf16_bcast()
    Y = torch.full((8, 16, 512, 768), float("nan"), dtype=torch.bfloat16, device="cuda")
    om.matmul(dev(c["A"], "bf16"), dev(c["B"], "bf16"), Y)
    torch.cuda.synchronize()
    got = host_f32(Y)
    y, t = oracle.matmul(c["A"], c["B"], dt="bf16")
    check_close(got, y, t, "bf16", "MatMul bf16 [8,1,512,1024]x[1,16,1024,768]")


@pytest.fixture(scope="module")
def gemm8192():
    """The 8192^3 Gemm computed once on the GPU; its output kept on the host as fp32 (exact for bf16)."""
    c = synth.gemm_bf16_8192()
    Y = torch.full((8192, 8192), float("nan"), dtype=torch.bfloat16, device="cuda")
    om.gemm(dev(c["A"], "bf16"), dev(c["B"], "bf16"), dev(c["C"], "bf16"), 1.0, 1.0, 0, 1, Y)
    torch.cuda.synchronize()
    got = host_f32(Y)
    del Y
    return c, got


@pytest.mark.parametrize("part", range(4))
def test_gemm_bf16_8192_full(gemm8192, part):
    """Rows [2048 part, 2048 (part + 1)) of the 8192^3 Gemm, every element."""
    c, got = gemm8192
    r0, r1 = 2048 * part, 2048 * (part + 1)
    sel = np.arange(r0 * 8192, r1 * 8192, dtype=np.int64)
    y, t = oracle.gemm(c["A"], c["B"], c["C"], 1.0, 1.0, 0, 1, dt="bf16", sel=sel)
    check_close(got[r0:r1], y, t, "bf16", "Gemm bf16 8192^3 transB rows %d..%d" % (r0, r1))


def test_qlinear_i8_4096_full_exact():
    c = synth.qlinear_i8_4096()
    keys = ("a", "a_scale", "a_zero_point", "b", "b_scale", "b_zero_point", "y_scale", "y_zero_point")
    y = torch.full((4096, 4096), 77, dtype=torch.int8, device="cuda")
    om.qlinear_matmul(*(dev(c[k]) for k in keys), y)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    ref, _ = oracle.qlinear_matmul(*(c[k] for k in keys))
    bad = np.argwhere(got != ref)
    assert bad.size == 0, "%d of %d outputs differ, first at %s: got %d want %d" % (
        len(bad), got.size, tuple(bad[0]), got[tuple(bad[0])], ref[tuple(bad[0])])


def test_grouped_bf16_moe_tile_rows():
    c = synth.grouped_bf16_moe()
    M, S = c["group_indices"].shape
    G, K, N = c["weights"].shape
    out = torch.full((M, S, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    out, ws = om.grouped_matmul(dev(c["input"], "bf16"), dev(c["weights"], "bf16"), dev(c["group_indices"]),
                                dev(c["bias"], "bf16"), output=out)
    assert om.grouped_matmul_check(ws) == 0
    idx = c["group_indices"].reshape(-1)

    # the routing: a counting sort of the pairs by group, cut into 256-row tiles
    bad, tiles, sorted_ids, raw = routing_from_workspace(ws, M, S, G, 256)
    assert bad == 0
    check_routing(idx, tiles, sorted_ids, G, 256, raw)
    # eight complete output rows per routed tile, over every row slot of a tile
    pairs = tile_row_pairs(tiles, sorted_ids, 8, 256)
    assert len(pairs) > 3000
    sel = (pairs[:, None] * N + np.arange(N, dtype=np.int64)[None, :]).ravel()
    y, t = oracle.grouped_matmul(c["input"], c["weights"], c["group_indices"], c["bias"], dt="bf16", sel=sel)
    check_close(pick(out, sel), y, t, "bf16", "GroupedMatMul bf16 16384x8 -> 2048, G=64: %d whole rows" % len(pairs))

    # plus a random sample of single elements anywhere, and every element written
    sel = sample_indices(out.numel(), 50000, 4)
    y, t = oracle.grouped_matmul(c["input"], c["weights"], c["group_indices"], c["bias"], dt="bf16", sel=sel)
    check_close(pick(out, sel), y, t, "bf16", "GroupedMatMul bf16 sampled")
    assert torch.isfinite(out.float()).all()
