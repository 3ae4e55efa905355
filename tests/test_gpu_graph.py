"""The five workloads' calls captured into HIP graphs and replayed: every replay
must reproduce the eager call's output bit for bit (no memset or other node
whose replays differ).  Between the replays the program's own eager work
overwrites the outputs and the stream is synchronised."""
import numpy as np
import pytest
import torch

from onnx_matmul_family_amd import synth
from onnx_matmul_family_amd.hostdev import dev

pytestmark = pytest.mark.gpu

om = pytest.importorskip("onnx_matmul_family_amd._omm")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    om.lib()


def workloads():
    c = synth.gemm_f32_64x32x48()
    d1 = dict(A=dev(c["A"]), B=dev(c["B"]), C=dev(c["C"]), Y=torch.empty((64, 32), device="cuda"))
    yield "gemm_f32_64x32x48", d1["Y"], lambda: om.gemm(d1["A"], d1["B"], d1["C"], c["alpha"], c["beta"], 1, 1, d1["Y"])
    c2 = synth.matmul_bf16_bcast()
    d2 = dict(A=dev(c2["A"], "bf16"), B=dev(c2["B"], "bf16"),
              Y=torch.empty((8, 16, 512, 768), dtype=torch.bfloat16, device="cuda"))
    yield "matmul_bf16_bcast", d2["Y"], lambda: om.matmul(d2["A"], d2["B"], d2["Y"])
    del d2
    c3 = synth.gemm_bf16_8192()
    d3 = dict(A=dev(c3["A"], "bf16"), B=dev(c3["B"], "bf16"), C=dev(c3["C"], "bf16"),
              Y=torch.empty((8192, 8192), dtype=torch.bfloat16, device="cuda"))
    yield "gemm_bf16_8192", d3["Y"], lambda: om.gemm(d3["A"], d3["B"], d3["C"], 1.0, 1.0, 0, 1, d3["Y"])
    del d3
    c4 = synth.qlinear_i8_4096()
    keys = ("a", "a_scale", "a_zero_point", "b", "b_scale", "b_zero_point", "y_scale", "y_zero_point")
    d4 = {k: dev(c4[k]) for k in keys}
    y4 = torch.empty((4096, 4096), dtype=torch.int8, device="cuda")
    yield "qlinear_i8_4096", y4, lambda: om.qlinear_matmul(*(d4[k] for k in keys), y4)
    del d4
    c5 = synth.grouped_bf16_moe()
    d5 = dict(i=dev(c5["input"], "bf16"), w=dev(c5["weights"], "bf16"), x=dev(c5["group_indices"]),
              b=dev(c5["bias"], "bf16"), o=torch.empty((16384, 8, 2048), dtype=torch.bfloat16, device="cuda"))
    ws = torch.empty(om.grouped_matmul_workspace_size(16384, 8, 64), dtype=torch.uint8, device="cuda")
    yield "grouped_bf16_moe", d5["o"], lambda: om.grouped_matmul(d5["i"], d5["w"], d5["x"], d5["b"], d5["o"], ws)


def bits(t):
    """The tensor's bit patterns (NaN compares equal to itself)."""
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


def test_graph_replays_match_eager():
    for name, out, fn in workloads():
        fn()
        torch.cuda.synchronize()
        want = out.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for rep in range(3):
            out.fill_(0 if out.dtype == torch.int8 else float("nan"))  # eager work between the replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            same = torch.equal(bits(out), bits(want))
            assert same, (name, rep)
        del g, want
        torch.cuda.empty_cache()
