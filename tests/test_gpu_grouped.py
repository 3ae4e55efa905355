"""GPU parity of GroupedMatMul against the CPU oracle (and the page's examples).

Covers bf16 / fp16 / fp32 / fp64, int32 and int64 indices, bias present and absent,
ragged M/N/K and group sizes (several tiles per group, unused and empty
groups), zero tokens / zero selections, and invalid indices (counted, their
rows untouched, everything else still correct)."""
import numpy as np
import pytest
import torch

import oracle
from onnx_matmul_family_amd import synth
from tests.gpu_util import check_close, check_routing, dev, host_f64, routing_from_workspace, run_heights

pytestmark = pytest.mark.gpu

om = pytest.importorskip("onnx_matmul_family_amd._omm")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    om.lib()


def run(inp, w, idx, bias, dt):
    out, ws = om.grouped_matmul(dev(inp, dt), dev(w, dt), dev(idx), dev(bias, dt) if bias is not None else None)
    bad = om.grouped_matmul_check(ws)
    return out, bad


def test_page_examples(golden):
    from tests.test_oracle_examples import _grouped_inputs
    for ex in golden("groupedmatmul"):
        for T in ex.get("T_values", [None]):
            for Tind in ex.get("Tind_values", [None]):
                inp, w, idx, bias = _grouped_inputs(ex, T, Tind)
                dt = {"float16": "f16", None: "f32", "float32": "f32", "float64": "f64"}[T]
                out, bad = run(inp, w, idx, bias, dt)
                y, t = oracle.grouped_matmul(inp, w, idx, bias)
                assert bad == 0 and tuple(out.shape) == y.shape, ex["cite"]
                check_close(host_f64(out), y, t, dt, ex["cite"])


def test_fp64_page_values_exact():
    """fp64 GroupedMatMul: integer-valued inputs give exact results."""
    x = torch.tensor([[1.0, 2.0], [3.0, -4.0]], dtype=torch.float64, device="cuda")
    w = torch.tensor([[[1.0, 0.0], [0.0, 1.0]], [[0.0, 1.0], [1.0, 0.0]]], dtype=torch.float64, device="cuda")
    i = torch.tensor([[1, 0], [0, 1]], dtype=torch.int64, device="cuda")
    out, ws = om.grouped_matmul(x, w, i)
    assert om.grouped_matmul_check(ws) == 0
    assert out.cpu().tolist() == [[[2.0, 1.0], [1.0, 2.0]], [[3.0, -4.0], [-4.0, 3.0]]]


CASES = [  # M, K, N, G, S
    (300, 136, 264, 7, 3), (1000, 512, 512, 16, 4), (64, 64, 64, 1, 1), (5, 8, 8, 40, 2), (513, 200, 300, 5, 5),
]


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32", "f64"])
@pytest.mark.parametrize("M,K,N,G,S", CASES)
@pytest.mark.parametrize("with_bias", [True, False])
def test_random(dt, M, K, N, G, S, with_bias):
    rng = np.random.default_rng(M + K + N + G + S + with_bias)
    inp = synth.store(synth.normal(rng, (M, K)), dt)
    w = synth.store(synth.normal(rng, (G, K, N), 0.05), dt)
    bias = synth.store(synth.uniform(rng, (G, N), -0.1, 0.1), dt) if with_bias else None
    idx = synth.distinct_groups(rng, M, min(S, G), G, np.int64 if M % 2 else np.int32)
    out, bad = run(inp, w, idx, bias, dt)
    y, t = oracle.grouped_matmul(inp, w, idx, bias, dt=dt)
    assert bad == 0
    check_close(host_f64(out), y, t, dt, "grouped %s M=%d K=%d N=%d G=%d S=%d" % (dt, M, K, N, G, S))


def test_skewed_groups_bf16():
    """One hot group with many tiles, several groups of one row, empty groups."""
    rng = np.random.default_rng(5)
    M, K, N, G, S = 1500, 256, 512, 12, 2
    inp = synth.store(synth.normal(rng, (M, K)), "bf16")
    w = synth.store(synth.normal(rng, (G, K, N), 0.05), "bf16")
    idx = np.zeros((M, S), np.int32)
    idx[:, 1] = 3
    idx[:4, 0] = [5, 6, 7, 11]
    out, bad = run(inp, w, idx, None, "bf16")
    y, t = oracle.grouped_matmul(inp, w, idx, None, dt="bf16")
    assert bad == 0
    check_close(host_f64(out), y, t, "bf16", "skewed groups")


# expected walk runs (row tiles per run, per group) of the routing in
# test_group_runs: a group of at most 12 row tiles is one run, a larger one
# balanced runs of at most 8
GROUP_RUNS = {256: {0: [8, 8], 1: [6, 7], 2: [4], 3: [12], 4: [4]},
              128: {0: [8, 8, 8, 8], 1: [6, 6, 6, 7], 2: [7], 3: [8, 8, 8], 4: [8]}}


@pytest.mark.parametrize("dt", ["bf16", "f32", "f64"])
def test_group_runs(dt):
    """Groups of 4000, 3200 and 3000 pairs beside smaller ones and an empty
    group: several walk runs per group (256-row tiles for bf16, 128-row
    tiles for fp32 / fp64); the routing's run table and every output checked."""
    rng = np.random.default_rng(21)
    M, K, N, G, S = 4000, 128, 512, 6, 3
    BM = 256 if dt == "bf16" else 128
    inp = synth.store(synth.normal(rng, (M, K)), dt)
    w = synth.store(synth.normal(rng, (G, K, N), 0.05), dt)
    bias = synth.store(synth.uniform(rng, (G, N), -0.1, 0.1), dt)
    idx = np.zeros((M, S), np.int32)
    idx[:3200, 1], idx[3200:, 1] = 1, 2
    idx[:3000, 2], idx[3000:, 2] = 3, 4
    idx = idx[rng.permutation(M)]
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "f64": torch.float64}[dt]
    out = torch.full((M, S, N), float("nan"), dtype=tdt, device="cuda")
    out, ws = om.grouped_matmul(dev(inp, dt), dev(w, dt), dev(idx), dev(bias, dt), output=out)
    assert om.grouped_matmul_check(ws) == 0
    bad, tiles, sorted_ids, raw = routing_from_workspace(ws, M, S, G, BM)
    assert bad == 0
    check_routing(idx, tiles, sorted_ids, G, BM, raw)
    assert run_heights(raw) == GROUP_RUNS[BM]
    y, t = oracle.grouped_matmul(inp, w, idx, bias, dt=dt)
    check_close(host_f64(out), y, t, dt, "group runs")


def test_invalid_indices_counted_rows_untouched():
    rng = np.random.default_rng(9)
    M, K, N, G, S = 50, 64, 96, 4, 2
    inp = synth.store(synth.normal(rng, (M, K)), "bf16")
    w = synth.store(synth.normal(rng, (G, K, N), 0.05), "bf16")
    idx = synth.distinct_groups(rng, M, S, G, np.int64)
    idx[3, 1] = -1
    idx[10, 0] = G
    idx[20, 1] = 1 << 40  # beyond int32: must not wrap into range
    sentinel = torch.full((M, S, N), 7.0, dtype=torch.bfloat16, device="cuda")
    out, ws = om.grouped_matmul(dev(inp, "bf16"), dev(w, "bf16"), dev(idx), None, output=sentinel)
    assert om.grouped_matmul_check(ws) == 3
    got = host_f64(out)
    for (m, i) in [(3, 1), (10, 0), (20, 1)]:
        assert (got[m, i] == 7.0).all()
    ok = np.ones((M, S), bool)
    ok[3, 1] = ok[10, 0] = ok[20, 1] = False
    idx_fixed = np.where(ok, idx, 0)
    y, t = oracle.grouped_matmul(inp, w, idx_fixed, None, dt="bf16")
    check_close(got[ok], y[ok], t[ok], "bf16", "valid rows next to invalid ones")


@pytest.mark.parametrize("M,S", [(0, 3), (4, 0), (0, 0)])
def test_empty(M, S):
    inp = torch.zeros((M, 16), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((3, 16, 8), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((M, S), dtype=torch.int64, device="cuda")
    out, ws = om.grouped_matmul(inp, w, idx)
    assert tuple(out.shape) == (M, S, 8)
    assert om.grouped_matmul_check(ws) == 0


def test_output_8_byte_aligned_full_column_tiles():
    """Whole 256-column tiles with an output that is 8- but not 16-byte aligned:
    the 4-value store epilogue instead of whole-row segments."""
    rng = np.random.default_rng(21)
    M, K, N, G, S = 300, 128, 512, 6, 2
    inp = synth.store(synth.normal(rng, (M, K)), "bf16")
    w = synth.store(synth.normal(rng, (G, K, N), 0.05), "bf16")
    bias = synth.store(synth.uniform(rng, (G, N), -0.1, 0.1), "bf16")
    idx = synth.distinct_groups(rng, M, S, G, np.int32)
    flat = torch.full((M * S * N + 8,), 3.0, dtype=torch.bfloat16, device="cuda")
    out = flat[4:4 + M * S * N].view(M, S, N)
    assert out.data_ptr() % 16 == 8
    _, ws = om.grouped_matmul(dev(inp, "bf16"), dev(w, "bf16"), dev(idx), dev(bias, "bf16"), output=out)
    assert om.grouped_matmul_check(ws) == 0
    y, t = oracle.grouped_matmul(inp, w, idx, bias, dt="bf16")
    check_close(host_f64(out), y, t, "bf16", "grouped, 8-byte aligned output")
    assert (flat[:4].float() == 3.0).all() and (flat[-4:].float() == 3.0).all()


def test_output_beyond_2gib_sampled():
    """An output of 2 GiB (row byte offsets no longer fit the 32-bit buffer
    offsets of the whole-tile epilogue): rows are stored through row pointers."""
    rng = np.random.default_rng(22)
    M, K, N, G, S = 65536, 64, 2048, 8, 8
    inp = synth.store(synth.normal(rng, (M, K)), "bf16")
    w = synth.store(synth.normal(rng, (G, K, N), 0.05), "bf16")
    bias = synth.store(synth.uniform(rng, (G, N), -0.1, 0.1), "bf16")
    idx = synth.distinct_groups(rng, M, S, G, np.int32)
    out = torch.full((M, S, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    assert out.numel() * 2 >= 1 << 31
    _, ws = om.grouped_matmul(dev(inp, "bf16"), dev(w, "bf16"), dev(idx), dev(bias, "bf16"), output=out)
    assert om.grouped_matmul_check(ws) == 0
    rows = rng.choice(M * S, size=64, replace=False)
    got = out.view(M * S, N)[torch.from_numpy(rows).cuda()]
    assert torch.isfinite(got.float()).all()
    sel = (rows[:, None] * N + np.arange(N)[None, :]).reshape(-1)
    y, t = oracle.grouped_matmul(inp, w, idx, bias, dt="bf16", sel=sel)
    check_close(host_f64(got).reshape(-1), y, t, "bf16", "grouped, 2 GiB output, sampled rows")
    del out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dt", ["f32", "f64"])
def test_fp_matrix_core_workload_full(dt):
    """fp32 / fp64 on the matrix cores at the size the benchmark times
    (4096 tokens x 4 of 16 experts, K = N = 1024): the routing into 128-row
    tiles checked as a counting sort, every output element against the oracle."""
    c = synth.grouped_fp_moe(dt)
    M, S = c["group_indices"].shape
    G, K, N = c["weights"].shape
    tdt = torch.float64 if dt == "f64" else torch.float32
    out = torch.full((M, S, N), float("nan"), dtype=tdt, device="cuda")
    out, ws = om.grouped_matmul(dev(c["input"]), dev(c["weights"]), dev(c["group_indices"]), dev(c["bias"]),
                                output=out)
    bad, tiles, sorted_ids, raw = routing_from_workspace(ws, M, S, G, 128)
    assert bad == 0
    check_routing(c["group_indices"], tiles, sorted_ids, G, 128, raw)
    y, t = oracle.grouped_matmul(c["input"], c["weights"], c["group_indices"], c["bias"])
    check_close(host_f64(out), y, t, dt, "grouped %s %dx%d, K=%d N=%d G=%d" % (dt, M, S, K, N, G))


@pytest.mark.parametrize("dt", ["f32", "f64"])
def test_fp_small_integers_exact(dt):
    """Integer inputs in {-2..2} and an integer bias (|sums| far below 2^24):
    every fp32 / fp64 partial sum is exact, so the results must be bit-exact.
    Ragged K (K % 16 != 0), N (two 128-column tiles, the second partial) and a
    hot group of several 128-row tiles next to one-row groups."""
    rng = np.random.default_rng(31)
    M, K, N, G, S = 700, 203, 200, 9, 2
    inp = synth.store(synth.small_ints(rng, (M, K)), dt)
    w = synth.store(synth.small_ints(rng, (G, K, N)), dt)
    bias = synth.store(synth.small_ints(rng, (G, N), -8, 8), dt)
    idx = np.zeros((M, S), np.int64)
    idx[:, 1] = 4
    idx[:3, 0] = [1, 7, 8]
    out, bad = run(inp, w, idx, bias, dt)
    assert bad == 0
    y, _ = oracle.grouped_matmul(inp, w, idx, bias)
    assert np.array_equal(host_f64(out), y)


@pytest.mark.parametrize("dt", ["f32", "f64"])
def test_fp_invalid_indices_counted_rows_untouched(dt):
    rng = np.random.default_rng(33)
    M, K, N, G, S = 300, 64, 150, 5, 2
    inp = synth.store(synth.normal(rng, (M, K)), dt)
    w = synth.store(synth.normal(rng, (G, K, N), 0.05), dt)
    idx = synth.distinct_groups(rng, M, S, G, np.int64)
    idx[7, 0] = -3
    idx[200, 1] = G
    sentinel = torch.full((M, S, N), 7.0, dtype=torch.float64 if dt == "f64" else torch.float32, device="cuda")
    out, ws = om.grouped_matmul(dev(inp), dev(w), dev(idx), None, output=sentinel)
    assert om.grouped_matmul_check(ws) == 2
    got = host_f64(out)
    assert (got[7, 0] == 7.0).all() and (got[200, 1] == 7.0).all()
    ok = np.ones((M, S), bool)
    ok[7, 0] = ok[200, 1] = False
    y, t = oracle.grouped_matmul(inp, w, np.where(ok, idx, 0), None)
    check_close(got[ok], y[ok], t[ok], dt, "fp grouped next to invalid indices")
