"""GPU parity of GroupedMatMul over DequantizeLinear weights against the CPU oracle.

Covers bf16 / fp16 / fp32, int8 and uint8 weights, zero points present and
absent, the three 16-bit kernels (int8 weight tile by DMA and dequantised
after the transposing LDS read; weights register-staged and dequantised
before the LDS store; element-wise for other block sizes and layouts), one block per group and column (block_size >= K), ragged M / N / K,
the rounding of each dequantised weight to T, exact small-integer results,
invalid indices, and the full-size workload on sampled outputs."""
import numpy as np
import pytest
import torch

import oracle
from onnx_matmul_family_amd import synth
from tests.gpu_util import (check_close, check_routing, dev, host_f64, routing_from_workspace, run_heights,
                            sample_indices, tile_row_pairs)

pytestmark = pytest.mark.gpu

om = pytest.importorskip("onnx_matmul_family_amd._omm")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    om.lib()


def run(inp, q, scale, zp, bs, idx, bias, dt):
    out, ws = om.grouped_matmul_dequant(dev(inp, dt), dev(q), dev(scale, dt), dev(zp) if zp is not None else None,
                                        bs, dev(idx), dev(bias, dt) if bias is not None else None)
    return out, om.grouped_matmul_check(ws)


def make(rng, M, K, N, G, S, bs, qdt, with_zp, dt, with_bias=True, srange=(0.002, 0.02)):
    lo, hi = (-128, 127) if qdt == np.int8 else (0, 255)
    nkb = -(-K // bs)
    q = rng.integers(lo, hi + 1, (G, K, N)).astype(qdt)
    zp = rng.integers(lo, hi + 1, (G, nkb, N)).astype(qdt) if with_zp else None
    scale = synth.store(synth.uniform(rng, (G, nkb, N), *srange), dt)
    inp = synth.store(synth.normal(rng, (M, K)), dt)
    bias = synth.store(synth.uniform(rng, (G, N), -0.1, 0.1), dt) if with_bias else None
    idx = synth.distinct_groups(rng, M, min(S, G), G, np.int64 if M % 2 else np.int32)
    return inp, q, scale, zp, idx, bias


CASES = [  # M, K, N, G, S, block_size
    (300, 256, 272, 7, 3, 128),    # weights by DMA; ragged last column tile
    (300, 256, 264, 7, 3, 128),    # register-staged fast path (N % 16 != 0); ragged last column tile
    (1000, 512, 512, 16, 4, 64),   # weights by DMA; several row tiles per group
    (150, 200, 256, 5, 2, 64),     # register-staged fast path; K tail inside the last stage
    (257, 192, 256, 3, 2, 192),    # weights by DMA; one block per group and column (block_size == K), odd stage count
    (513, 200, 300, 5, 5, 40),     # element-wise: block 40, N % 8 != 0
    (64, 136, 64, 1, 1, 136),      # element-wise: one block, block % 64 != 0
    (100, 100, 72, 4, 2, 1000),    # element-wise: block_size > K
    (40, 96, 40, 3, 3, 32),        # element-wise: block 32
]


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("M,K,N,G,S,bs", CASES)
@pytest.mark.parametrize("qdt,with_zp", [(np.int8, True), (np.uint8, True), (np.int8, False)])
def test_random(dt, M, K, N, G, S, bs, qdt, with_zp):
    rng = np.random.default_rng(M + K + N + G + S + bs + (qdt == np.uint8) + 2 * with_zp)
    inp, q, scale, zp, idx, bias = make(rng, M, K, N, G, S, bs, qdt, with_zp, dt, with_bias=(M % 3 != 0))
    out, bad = run(inp, q, scale, zp, bs, idx, bias, dt)
    y, t = oracle.grouped_matmul_dequant(inp, q, scale, zp, bs, idx, bias, dt=dt)
    assert bad == 0
    check_close(host_f64(out), y, t, dt, "grouped dq %s q=%s zp=%s M=%d K=%d N=%d G=%d S=%d bs=%d"
                % (dt, np.dtype(qdt).name, with_zp, M, K, N, G, S, bs))


@pytest.mark.parametrize("bs", [64, 32])
@pytest.mark.parametrize("qdt", [np.int8, np.uint8])
def test_exact_small_integers_f16(bs, qdt):
    """Every weight, product and partial sum is exact in fp32 and the result in
    fp16, so the GPU result must equal the oracle's bit for bit."""
    rng = np.random.default_rng(7 + bs)
    M, K, N, G, S = 300, 128, 256, 3, 2
    base = 0 if qdt == np.int8 else 100
    q = (rng.integers(-3, 4, (G, K, N)) + base).astype(qdt)
    zp = (rng.integers(-1, 2, (G, K // bs, N)) + base).astype(qdt)
    scale = rng.choice([0.5, 1.0, 2.0], (G, K // bs, N)).astype(np.float16)
    inp = rng.integers(-1, 2, (M, K)).astype(np.float16)
    bias = rng.integers(-4, 5, (G, N)).astype(np.float16)
    idx = synth.distinct_groups(rng, M, S, G)
    out, bad = run(inp, q, scale, zp, bs, idx, bias, "f16")
    y, _ = oracle.grouped_matmul_dequant(inp, q, scale, zp, bs, idx, bias)
    assert bad == 0
    np.testing.assert_array_equal(host_f64(out), y)


@pytest.mark.parametrize("bs", [64, 1])
def test_dequantised_weight_rounded_to_bf16(bs):
    """(127 + 128) * 1.0078125 = 256.9921875 is held in bf16 as 256; a second
    weight that is exact makes the difference visible in the sum."""
    K, N = 64, 16  # bs 64: the weights-by-DMA kernel; bs 1: the element-wise path
    nkb = K // bs
    q = np.zeros((1, K, N), np.int8)
    zp = np.zeros((1, nkb, N), np.int8)
    scale = np.ones((1, nkb, N), np.float32)
    inp = np.zeros((1, K), np.float32)
    q[0, 0], zp[0, 0], scale[0, 0], inp[0, 0] = 127, -128, 1.0078125, 1.0   # w0 = 256 (256.99 unrounded)
    if bs == 1:
        q[0, 1], scale[0, 1], inp[0, 1] = -128, 2.0, 1.0                   # w1 = -256: sum 0 (0.99 unrounded)
        want = 0.0
    else:
        q[0, 1], inp[0, 1] = 0, -2.0    # same block: w1 = 128 * 1.0078125 = 129 exactly: sum -2 (-1.0078 unrounded)
        want = -2.0
    x, sc = synth.bf16_bits(inp), synth.bf16_bits(scale)
    idx = np.zeros((1, 1), np.int32)
    out, bad = run(x, q, sc, zp, bs, idx, None, "bf16")
    y, _ = oracle.grouped_matmul_dequant(x, q, sc, zp, bs, idx, None, dt="bf16")
    assert bad == 0
    assert np.all(y == want)
    np.testing.assert_array_equal(host_f64(out), y)


def test_invalid_indices_counted_rows_untouched():
    rng = np.random.default_rng(3)
    M, K, N, G, S, bs = 200, 128, 256, 4, 2, 64
    inp, q, scale, zp, idx, bias = make(rng, M, K, N, G, S, bs, np.int8, True, "bf16")
    idx = idx.astype(np.int32)
    idx[5, 1] = G
    idx[17, 0] = -1
    out = torch.full((M, S, N), 7.0, dtype=torch.bfloat16, device="cuda")
    out, ws = om.grouped_matmul_dequant(dev(inp, "bf16"), dev(q), dev(scale, "bf16"), dev(zp), bs, dev(idx),
                                        dev(bias, "bf16"), output=out)
    assert om.grouped_matmul_check(ws) == 2
    got = host_f64(out)
    assert np.all(got[5, 1] == 7.0) and np.all(got[17, 0] == 7.0)
    ok = np.ones((M, S), bool)
    ok[5, 1] = ok[17, 0] = False
    idx_ok = np.where(ok, idx, 0)
    y, t = oracle.grouped_matmul_dequant(inp, q, scale, zp, bs, idx_ok, bias, dt="bf16")
    check_close(got[ok], y[ok], t[ok], "bf16", "valid rows")


def test_empty_shapes():
    inp = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((2, 64, 16), dtype=torch.int8, device="cuda")
    sc = torch.ones((2, 1, 16), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((0, 2), dtype=torch.int32, device="cuda")
    out, _ = om.grouped_matmul_dequant(inp, q, sc, None, 64, idx)
    assert tuple(out.shape) == (0, 2, 16)
    # K = 0: no blocks; the result is the bias
    inp0 = torch.zeros((3, 0), dtype=torch.bfloat16, device="cuda")
    q0 = torch.zeros((2, 0, 16), dtype=torch.int8, device="cuda")
    sc0 = torch.ones((2, 0, 16), dtype=torch.bfloat16, device="cuda")
    b = torch.arange(32, dtype=torch.float32, device="cuda").reshape(2, 16).bfloat16()
    idx0 = torch.tensor([[1], [0], [1]], dtype=torch.int32, device="cuda")
    out0, _ = om.grouped_matmul_dequant(inp0, q0, sc0, None, 64, idx0, b)
    torch.cuda.synchronize()
    assert torch.equal(out0[:, 0].float(), b[idx0[:, 0].long()].float())


@pytest.mark.parametrize("qdt", [np.int8, np.uint8])
def test_f32_matrix_core_multi_tile(qdt):
    """fp32 over int8 / uint8 weights on the matrix cores: several 128-row tiles
    per group, ragged N and K, block 96 (not a multiple of the 16-deep stage),
    zero points present: every element against the oracle."""
    rng = np.random.default_rng(41)
    M, K, N, G, S, bs = 900, 300, 260, 6, 3, 96
    nkb = -(-K // bs)
    inp = synth.store(synth.normal(rng, (M, K)), "f32")
    lo, hi = (-128, 127) if qdt == np.int8 else (0, 255)
    q = rng.integers(lo, hi + 1, (G, K, N)).astype(qdt)
    sc = synth.uniform(rng, (G, nkb, N), 1e-3, 3e-3)
    zp = rng.integers(-8 if qdt == np.int8 else 120, 9 if qdt == np.int8 else 137, (G, nkb, N)).astype(qdt)
    bias = synth.uniform(rng, (G, N), -0.1, 0.1)
    idx = synth.distinct_groups(rng, M, S, G, np.int32)
    out, bad = run(inp, q, sc, zp, bs, idx, bias, "f32")
    assert bad == 0
    y, t = oracle.grouped_matmul_dequant(inp, q, sc, zp, bs, idx, bias, dt="f32")
    check_close(host_f64(out), y, t, "f32", "grouped dq f32 multi-tile")


@pytest.mark.parametrize("dt,N", [("bf16", 512), ("bf16", 264), ("f32", 512)])
def test_group_runs(dt, N):
    """Groups of 4000 and 3200 pairs beside one of 800: several walk runs per
    group on the weights-by-DMA kernel (N = 512), the register-staged one
    (N = 264) and the fp32 kernel (128-row tiles); run table and every output."""
    rng = np.random.default_rng(33)
    M, K, G, S, bs = 4000, 128, 3, 2, 64
    inp, q, scale, zp, _, bias = make(rng, M, K, N, G, S, bs, np.int8, True, dt)
    idx = np.zeros((M, S), np.int32)
    idx[:, 1] = np.where(np.arange(M) < 3200, 1, 2)
    idx = idx[rng.permutation(M)]
    BM = 128 if dt == "f32" else 256
    out, ws = om.grouped_matmul_dequant(dev(inp, dt), dev(q), dev(scale, dt), dev(zp), bs, dev(idx), dev(bias, dt))
    assert om.grouped_matmul_check(ws) == 0
    bad, tiles, sorted_ids, raw = routing_from_workspace(ws, M, S, G, BM)
    check_routing(idx, tiles, sorted_ids, G, BM, raw)
    assert run_heights(raw) == ({0: [8, 8], 1: [6, 7], 2: [4]} if BM == 256 else
                                {0: [8, 8, 8, 8], 1: [6, 6, 6, 7], 2: [7]})
    y, t = oracle.grouped_matmul_dequant(inp, q, scale, zp, bs, idx, bias, dt=dt)
    check_close(host_f64(out), y, t, dt, "quantised experts, group runs")


def test_full_size_workload_tile_rows():
    """The benchmark's quantised-experts workload at full size: the routing
    checked as a counting sort, two complete output rows of every routed tile
    (over every row slot of a tile) and 4000 sampled elements."""
    c = synth.grouped_dq_int8_moe()
    M, S = c["group_indices"].shape
    G, K, N = c["qweights"].shape
    out = torch.full((M, S, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    out, ws = om.grouped_matmul_dequant(dev(c["input"], "bf16"), dev(c["qweights"]), dev(c["scale"], "bf16"),
                                        dev(c["zero_point"]), c["block_size"], dev(c["group_indices"]),
                                        dev(c["bias"], "bf16"), output=out)
    assert om.grouped_matmul_check(ws) == 0
    bad, tiles, sorted_ids, raw = routing_from_workspace(ws, M, S, G, 256)
    assert bad == 0
    check_routing(c["group_indices"], tiles, sorted_ids, G, 256, raw)
    pairs = tile_row_pairs(tiles, sorted_ids, 2, 256)
    sel = np.concatenate([(pairs[:, None] * N + np.arange(N, dtype=np.int64)[None, :]).ravel(),
                          sample_indices(M * S * N, 4000, 11)])
    y, t = oracle.grouped_matmul_dequant(c["input"], c["qweights"], c["scale"], c["zero_point"], c["block_size"],
                                         c["group_indices"], c["bias"], dt="bf16", sel=sel)
    got = host_f64(out.reshape(-1)[torch.from_numpy(sel).cuda()])
    check_close(got, y, t, "bf16", "grouped dq full size: %d whole rows + samples" % len(pairs))
    assert torch.isfinite(out.float()).all()
