"""Pins of the oracle's GroupedMatMul over DequantizeLinear weights (CPU only).

The GroupedMatMul page names the composition "DequantizeLinear of quantised
weights, fed to GroupedMatMul" without printing an example, so the pins are:
the oracle's rounding against numpy's / torch's IEEE conversions, worked
examples whose values follow by hand from (q - zero_point) * scale, a block
layout case where a wrong block index changes the result, the rounding of the
dequantised weight to the scale's type, and brute force on small inputs with
library rounding and a library matmul.
"""
import numpy as np
import pytest
import torch

import oracle
from onnx_matmul_family_amd import synth


def bf16(x):
    return synth.bf16_bits(np.asarray(x, dtype=np.float32))


# ---- rounding to the storage types ------------------------------------------

def _draws(rng, n):
    mant = rng.uniform(-2.0, 2.0, n)
    exps = rng.integers(-30, 30, n)
    return np.ldexp(mant, exps)


def test_round_f16_matches_numpy():
    rng = np.random.default_rng(10)
    v = np.concatenate([_draws(rng, 3000), np.ldexp(rng.uniform(-1, 1, 500), -14),  # subnormal range
                        rng.uniform(65000, 66000, 300) * rng.choice([-1, 1], 300),   # overflow boundary
                        [65504.0, 65519.99, 65520.0, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -25, 3 * 2.0 ** -26]])
    got = oracle.round_to(v, "f16")
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal(got, ref)


def test_round_f32_matches_numpy():
    rng = np.random.default_rng(11)
    v = np.concatenate([_draws(rng, 3000), np.ldexp(rng.uniform(-1, 1, 300), -126),
                        [1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, 2.0 ** -150, 3 * 2.0 ** -150]])
    np.testing.assert_array_equal(oracle.round_to(v, "f32"), v.astype(np.float32).astype(np.float64))


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(12)
    v32 = np.concatenate([_draws(rng, 3000), np.ldexp(rng.uniform(-1, 1, 300), -126),
                          [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 3.3895313892515355e38]]).astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_to(v32.astype(np.float64), "bf16"), ref)


def test_round_ties_to_even():
    # bf16 keeps 8 significant bits: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert oracle.round_to([1 + 2.0 ** -8], "bf16")[0] == 1.0
    assert oracle.round_to([1 + 3 * 2.0 ** -8], "bf16")[0] == 1 + 2.0 ** -6
    assert oracle.round_to([-(1 + 2.0 ** -8)], "bf16")[0] == -1.0
    assert np.isinf(oracle.round_to([70000.0], "f16")[0])


# ---- worked examples ----------------------------------------------------------

def _example(dt):
    f = (lambda x: bf16(x)) if dt == "bf16" else (lambda x: np.asarray(x, dtype=np.float32 if dt == "f32" else np.float16))
    inp = f([[1.0, 2.0]])
    q = np.array([[[3, -1], [0, 5]], [[-128, 127], [10, 20]]], dtype=np.int8)
    scale = f([[[0.5, 2.0], [1.0, 0.25]], [[1.0, 1.0], [0.5, 0.5]]])
    zp = np.array([[[1, 0], [0, 1]], [[0, 0], [10, 0]]], dtype=np.int8)
    idx = np.array([[1, 0]], dtype=np.int32)
    bias = f([[0.5, 0.0], [0.0, -1.0]])
    return inp, q, scale, zp, idx, bias


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_worked_example(dt):
    inp, q, scale, zp, idx, bias = _example(dt)
    # group 0: w = [[(3-1)*.5, (-1-0)*2], [(0-0)*1, (5-1)*.25]] = [[1, -2], [0, 1]]
    # group 1: w = [[-128, 127], [(10-10)*.5, 20*.5]] = [[-128, 127], [0, 10]]
    # token [1, 2]: selection 0 (group 1) -> [-128, 147] + [0, -1]; selection 1 (group 0) -> [1, 0] + [.5, 0]
    y, t = oracle.grouped_matmul_dequant(inp, q, scale, zp, 1, idx, bias, dt=dt)
    np.testing.assert_array_equal(y, [[[-128.0, 146.0], [1.5, 0.0]]])
    np.testing.assert_array_equal(t, [[[128.0, 147.0], [1.0, 4.0]]])
    y0, _ = oracle.grouped_matmul_dequant(inp, q, scale, zp, 1, idx, None, dt=dt)
    np.testing.assert_array_equal(y0, [[[-128.0, 147.0], [1.0, 0.0]]])
    # no zero point: group 0 w = [[1.5, -2], [0, 1.25]], group 1 w = [[-128, 127], [5, 10]]
    y1, _ = oracle.grouped_matmul_dequant(inp, q, scale, None, 1, idx, None, dt=dt)
    np.testing.assert_array_equal(y1, [[[-118.0, 147.0], [1.5, 0.5]]])


def test_uint8_example():
    inp = bf16([[1.0, 1.0, 1.0]])
    q = np.array([[[200], [0], [255]]], dtype=np.uint8)
    scale = bf16([[[0.25]]])
    zp = np.array([[[100]]], dtype=np.uint8)
    # one block of 3 (block_size 4 > K): (200-100)/4 + (0-100)/4 + (255-100)/4 = 25 - 25 + 38.75
    y, _ = oracle.grouped_matmul_dequant(inp, q, scale, zp, 4, np.zeros((1, 1), np.int64), None, dt="bf16")
    assert y[0, 0, 0] == 38.75


def test_block_index_along_k():
    # K = 4, block_size 2: k = 0, 1 use block 0 (scale 1), k = 2, 3 block 1 (scale 10)
    inp = bf16([[1.0, 2.0, 3.0, 4.0]])
    q = np.ones((1, 4, 1), np.int8)
    scale = bf16([[[1.0], [10.0]]])
    y, _ = oracle.grouped_matmul_dequant(inp, q, scale, None, 2, np.zeros((1, 1), np.int32), None, dt="bf16")
    assert y[0, 0, 0] == 1 + 2 + 30 + 40  # k % bs indexing would give 64
    # a ragged last block: K = 5, block_size 2 -> blocks {0,1}, {2,3}, {4}
    inp5 = bf16([[1.0, 1.0, 1.0, 1.0, 1.0]])
    q5 = np.ones((1, 5, 1), np.int8)
    s5 = bf16([[[1.0], [2.0], [4.0]]])
    y5, _ = oracle.grouped_matmul_dequant(inp5, q5, s5, None, 2, np.zeros((1, 1), np.int32), None, dt="bf16")
    assert y5[0, 0, 0] == 1 + 1 + 2 + 2 + 4


def test_scale_per_column_and_group():
    inp = bf16([[1.0]])
    q = np.full((2, 1, 3), 2, np.int8)
    scale = bf16([[[1.0, 2.0, 4.0]], [[8.0, 16.0, 32.0]]])
    idx = np.array([[1, 0]], np.int32)
    y, _ = oracle.grouped_matmul_dequant(inp, q, scale, None, 1, idx, None, dt="bf16")
    np.testing.assert_array_equal(y, [[[16.0, 32.0, 64.0], [2.0, 4.0, 8.0]]])


def test_dequantised_weight_is_rounded_to_the_scale_type():
    # (127 - (-128)) * 1.0078125 = 256.9921875; bf16 spacing at 256 is 2 -> 256
    inp = bf16([[1.0]])
    q = np.array([[[127]]], np.int8)
    zp = np.array([[[-128]]], np.int8)
    y, _ = oracle.grouped_matmul_dequant(inp, q, bf16([[[1.0078125]]]), zp, 1, np.zeros((1, 1), np.int32),
                                         None, dt="bf16")
    assert y[0, 0, 0] == 256.0
    # fp16 keeps it (11 bits: spacing 0.25 at 256) -> 257 after rounding 256.9921875
    y16, _ = oracle.grouped_matmul_dequant(np.array([[1.0]], np.float16), q, np.array([[[1.0078125]]], np.float16),
                                           zp, 1, np.zeros((1, 1), np.int32), None)
    assert y16[0, 0, 0] == 257.0


def test_invalid_index_is_reported():
    inp = bf16([[1.0]])
    q = np.ones((2, 1, 1), np.int8)
    with pytest.raises(oracle.OracleError):
        oracle.grouped_matmul_dequant(inp, q, bf16(np.ones((2, 1, 1))), None, 1, np.array([[2]], np.int32), None,
                                      dt="bf16")


# ---- brute force with library rounding ----------------------------------------

@pytest.mark.parametrize("dt,qdt,bs,with_zp", [("bf16", np.int8, 3, True), ("f16", np.uint8, 4, True),
                                                ("f32", np.int8, 7, False), ("bf16", np.uint8, 16, False)])
def test_brute_force_small(dt, qdt, bs, with_zp):
    rng = np.random.default_rng(20 + bs)
    M, K, N, G, S = 5, 13, 6, 3, 2
    lo, hi = (-128, 127) if qdt == np.int8 else (0, 255)
    q = rng.integers(lo, hi + 1, (G, K, N)).astype(qdt)
    nkb = -(-K // bs)
    zp = rng.integers(lo, hi + 1, (G, nkb, N)).astype(qdt) if with_zp else None
    s32 = rng.uniform(0.001, 0.02, (G, nkb, N)).astype(np.float32)
    x32 = rng.standard_normal((M, K)).astype(np.float32)
    b32 = rng.uniform(-0.1, 0.1, (G, N)).astype(np.float32)
    idx = synth.distinct_groups(rng, M, S, G)
    if dt == "bf16":
        to = lambda a: bf16(a)
        back = lambda a: synth.bf16_to_f32(a).astype(np.float64)
        rnd = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    else:
        npt = np.float16 if dt == "f16" else np.float32
        to = lambda a: a.astype(npt)
        back = lambda a: a.astype(np.float64)
        rnd = lambda a: a.astype(npt).astype(np.float64)
    x, s, b = to(x32), to(s32), to(b32)
    kb = np.arange(K) // bs
    zz = zp.astype(np.float64)[:, kb, :] if with_zp else 0.0
    # (q - zp) * s is exact in fp64 and in fp32; one library rounding to the type
    w = rnd((q.astype(np.float64) - zz) * back(s)[:, kb, :])
    ref = np.einsum("mk,mskn->msn", back(x), w[idx])
    ref += back(b)[idx]
    y, t = oracle.grouped_matmul_dequant(x, q, s, zp, bs, idx, b, dt=dt if dt == "bf16" else None)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(t, np.einsum("mk,mskn->msn", np.abs(back(x)), np.abs(w[idx])), rtol=1e-12)
