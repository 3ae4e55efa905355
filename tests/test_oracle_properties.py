"""Pins of the CPU oracle beyond the printed examples.

Each check compares the oracle with something other than itself: a library
routine (numpy / torch), a closed form, an algebraic identity or a Python
big-integer brute force, chosen so that a dropped term, a wrong sign or index,
a transposed operand or a wrong rounding rule fails at least one of them.
"""
import numpy as np
import pytest
import torch

import oracle
from onnx_matmul_family_amd import synth


# ---------------------------------------------------------------- decoders

def test_fp16_decoder_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_decoder_vs_torch():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 65536, size=4096).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite patterns
    got = oracle.decode(bits, "bf16")
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- MatMul

SHAPES = [
    ((5,), (5,)), ((3,), (3, 4)), ((4, 3), (3,)), ((2, 3, 4), (4, 5)), ((4, 5), (2, 5, 3)),
    ((2, 1, 3, 4), (5, 4, 2)), ((1, 6, 2), (3, 1, 2, 7)), ((7,), (2, 3, 7, 2)), ((2, 3, 4, 5), (5,)),
    ((0, 3), (3, 4)), ((2, 0), (0, 3)), ((3, 0, 2, 3), (1, 3, 2)), ((1, 1), (1, 1)),
]


@pytest.mark.parametrize("sa,sb", SHAPES)
def test_matmul_vs_numpy(sa, sb):
    rng = np.random.default_rng(hash((sa, sb)) % 2**32)
    A = rng.standard_normal(sa).astype(np.float32)
    B = rng.standard_normal(sb).astype(np.float32)
    y, t = oracle.matmul(A, B)
    ref = np.matmul(A.astype(np.float64), B.astype(np.float64))
    assert y.shape == ref.shape
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)
    tref = np.matmul(np.abs(A.astype(np.float64)), np.abs(B.astype(np.float64)))
    assert np.allclose(t, tref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("sa,sb", [((2, 3), (4, 5)), ((2, 2, 3), (3, 3, 4)), ((3,), (4,))])
def test_matmul_incompatible(sa, sb):
    with pytest.raises(oracle.OracleError):
        oracle.matmul(np.zeros(sa, np.float32), np.zeros(sb, np.float32))


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16", "f64"])
def test_matmul_identity_and_permutation(dt):
    rng = np.random.default_rng(5)
    A32 = rng.standard_normal((3, 7, 9)).astype(np.float32)
    A = synth.store(A32, dt)
    Aval = oracle.decode(A.ravel(), dt).reshape(A.shape)
    I = synth.store(np.eye(9, dtype=np.float32), dt)
    y, _ = oracle.matmul(A, I, dt=dt)
    assert np.array_equal(y, Aval)
    perm = rng.permutation(9)
    P = np.zeros((9, 9), np.float32)
    P[perm, np.arange(9)] = 1.0       # column j of A @ P is column perm[j] of A
    y, _ = oracle.matmul(A, synth.store(P, dt), dt=dt)
    assert np.array_equal(y, Aval[..., perm])


def test_matmul_batch_broadcast_structure():
    """Y[i, j] must equal A[i, 0] @ B[0, j] for A[I,1,m,k] x B[1,J,k,n]."""
    rng = np.random.default_rng(9)
    A = rng.standard_normal((3, 1, 4, 5)).astype(np.float32)
    B = rng.standard_normal((1, 2, 5, 6)).astype(np.float32)
    y, _ = oracle.matmul(A, B)
    for i in range(3):
        for j in range(2):
            yy, _ = oracle.matmul(A[i, 0], B[0, j])
            assert np.array_equal(y[i, j], yy)


def test_matmul_sampled_equals_full():
    rng = np.random.default_rng(3)
    A = synth.store(rng.standard_normal((2, 1, 17, 33)).astype(np.float32), "bf16")
    B = synth.store(rng.standard_normal((3, 33, 19)).astype(np.float32), "bf16")
    y, t = oracle.matmul(A, B, dt="bf16")
    sel = rng.integers(0, y.size, 50)
    ys, ts = oracle.matmul(A, B, dt="bf16", sel=sel)
    assert np.array_equal(ys, y.ravel()[sel]) and np.array_equal(ts, t.ravel()[sel])


# ---------------------------------------------------------------- Gemm

@pytest.mark.parametrize("tA,tB", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_gemm_transposes(tA, tB):
    rng = np.random.default_rng(17 + 2 * tA + tB)
    M, N, K = 5, 7, 3
    A = rng.standard_normal((K, M) if tA else (M, K)).astype(np.float32)
    B = rng.standard_normal((N, K) if tB else (K, N)).astype(np.float32)
    y, _ = oracle.gemm(A, B, None, 1.0, 0.0, tA, tB)
    Ap = A.T if tA else A
    Bp = B.T if tB else B
    ref = np.matmul(Ap.astype(np.float64), Bp.astype(np.float64))
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)
    # the same product with materialised transposes and no flags
    y2, _ = oracle.gemm(np.ascontiguousarray(Ap), np.ascontiguousarray(Bp), None, 1.0, 0.0, 0, 0)
    assert np.array_equal(y, y2)


@pytest.mark.parametrize("cshape", [(), (1,), (6,), (1, 6), (4, 1), (4, 6), (1, 1)])
def test_gemm_c_broadcast_forms(cshape):
    rng = np.random.default_rng(23)
    A = rng.standard_normal((4, 3)).astype(np.float32)
    B = rng.standard_normal((3, 6)).astype(np.float32)
    C = rng.standard_normal(cshape).astype(np.float32)
    y, _ = oracle.gemm(A, B, C, 0.75, -1.5)
    ref = 0.75 * (A.astype(np.float64) @ B.astype(np.float64)) + (-1.5) * np.broadcast_to(C.astype(np.float64), (4, 6))
    assert np.allclose(y, ref, rtol=1e-14, atol=1e-14)
    y2, _ = oracle.gemm(A, B, np.ascontiguousarray(np.broadcast_to(C, (4, 6))), 0.75, -1.5)
    assert np.array_equal(y, y2)


@pytest.mark.parametrize("cshape", [(4,), (3, 6), (6, 1), (2, 4, 6)])
def test_gemm_c_not_broadcastable(cshape):
    A = np.zeros((4, 3), np.float32)
    B = np.zeros((3, 6), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.gemm(A, B, np.zeros(cshape, np.float32))


def test_gemm_k_zero_gives_beta_c():
    A = np.zeros((3, 0), np.float32)
    B = np.zeros((0, 2), np.float32)
    C = np.array([1.0, -2.0], np.float32)
    y, _ = oracle.gemm(A, B, C, 2.0, 0.5)
    assert np.array_equal(y, np.tile([0.5, -1.0], (3, 1)))


# ---------------------------------------------------------------- QLinearMatMul

def q(a, asc, az, b, bsc, bz, ys, yz, **kw):
    return oracle.qlinear_matmul(a, np.float32(asc) if np.isscalar(asc) else asc,
                                 az, b, np.float32(bsc) if np.isscalar(bsc) else bsc, bz,
                                 np.array(ys, np.float32), yz, **kw)


@pytest.mark.parametrize("v,exp", [(1, 0), (3, 2), (5, 2), (7, 4), (-1, 0), (-3, -2), (-5, -2), (9, 4)])
def test_qlinear_round_half_even(v, exp):
    """x = v / 2 lands exactly on .5: rounding must go to the even neighbour."""
    i8 = lambda x: np.array(x, np.int8)
    y, acc = q(i8([[1]]), 1.0, i8(0), i8([[v]]), 1.0, i8(0), 2.0, i8(0))
    assert acc[0, 0] == v and y[0, 0] == exp


def test_qlinear_round_then_add_zero_point():
    i8 = lambda x: np.array(x, np.int8)
    # x = 2.5 -> 2 (even), + zp 3 -> 5; adding first (5.5) would round to 6
    y, _ = q(i8([[5]]), 1.0, i8(0), i8([[1]]), 1.0, i8(0), 2.0, i8(3))
    assert y[0, 0] == 5


@pytest.mark.parametrize("a_dt,b_dt,y_dt", [(np.int8, np.int8, np.int8), (np.uint8, np.int8, np.uint8),
                                            (np.int8, np.uint8, np.uint8), (np.uint8, np.uint8, np.int8)])
def test_qlinear_acc_brute_force(a_dt, b_dt, y_dt):
    rng = np.random.default_rng(31)
    M, K, N = 5, 37, 6
    info = lambda d: (np.iinfo(d).min, np.iinfo(d).max)
    a = rng.integers(*info(a_dt), size=(M, K), endpoint=True).astype(a_dt)
    b = rng.integers(*info(b_dt), size=(K, N), endpoint=True).astype(b_dt)
    az = rng.integers(*info(a_dt), size=(M, 1), endpoint=True).astype(a_dt)
    bz = rng.integers(*info(b_dt), size=(1, N), endpoint=True).astype(b_dt)
    asc = synth.uniform(rng, (M, 1), 0.002, 0.01)
    bsc = synth.uniform(rng, (1, N), 0.002, 0.01)
    y, acc = q(a, asc, az, b, bsc, bz, 0.05, np.array(3, y_dt))
    for m in range(M):
        for n in range(N):
            s = sum((int(a[m, k]) - int(az[m, 0])) * (int(b[k, n]) - int(bz[0, n])) for k in range(K))
            assert acc[m, n] == s
    # zero-point expansion, computed in int64 with numpy: sum ab - zb*Ra - za*Cb + K*za*zb
    a64, b64, za, zb = (x.astype(np.int64) for x in (a, b, az, bz))
    exp = a64 @ b64 - zb * a64.sum(1, keepdims=True) - za * b64.sum(0, keepdims=True) + K * za * zb
    assert np.array_equal(acc.astype(np.int64), exp)
    lo, hi = info(y_dt)
    assert y.dtype == y_dt and y.min() >= lo and y.max() <= hi


def test_qlinear_int32_wraparound():
    """Only the 32-bit accumulation may overflow: the accumulator wraps mod 2^32."""
    K = 40000
    a = np.full((1, K), -128, np.int8)
    b = np.full((K, 1), -128, np.int8)
    az, bz = np.array(127, np.int8), np.array(127, np.int8)
    y, acc = q(a, 1.0, az, b, 1.0, bz, 1.0, np.array(0, np.int8))
    true = 255 * 255 * K
    wrapped = (true + 2**31) % 2**32 - 2**31
    assert wrapped != true and acc[0, 0] == wrapped
    assert y[0, 0] == (-128 if wrapped < 0 else 127)


def test_qlinear_uint8_is_shifted_int8():
    """a_u8 = a_i8 + 128 with zp_u8 = zp_i8 + 128 leaves every (a - zp) unchanged."""
    rng = np.random.default_rng(41)
    a = rng.integers(-128, 128, (4, 9)).astype(np.int8)
    b = rng.integers(-128, 128, (9, 3)).astype(np.int8)
    az, bz = np.array(-7, np.int8), np.array(5, np.int8)
    to_u = lambda x: (x.astype(np.int16) + 128).astype(np.uint8)
    y1, acc1 = q(a, 0.01, az, b, 0.02, bz, 0.03, np.array(2, np.int8))
    y2, acc2 = q(to_u(a), 0.01, to_u(az), to_u(b), 0.02, to_u(bz), 0.03, np.array(2, np.int8))
    assert np.array_equal(acc1, acc2) and np.array_equal(y1, y2)


def test_qlinear_per_row_col_constant_equals_per_tensor():
    rng = np.random.default_rng(43)
    M, K, N = 6, 11, 5
    a = rng.integers(-128, 128, (M, K)).astype(np.int8)
    b = rng.integers(-128, 128, (K, N)).astype(np.int8)
    ref = q(a, 0.004, np.array(3, np.int8), b, 0.007, np.array(-2, np.int8), 0.05, np.array(1, np.int8))
    for ash, bsh in [((M,), (N,)), ((M, 1), (1, N))]:
        got = q(a, np.full(ash, 0.004, np.float32), np.full(ash, 3, np.int8),
                b, np.full(bsh, 0.007, np.float32), np.full(bsh, -2, np.int8), 0.05, np.array(1, np.int8))
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def test_qlinear_row_col_axes():
    """a's vector parameters index rows m, b's index columns n (a transposed axis fails)."""
    rng = np.random.default_rng(47)
    M, K, N = 4, 8, 3
    a = rng.integers(-128, 128, (M, K)).astype(np.int8)
    b = rng.integers(-128, 128, (K, N)).astype(np.int8)
    az = rng.integers(-16, 17, (M, 1)).astype(np.int8)
    bz = rng.integers(-16, 17, (1, N)).astype(np.int8)
    asc = synth.uniform(rng, (M, 1), 0.002, 0.01)
    bsc = synth.uniform(rng, (1, N), 0.002, 0.01)
    y, acc = q(a, asc, az, b, bsc, bz, 0.05, np.array(0, np.int8))
    for m in range(M):
        for n in range(N):
            ym, am = q(a[m:m + 1], asc[m, 0], az[m, 0], b[:, n:n + 1], bsc[0, n], bz[0, n], 0.05, np.array(0, np.int8))
            assert am[0, 0] == acc[m, n] and ym[0, 0] == y[m, n]


def test_qlinear_batched_params():
    """N-D per-row params [D, M, 1] and per-column [D, 1, N] follow the batch index."""
    rng = np.random.default_rng(53)
    D, M, K, N = 3, 4, 6, 5
    a = rng.integers(-128, 128, (D, M, K)).astype(np.int8)
    b = rng.integers(-128, 128, (D, K, N)).astype(np.int8)
    az = rng.integers(-16, 17, (D, M, 1)).astype(np.int8)
    bz = rng.integers(-16, 17, (D, 1, N)).astype(np.int8)
    asc = synth.uniform(rng, (D, M, 1), 0.002, 0.01)
    bsc = synth.uniform(rng, (D, 1, N), 0.002, 0.01)
    y, acc = q(a, asc, az, b, bsc, bz, 0.05, np.array(0, np.int8))
    for d in range(D):
        yd, ad = q(a[d], asc[d], az[d], b[d], bsc[d], bz[d], 0.05, np.array(0, np.int8))
        assert np.array_equal(yd, y[d]) and np.array_equal(ad, acc[d])


def test_qlinear_requant_order_fp32():
    """Requantisation follows mult = fp32(fp32(sa*sb)/sy), x = fp32(fp32(acc)*mult), then rint."""
    rng = np.random.default_rng(59)
    M, K, N = 64, 64, 64
    a = rng.integers(-128, 128, (M, K)).astype(np.int8)
    b = rng.integers(-128, 128, (K, N)).astype(np.int8)
    asc = synth.uniform(rng, (M, 1), 0.002, 0.01)
    bsc = synth.uniform(rng, (1, N), 0.002, 0.01)
    z8 = lambda s: np.zeros(s, np.int8)
    y, acc = q(a, asc, z8((M, 1)), b, bsc, z8((1, N)), 0.05, np.array(0, np.int8))
    mult = (asc * bsc) / np.float32(0.05)
    x = acc.astype(np.float32) * mult
    assert x.dtype == np.float32
    exp = np.clip(np.rint(x), -128, 127).astype(np.int8)
    assert np.array_equal(y, exp)


def _f32(x):
    """Round a rational to the nearest IEEE binary32 value, ties to even
    (normal range only: 24 significant bits, the unit of the last place is
    2^(e-23) for 2^e <= |x| < 2^(e+1))."""
    from fractions import Fraction
    if x == 0:
        return Fraction(0)
    s, ax = (-1 if x < 0 else 1), abs(x)
    e = ax.numerator.bit_length() - ax.denominator.bit_length()
    if Fraction(2) ** e > ax:
        e -= 1
    ulp = Fraction(2) ** (e - 23)
    return s * round(ax / ulp) * ulp  # round() of a Fraction is half-to-even


def _requant_exact(acc, sa, sb, sy, zy, lo, hi):
    """The requantisation reading in exact arithmetic: every step an exactly
    evaluated operation followed by one binary32 rounding."""
    from fractions import Fraction
    mult = _f32(_f32(Fraction(sa) * Fraction(sb)) / Fraction(sy))
    x = _f32(_f32(Fraction(acc)) * mult)
    return min(hi, max(lo, round(x) + zy))


def test_qlinear_requant_rounding_chain_near_ties():
    """Cases built so that the real-valued x sits within a few binary32 ulps of
    a half-integer: evaluating in double, or multiplying the scales in another
    order, changes the integer result on many of them.  The oracle must give
    the binary32 chain's answer on every case."""
    from fractions import Fraction
    rng = np.random.default_rng(97)
    i8 = lambda v: np.array(v, np.int8)
    n_real_differs = 0
    for _ in range(400):
        pa, pb = int(rng.integers(40, 128)), int(rng.integers(40, 128))
        acc = pa * pb
        sa, sb = np.float32(rng.uniform(0.002, 0.01)), np.float32(rng.uniform(0.002, 0.01))
        j = int(rng.integers(0, 100))
        sign = 1 if rng.random() < 0.5 else -1
        # y_scale that puts the real-valued |x| at j + 0.5
        sy = np.float32(float(Fraction(acc) * Fraction(float(sa)) * Fraction(float(sb)) / (Fraction(j) + Fraction(1, 2))))
        exp = _requant_exact(acc, float(sa), float(sb), float(sy), 0, -128, 127)
        real = Fraction(acc) * Fraction(float(sa)) * Fraction(float(sb)) / Fraction(float(sy))
        if min(127, max(-128, round(real))) != exp:
            n_real_differs += 1
        y, got_acc = q(i8([[pa]]), float(sa), i8(0), i8([[sign * pb]]), float(sb), i8(0), float(sy), i8(0))
        assert got_acc[0, 0] == sign * acc
        exp = _requant_exact(sign * acc, float(sa), float(sb), float(sy), 0, -128, 127)
        assert y[0, 0] == exp, (pa, pb, sa, sb, sy)
    assert n_real_differs > 20  # the cases really discriminate


def test_qlinear_scale_zp_shape_mismatch():
    a = np.zeros((2, 3), np.int8)
    b = np.zeros((3, 2), np.int8)
    with pytest.raises(oracle.OracleError):
        oracle.qlinear_matmul(a, np.ones((2,), np.float32), np.zeros((), np.int8), b,
                              np.float32(1), np.int8(0), np.float32(1), np.int8(0))


# ---------------------------------------------------------------- GroupedMatMul

def test_grouped_single_group_is_matmul_plus_bias():
    rng = np.random.default_rng(61)
    M, K, N = 7, 5, 4
    inp = rng.standard_normal((M, K)).astype(np.float32)
    w = rng.standard_normal((1, K, N)).astype(np.float32)
    bias = rng.standard_normal((1, N)).astype(np.float32)
    idx = np.zeros((M, 3), np.int32)
    y, _ = oracle.grouped_matmul(inp, w, idx, bias)
    ref = inp.astype(np.float64) @ w[0].astype(np.float64) + bias[0].astype(np.float64)
    for i in range(3):
        assert np.allclose(y[:, i], ref, rtol=1e-14, atol=1e-14)


def test_grouped_selection_permutation():
    rng = np.random.default_rng(67)
    M, K, N, G, S = 6, 5, 3, 4, 3
    inp = rng.standard_normal((M, K)).astype(np.float32)
    w = rng.standard_normal((G, K, N)).astype(np.float32)
    idx = synth.distinct_groups(rng, M, S, G, np.int64)
    y, _ = oracle.grouped_matmul(inp, w, idx)
    p = np.array([2, 0, 1])
    y2, _ = oracle.grouped_matmul(inp, w, np.ascontiguousarray(idx[:, p]))
    assert np.array_equal(y2, y[:, p])
    for m in range(M):
        for i in range(S):
            ref = inp[m].astype(np.float64) @ w[idx[m, i]].astype(np.float64)
            assert np.allclose(y[m, i], ref, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("bad", [-1, 4, 100])
def test_grouped_invalid_index(bad):
    inp = np.ones((2, 3), np.float32)
    w = np.ones((4, 3, 2), np.float32)
    idx = np.array([[0, bad], [1, 2]], np.int64)
    with pytest.raises(oracle.OracleError):
        oracle.grouped_matmul(inp, w, idx)


def test_grouped_sampled_equals_full():
    rng = np.random.default_rng(71)
    M, K, N, G, S = 9, 16, 10, 5, 2
    inp = synth.store(rng.standard_normal((M, K)).astype(np.float32), "bf16")
    w = synth.store(rng.standard_normal((G, K, N)).astype(np.float32), "bf16")
    bias = synth.store(rng.standard_normal((G, N)).astype(np.float32), "bf16")
    idx = synth.distinct_groups(rng, M, S, G)
    y, t = oracle.grouped_matmul(inp, w, idx, bias, dt="bf16")
    sel = rng.integers(0, y.size, 40)
    ys, ts = oracle.grouped_matmul(inp, w, idx, bias, dt="bf16", sel=sel)
    assert np.array_equal(ys, y.ravel()[sel]) and np.array_equal(ts, t.ravel()[sel])


def test_workload_generators_shapes():
    c1 = synth.gemm_f32_64x32x48()
    assert c1["A"].shape == (48, 64) and c1["B"].shape == (32, 48) and c1["C"].shape == (1, 32)
    y, _ = oracle.gemm(c1["A"], c1["B"], c1["C"], c1["alpha"], c1["beta"], 1, 1)
    assert y.shape == (64, 32)
    c2 = synth.matmul_bf16_bcast(scale=8)
    assert oracle.matmul_shape(c2["A"].shape, c2["B"].shape) == (8, 16, 64, 96)
    idx = synth.distinct_groups(np.random.default_rng(0), 100, 8, 64)
    assert all(len(set(r)) == 8 for r in idx.tolist()) and idx.min() >= 0 and idx.max() < 64
