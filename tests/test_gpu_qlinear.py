"""GPU parity of QLinearMatMul against the CPU oracle: bit-exact int8/uint8 outputs.

Covers the pages' printed examples, every int8/uint8 combination of a, b and y,
per-tensor / per-row / per-column parameters (1-D and N-D forms), batched
operands, ragged tiles, the element-wise path for unaligned extents,
constructed round-half-even ties, saturation and 32-bit wraparound."""
import numpy as np
import pytest
import torch

import oracle
from onnx_matmul_family_amd import synth
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

om = pytest.importorskip("onnx_matmul_family_amd._omm")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    om.lib()


def run(a, asc, az, b, bsc, bz, ys, yz):
    # fp16 scales go to the library as fp16; anything else as fp32
    f16 = np.asarray(asc).dtype == np.float16
    asc, bsc, ys = (np.asarray(x, np.float16 if f16 else np.float32) for x in (asc, bsc, ys))
    y = om.qlinear_matmul(dev(a), dev(asc), dev(az), dev(b), dev(bsc), dev(bz), dev(ys), dev(yz))
    torch.cuda.synchronize()
    ref, _ = oracle.qlinear_matmul(a, asc, az, b, bsc, bz, ys, yz)
    return y.cpu().numpy(), ref


def test_printed_examples(golden):
    """Every printed example, its scales passed as printed (fp32 or fp16)."""
    from tests.test_oracle_examples import arr
    seen = set()
    for ex in golden("qlinearmatmul"):
        i = ex["inputs"]
        sc = lambda k: arr(i[k])
        seen.add(sc("a_scale").dtype)
        got, ref = run(arr(i["a"]), sc("a_scale"), arr(i["a_zero_point"]), arr(i["b"]), sc("b_scale"),
                       arr(i["b_zero_point"]), sc("y_scale"), arr(i["y_zero_point"]))
        exp = arr(ex["outputs"]["y"])
        assert np.array_equal(got, exp), (ex["cite"], got, exp)
        assert np.array_equal(got, ref), ex["cite"]
    assert np.dtype(np.float16) in seen and np.dtype(np.float32) in seen


@pytest.mark.parametrize("M,K,N", [(300, 272, 208), (512, 512, 512)])
def test_fp16_scales_per_row_and_column(M, K, N):
    """fp16 scales (upcast exactly) against the oracle, per row / per column, full and ragged tiles."""
    rng = np.random.default_rng(M + N)
    a = rng.integers(-128, 128, (M, K)).astype(np.int8)
    b = rng.integers(-128, 128, (K, N)).astype(np.int8)
    asc = rng.uniform(0.002, 0.01, (M, 1)).astype(np.float16)
    bsc = rng.uniform(0.002, 0.01, (1, N)).astype(np.float16)
    az = rng.integers(-16, 17, (M, 1)).astype(np.int8)
    bz = rng.integers(-16, 17, (1, N)).astype(np.int8)
    ys, yz = np.array(0.05, np.float16), np.array(3, np.int8)
    got, ref = run(a, asc, az, b, bsc, bz, ys, yz)
    assert np.array_equal(got, ref)


TYPES = [(np.int8, np.int8, np.int8), (np.uint8, np.int8, np.uint8), (np.int8, np.uint8, np.int8),
         (np.uint8, np.uint8, np.uint8)]
SHAPES = [(1, 1, 1), (33, 45, 17), (300, 272, 208), (256, 256, 256), (300, 200, 272), (512, 512, 512), (5, 7, 0)]


def rint(rng, shape, dt, lo=None, hi=None):
    info = np.iinfo(dt)
    return rng.integers(info.min if lo is None else lo, (info.max if hi is None else hi) + 1, size=shape).astype(dt)


@pytest.mark.parametrize("ta,tb,ty", TYPES)
@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("mode", ["tensor", "rowcol", "vector"])
def test_random(ta, tb, ty, M, N, K, mode):
    rng = np.random.default_rng(M * 1000 + N * 10 + K + len(mode))
    a, b = rint(rng, (M, K), ta), rint(rng, (K, N), tb)
    zlo = lambda d: 0 if d == np.uint8 else -16
    zhi = lambda d: 32 if d == np.uint8 else 16
    if mode == "tensor":
        asc, bsc = np.float32(0.004), np.float32(0.007)
        az, bz = np.array(rint(rng, (), ta, zlo(ta), zhi(ta))), np.array(rint(rng, (), tb, zlo(tb), zhi(tb)))
    else:
        ash, bsh = ((M, 1), (1, N)) if mode == "rowcol" else ((M,), (N,))
        asc = synth.uniform(rng, ash, 0.002, 0.01)
        bsc = synth.uniform(rng, bsh, 0.002, 0.01)
        az, bz = rint(rng, ash, ta, zlo(ta), zhi(ta)), rint(rng, bsh, tb, zlo(tb), zhi(tb))
        if M == 1:
            asc, az = asc.reshape(()) if mode == "vector" else asc, az.reshape(()) if mode == "vector" else az
        if N == 1 and mode == "vector":
            bsc, bz = bsc.reshape(()), bz.reshape(())
    yz = np.array(3 if ty == np.int8 else 120, ty)
    got, ref = run(a, asc, az, b, bsc, bz, 0.05, yz)
    assert got.dtype == ty
    assert np.array_equal(got, ref), (np.argwhere(got != ref)[:5], M, N, K)


@pytest.mark.parametrize("ta,tb,ty", [(np.uint8, np.uint8, np.uint8), (np.uint8, np.int8, np.int8),
                                      (np.int8, np.uint8, np.uint8)])
def test_mixed_types_at_scale(ta, tb, ty):
    """uint8 / mixed operands on the full-tile fast path at a larger size
    (K a multiple of 256 for uint8 a), every output compared."""
    rng = np.random.default_rng(90 + (ta == np.uint8) + 2 * (tb == np.uint8))
    M, K, N = 1024, 2048, 1536
    a, b = rint(rng, (M, K), ta), rint(rng, (K, N), tb)
    zl = lambda d: (100, 150) if d == np.uint8 else (-16, 16)
    az, bz = rint(rng, (M, 1), ta, *zl(ta)), rint(rng, (1, N), tb, *zl(tb))
    asc, bsc = synth.uniform(rng, (M, 1), 0.002, 0.01), synth.uniform(rng, (1, N), 0.002, 0.01)
    yz = np.array(128 if ty == np.uint8 else 0, ty)
    got, ref = run(a, asc, az, b, bsc, bz, 0.05, yz)
    assert got.dtype == ty
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]


def test_batched_params_larger():
    """3-D batch with per-row / per-column parameters per batch entry, full 256x256 tiles."""
    rng = np.random.default_rng(79)
    D, M, K, N = 4, 512, 512, 512
    a, b = rint(rng, (D, M, K), np.int8), rint(rng, (D, K, N), np.uint8)
    az, bz = rint(rng, (D, M, 1), np.int8, -16, 16), rint(rng, (D, 1, N), np.uint8, 100, 150)
    asc, bsc = synth.uniform(rng, (D, M, 1), 0.002, 0.01), synth.uniform(rng, (D, 1, N), 0.002, 0.01)
    got, ref = run(a, asc, az, b, bsc, bz, 0.04, np.array(-5, np.int8))
    assert np.array_equal(got, ref)


def test_batched_params():
    rng = np.random.default_rng(77)
    D, M, K, N = 3, 130, 96, 70
    a, b = rint(rng, (D, M, K), np.int8), rint(rng, (D, K, N), np.int8)
    az, bz = rint(rng, (D, M, 1), np.int8, -16, 16), rint(rng, (D, 1, N), np.int8, -16, 16)
    asc, bsc = synth.uniform(rng, (D, M, 1), 0.002, 0.01), synth.uniform(rng, (D, 1, N), 0.002, 0.01)
    got, ref = run(a, asc, az, b, bsc, bz, 0.05, np.array(0, np.int8))
    assert np.array_equal(got, ref)


def test_broadcast_batch_and_shared_params():
    rng = np.random.default_rng(78)
    a, b = rint(rng, (2, 1, 40, 64), np.uint8), rint(rng, (3, 64, 48), np.int8)
    az, bz = rint(rng, (40, 1), np.uint8, 100, 150), rint(rng, (1, 48), np.int8, -16, 16)
    asc, bsc = synth.uniform(rng, (40, 1), 0.002, 0.01), synth.uniform(rng, (1, 48), 0.002, 0.01)
    got, ref = run(a, asc, az, b, bsc, bz, 0.03, np.array(7, np.int8))
    assert got.shape == (2, 3, 40, 48) and np.array_equal(got, ref)


def test_round_half_even_ties():
    """x = v / 2 exactly: y_scale 2, unit scales.  Ties must go to the even integer."""
    v = np.array([[1, 3, 5, 7, -1, -3, -5, 9, 127, -127]], np.int8)
    a = np.ones((1, 1), np.int8)
    got, ref = run(a, 1.0, np.array(0, np.int8), v, 1.0, np.array(0, np.int8), 2.0, np.array(0, np.int8))
    assert np.array_equal(got[0], [0, 2, 2, 4, 0, -2, -2, 4, 64, -64])
    assert np.array_equal(got, ref)


def test_saturation_and_wraparound():
    K = 40000  # 255 * 255 * K exceeds 2^31: the int32 accumulator wraps
    a = np.full((3, K), -128, np.int8)
    b = np.full((K, 2), -128, np.int8)
    got, ref = run(a, 1.0, np.array(127, np.int8), b, 1.0, np.array(127, np.int8), 1.0, np.array(0, np.int8))
    assert np.array_equal(got, ref)
    a = np.full((2, 64), 127, np.int8)
    b = np.full((64, 2), 127, np.int8)
    got, ref = run(a, 1.0, np.array(0, np.int8), b, 1.0, np.array(0, np.int8), 1.0, np.array(0, np.int8))
    assert np.array_equal(got, ref) and (got == 127).all()


@pytest.mark.parametrize("ta,tb", [(np.int8, np.int8), (np.uint8, np.int8), (np.int8, np.uint8), (np.uint8, np.uint8)])
@pytest.mark.parametrize("scales", ["tame", "tiny", "huge", "zeros"])
def test_full_tiles_scale_ranges(ta, tb, scales):
    """Whole 256x256 tiles (the fast requantisation path): scales inside and
    outside the range where the corrected reciprocal divide is used, and zero
    scales, all bit-exact against the oracle's true division."""
    rng = np.random.default_rng(501 + len(scales) + 3 * (ta == np.uint8) + 7 * (tb == np.uint8))
    M, N, K = 512, 768, 512
    a, b = rint(rng, (M, K), ta), rint(rng, (K, N), tb)
    zlo = lambda d: 0 if d == np.uint8 else -16
    zhi = lambda d: 32 if d == np.uint8 else 16
    az, bz = rint(rng, (M, 1), ta, zlo(ta), zhi(ta)), rint(rng, (1, N), tb, zlo(tb), zhi(tb))
    asc = synth.uniform(rng, (M, 1), 0.002, 0.01)
    bsc = synth.uniform(rng, (1, N), 0.002, 0.01)
    # uint8 operands sit far from their zero points: a larger y_scale keeps y off the rails
    ys = np.float32(0.05 * (64 if (ta == np.uint8 or tb == np.uint8) else 1))
    if scales == "tiny":     # products near 2^-80: outside the fast range
        asc, bsc, ys = asc * np.float32(2.0 ** -32), bsc * np.float32(2.0 ** -32), ys * np.float32(2.0 ** -64)
    elif scales == "huge":   # a scale beyond 2^30
        asc = asc * np.float32(2.0 ** 40)
        ys = ys * np.float32(2.0 ** 40)
    elif scales == "zeros":
        asc[::7] = 0.0
        bsc[:, ::5] = 0.0
    got, ref = run(a, asc, az, b, bsc, bz, ys, np.array(5 if ta == np.int8 else 9, np.int8))
    assert np.array_equal(got, ref), (scales, np.argwhere(got != ref)[:5])
    if scales != "zeros":
        assert len(np.unique(got)) > 50  # the test is not trivially saturated


@pytest.mark.parametrize("M,N,K", [(512, 512, 128), (512, 768, 384), (256, 512, 640), (768, 256, 1152),
                                   (256, 256, 32768)])
def test_int8_whole_tiles_stage_counts(M, N, K):
    """int8 x int8 on whole 256x256 tiles (the 16x16x64 kernel): one stage,
    odd stage counts (the loop then runs one stage of zeros, whose bytes the
    row / column sums must not count), several tile rows and columns, and the
    largest K of that kernel; per-row a and per-column b parameters, uint8
    output, compared in full and bit for bit."""
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    a, b = rint(rng, (M, K), np.int8), rint(rng, (K, N), np.int8)
    az, bz = rint(rng, (M, 1), np.int8, -16, 16), rint(rng, (1, N), np.int8, -16, 16)
    asc = synth.uniform(rng, (M, 1), 0.002, 0.01)
    bsc = synth.uniform(rng, (1, N), 0.002, 0.01)
    ys = np.float32(0.05 * np.sqrt(K / 4096))
    got, ref = run(a, asc, az, b, bsc, bz, ys, np.array(128, np.uint8))
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]
    assert len(np.unique(got)) > 100


def test_int8_whole_tiles_batched_broadcast():
    """The whole-tile kernel over two batch levels (a broadcast over the second),
    per-row / per-column parameters batched like their operands."""
    rng = np.random.default_rng(8)
    a, b = rint(rng, (2, 1, 256, 256), np.int8), rint(rng, (1, 3, 256, 512), np.int8)
    az, bz = rint(rng, (2, 1, 256, 1), np.int8, -16, 16), rint(rng, (1, 3, 1, 512), np.int8, -16, 16)
    asc, bsc = synth.uniform(rng, (2, 1, 256, 1), 0.002, 0.01), synth.uniform(rng, (1, 3, 1, 512), 0.002, 0.01)
    got, ref = run(a, asc, az, b, bsc, bz, np.float32(0.02), np.array(-3, np.int8))
    assert got.shape == (2, 3, 256, 512)
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]


@pytest.mark.parametrize("yz", [0, 3])
def test_int8_whole_tiles_exact_ties(yz):
    """Exact rounding ties on the whole-tile kernel: row m of a holds
    64 (2j + 1) entries of +1 (rows < 128) or -1 (rows >= 128), b is all ones,
    scales 1, zero points 0 and y_scale 128, so x = acc / 128 = +-(j + 0.5)
    exactly and round-half-even decides every output; y_zero_point 0 (the
    epilogue that skips the add) and 3 (odd: the add follows the rounding)."""
    M, N, K = 256, 256, 1024
    a = np.zeros((M, K), np.int8)
    for m in range(M):
        j = m % 8
        a[m, :64 * (2 * j + 1)] = 1 if m < 128 else -1
    b = np.ones((K, N), np.int8)
    z = np.array(0, np.int8)
    got, ref = run(a, 1.0, z, b, 1.0, z, 128.0, np.array(yz, np.int8))
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]
    # the ties really are ties: j + 0.5 rounds to the even neighbour
    want = np.array([[int(np.rint(((1 if m < 128 else -1) * (j + 0.5)))) + yz for _ in range(1)]
                     for m, j in ((m, m % 8) for m in range(M))])
    assert np.array_equal(got[:, :1].astype(int), want)


@pytest.mark.parametrize("ta,tb,ty", [(np.uint8, np.uint8, np.uint8), (np.uint8, np.int8, np.int8),
                                      (np.int8, np.uint8, np.uint8)])
@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (512, 768, 768), (256, 512, 384), (256, 256, 32768)])
def test_uint8_whole_tiles_stage_counts(ta, tb, ty, M, N, K):
    """uint8 and mixed operands on whole 256x256 tiles: the 16x16x64 kernel
    flips uint8 fragments to int8 in registers (K a multiple of 256: the
    fewest stages, several tiles, the largest K); K = 384 (an odd stage count)
    takes the other kernel.  Zero points far from 0 on the uint8 side,
    compared in full and bit for bit."""
    rng = np.random.default_rng(M + 3 * N + 7 * K + 11 * (ta == np.uint8) + 13 * (tb == np.uint8))
    a, b = rint(rng, (M, K), ta), rint(rng, (K, N), tb)
    zl = lambda d: (100, 150) if d == np.uint8 else (-16, 16)
    az, bz = rint(rng, (M, 1), ta, *zl(ta)), rint(rng, (1, N), tb, *zl(tb))
    asc = synth.uniform(rng, (M, 1), 0.002, 0.01)
    bsc = synth.uniform(rng, (1, N), 0.002, 0.01)
    ys = np.float32(0.05 * np.sqrt(K / 4096))
    got, ref = run(a, asc, az, b, bsc, bz, ys, np.array(128 if ty == np.uint8 else -2, ty))
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]
    assert len(np.unique(got)) > 100


@pytest.mark.parametrize("ta,tb", [(np.uint8, np.uint8), (np.uint8, np.int8), (np.int8, np.uint8)])
def test_uint8_whole_tiles_exact_ties(ta, tb):
    """The exact-tie construction of the int8 test with uint8 operands: a uint8
    entry is the int8 one + 128 and its zero point 128, so a - a_zero_point
    (and b - b_zero_point) are the same +-1 / 0 values and every output is a
    rounding tie."""
    M, N, K = 256, 256, 1024
    a = np.zeros((M, K), np.int16)
    for m in range(M):
        j = m % 8
        a[m, :64 * (2 * j + 1)] = 1 if m < 128 else -1
    b = np.ones((K, N), np.int16)
    off = lambda d: 128 if d == np.uint8 else 0
    za, zb = np.array(off(ta), ta), np.array(off(tb), tb)
    got, ref = run((a + off(ta)).astype(ta), 1.0, za, (b + off(tb)).astype(tb), 1.0, zb, 128.0, np.array(3, np.int8))
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]
    want = np.array([int(np.rint((1 if m < 128 else -1) * (m % 8 + 0.5))) + 3 for m in range(M)])
    assert np.array_equal(got[:, 0].astype(int), want)


DECODE = [  # (M, K, N): at most 4 rows, one batch -> b streamed on the vector ALU
    (1, 4096, 4096), (2, 256, 16), (3, 4112, 1024), (4, 8192, 4096), (1, 8192, 11008), (4, 1040, 528),
]


@pytest.mark.parametrize("ta,tb,ty", [(np.int8, np.int8, np.int8), (np.uint8, np.uint8, np.uint8),
                                      (np.uint8, np.int8, np.int8), (np.int8, np.uint8, np.uint8)])
@pytest.mark.parametrize("M,K,N", DECODE)
def test_decode_rows(ta, tb, ty, M, K, N):
    """Decode-like shapes (1-4 rows, one batch): every output bit-exact, with
    per-row / per-column parameters, a K tail inside the last 64-row group and
    a single 16-column group."""
    rng = np.random.default_rng(M * 7 + K + N + (ta == np.uint8) + 2 * (tb == np.uint8))
    a, b = rint(rng, (M, K), ta), rint(rng, (K, N), tb)
    zl = lambda d: (100, 150) if d == np.uint8 else (-16, 16)
    az, bz = rint(rng, (M, 1), ta, *zl(ta)), rint(rng, (1, N), tb, *zl(tb))
    asc, bsc = synth.uniform(rng, (M, 1), 0.002, 0.01), synth.uniform(rng, (1, N), 0.002, 0.01)
    yz = np.array(128 if ty == np.uint8 else -3, ty)
    got, ref = run(a, asc, az, b, bsc, bz, 0.05, yz)
    assert got.dtype == ty
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]


def test_decode_rows_scalar_params_fp16_and_saturation():
    """Decode-like rows with per-tensor parameters and fp16 scales, then unit
    scales and extreme zero points so that most outputs saturate."""
    rng = np.random.default_rng(4242)
    M, K, N = 2, 2048, 2048
    a, b = rint(rng, (M, K), np.int8), rint(rng, (K, N), np.int8)
    got, ref = run(a, np.float16(0.004), np.array(3, np.int8), b, np.float16(0.006), np.array(-7, np.int8),
                   np.float16(0.05), np.array(1, np.int8))
    assert np.array_equal(got, ref)
    got, ref = run(a, 1.0, np.array(127, np.int8), b, 1.0, np.array(-128, np.int8), 1.0, np.array(0, np.int8))
    assert np.array_equal(got, ref)
    assert (np.abs(got.astype(np.int32)) >= 127).mean() > 0.5
