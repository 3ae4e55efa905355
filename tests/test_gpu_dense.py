"""GPU parity of MatMul and Gemm (bf16 / fp16 / fp32 / fp64) against the CPU oracle,
through the C ABI.  Shapes span several tiles with ragged tails in every dim,
all four transpose combinations, every C broadcast form, 1-D promotion and
batch broadcasting, plus bit-exact small-integer cases."""
import numpy as np
import pytest
import torch

import oracle
from onnx_matmul_family_amd import synth
from tests.gpu_util import check_close, dev, host_f32, host_f64, sample_indices

pytestmark = pytest.mark.gpu

om = pytest.importorskip("onnx_matmul_family_amd._omm")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    om.lib()


def draw(rng, shape, dt, kind="normal"):
    x = synth.small_ints(rng, shape) if kind == "int" else synth.normal(rng, shape)
    return synth.store(x, dt)


GEMM_SHAPES = [(1, 1, 1), (7, 5, 3), (64, 32, 48), (300, 520, 200), (257, 129, 199), (130, 264, 136), (33, 17, 0)]


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32", "f64"])
@pytest.mark.parametrize("tA,tB", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_shapes(dt, tA, tB, M, N, K):
    rng = np.random.default_rng(M * 7919 + N * 31 + K + 2 * tA + tB)
    A = draw(rng, (K, M) if tA else (M, K), dt)
    B = draw(rng, (N, K) if tB else (K, N), dt)
    C = draw(rng, (N,), dt)
    alpha, beta = 0.75, -1.25
    Y = om.gemm(dev(A, dt), dev(B, dt), dev(C, dt), alpha, beta, tA, tB)
    torch.cuda.synchronize()
    y, t = oracle.gemm(A, B, C, alpha, beta, tA, tB, dt=dt)
    cval = oracle.decode(C, dt)
    check_close(host_f64(Y), y, abs(alpha) * t + abs(beta) * np.abs(cval)[None, :], dt,
                "gemm %s %dx%dx%d tA=%d tB=%d" % (dt, M, N, K, tA, tB))


@pytest.mark.parametrize("dt", ["bf16", "f32", "f64"])
@pytest.mark.parametrize("cshape", [None, (), (1,), (90,), (1, 90), (70, 1), (70, 90), (1, 1)])
def test_gemm_c_forms(dt, cshape):
    rng = np.random.default_rng(101)
    M, N, K = 70, 90, 40
    A, B = draw(rng, (M, K), dt), draw(rng, (K, N), dt)
    C = draw(rng, cshape, dt) if cshape is not None else None
    Y = om.gemm(dev(A, dt), dev(B, dt), dev(C, dt) if C is not None else None, 1.5, 0.5)
    torch.cuda.synchronize()
    y, t = oracle.gemm(A, B, C, 1.5, 0.5, dt=dt)
    cm = 0.5 * np.abs(np.broadcast_to(oracle.decode(C.ravel(), dt).reshape(cshape), (M, N))) if C is not None else 0
    check_close(host_f64(Y), y, 1.5 * t + cm, dt, "gemm C %s" % (cshape,))


@pytest.mark.parametrize("dt", ["bf16", "f16", "f64"])
@pytest.mark.parametrize("tA,tB", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_gemm_small_integers_exact(dt, tA, tB):
    """Entries in {-2..2} with K = 64: every partial sum is an integer of
    magnitude <= 256, exact in fp32 and in the output type -> bit-exact."""
    rng = np.random.default_rng(7 + tA + 2 * tB)
    M, N, K = 300, 270, 64
    A = draw(rng, (K, M) if tA else (M, K), dt, "int")
    B = draw(rng, (N, K) if tB else (K, N), dt, "int")
    C = draw(rng, (M, N), dt, "int")
    Y = om.gemm(dev(A, dt), dev(B, dt), dev(C, dt), 1.0, 1.0, tA, tB)
    torch.cuda.synchronize()
    y, _ = oracle.gemm(A, B, C, 1.0, 1.0, tA, tB, dt=dt)
    assert np.array_equal(host_f64(Y), y)


@pytest.mark.parametrize("tA,tB", [(0, 1), (0, 0), (1, 0)])
def test_gemm_bf16_large_tile_path(tA, tB):
    """Enough output tiles for the 256x256 kernel, ragged M and N, K multiple of 64: every element."""
    rng = np.random.default_rng(211 + tA + tB)
    M, N, K = 4224, 4160, 256
    A = synth.store(synth.normal(rng, (K, M) if tA else (M, K), 0.05), "bf16")
    B = synth.store(synth.normal(rng, (N, K) if tB else (K, N), 0.05), "bf16")
    C = synth.store(synth.uniform(rng, (N,), -0.1, 0.1), "bf16")
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    om.gemm(dev(A, "bf16"), dev(B, "bf16"), dev(C, "bf16"), 1.0, 1.0, tA, tB, Y)
    torch.cuda.synchronize()
    y, t = oracle.gemm(A, B, C, 1.0, 1.0, tA, tB, dt="bf16")
    check_close(host_f32(Y), y, t, "bf16", "gemm 256-tile tA=%d tB=%d" % (tA, tB))


def rne(y, dt):
    """Exact integer-valued fp64 results (|y| < 2^24) rounded once, to nearest even, to bf16 / fp16, as fp64."""
    assert np.abs(y).max() < 2 ** 24
    to = torch.bfloat16 if dt == "bf16" else torch.float16
    return torch.from_numpy(np.ascontiguousarray(y)).to(torch.float32).to(to).to(torch.float64).numpy()


C_FORMS = {"MN": lambda M, N: (M, N), "M1": lambda M, N: (M, 1), "scalar": lambda M, N: (), "N": lambda M, N: (N,)}


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("tA,tB", [(0, 1), (0, 0), (1, 0), (1, 1)])
@pytest.mark.parametrize("cform", list(C_FORMS))
def test_ragged_256_tiles_k_tail_exact(dt, tA, tB, cform):
    """The 256x256 kernel on ragged tiles (M = 16.5, N = 16.25 tiles), a K tail
    (K = 200 = 3 stages of 64 + 8) and every C form: small integers in
    {-2..2}, so every fp32 partial sum is exact and each output is the one
    rounding of an exact integer -- compared bit for bit, every element."""
    rng = np.random.default_rng(500 + 8 * tA + 4 * tB + list(C_FORMS).index(cform))
    M, N, K = 4224, 4160, 200
    A = synth.store(synth.small_ints(rng, (K, M) if tA else (M, K)), dt)
    B = synth.store(synth.small_ints(rng, (N, K) if tB else (K, N)), dt)
    C = synth.store(synth.small_ints(rng, C_FORMS[cform](M, N), -8, 8), dt)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16 if dt == "bf16" else torch.float16, device="cuda")
    om.gemm(dev(A, dt), dev(B, dt), dev(C, dt), 1.0, 1.0, tA, tB, Y)
    torch.cuda.synchronize()
    y, _ = oracle.gemm(A, B, C, 1.0, 1.0, tA, tB, dt=dt)
    got, want = host_f32(Y), rne(y, dt)
    bad = np.argwhere(~(got == want))
    assert bad.size == 0, "%d differ, first at %s: got %r want %r" % (len(bad), tuple(bad[0]), got[tuple(bad[0])],
                                                                      want[tuple(bad[0])])


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("tA,tB", [(0, 1), (0, 0), (1, 0), (1, 1)])
@pytest.mark.parametrize("cform", list(C_FORMS))
def test_ragged_128_tiles_k_tail_exact(dt, tA, tB, cform):
    """Fewer than 256 tiles of 256x256 (here 4 x 5): 128x128 tiles on the same
    16x16x32 DMA kernel, ragged in M, N and K (1000 x 1064 x 1032: 16 stages
    of 64 + 8), every C form, small integers: bit for bit, every element."""
    rng = np.random.default_rng(700 + 8 * tA + 4 * tB + list(C_FORMS).index(cform))
    M, N, K = 1000, 1064, 1032
    A = synth.store(synth.small_ints(rng, (K, M) if tA else (M, K), -1, 1), dt)
    B = synth.store(synth.small_ints(rng, (N, K) if tB else (K, N), -1, 1), dt)
    C = synth.store(synth.small_ints(rng, C_FORMS[cform](M, N), -8, 8), dt)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16 if dt == "bf16" else torch.float16, device="cuda")
    om.gemm(dev(A, dt), dev(B, dt), dev(C, dt), 1.0, 1.0, tA, tB, Y)
    torch.cuda.synchronize()
    y, _ = oracle.gemm(A, B, C, 1.0, 1.0, tA, tB, dt=dt)
    got, want = host_f32(Y), rne(y, dt)
    bad = np.argwhere(~(got == want))
    assert bad.size == 0, "%d differ, first at %s: got %r want %r" % (len(bad), tuple(bad[0]), got[tuple(bad[0])],
                                                                      want[tuple(bad[0])])


@pytest.mark.parametrize("tA,tB", [(0, 1), (0, 0), (1, 0), (1, 1)])
def test_ragged_256_tiles_long_k_tail_exact(tA, tB):
    """The same kernel with K = 4104 (64 whole stages and a tail of 8, an odd
    stage count): complete rows from the first, a middle and the ragged last
    tile row, and complete columns from the first and the ragged last tile
    column, bit for bit.  dtype and C form vary with the transposes."""
    dt = "bf16" if tA == tB else "f16"
    cform = list(C_FORMS)[2 * tA + tB]
    rng = np.random.default_rng(600 + 2 * tA + tB)
    M, N, K = 4224, 4160, 4104
    A = synth.store(synth.small_ints(rng, (K, M) if tA else (M, K)), dt)
    B = synth.store(synth.small_ints(rng, (N, K) if tB else (K, N)), dt)
    C = synth.store(synth.small_ints(rng, C_FORMS[cform](M, N), -8, 8), dt)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16 if dt == "bf16" else torch.float16, device="cuda")
    om.gemm(dev(A, dt), dev(B, dt), dev(C, dt), 1.0, 1.0, tA, tB, Y)
    torch.cuda.synchronize()
    got = host_f32(Y)
    rows = np.unique(np.concatenate([np.arange(0, 256, 17), 2048 + np.arange(3, 256, 23), np.arange(4096, M, 9),
                                     [M - 1]]))
    cols = np.unique(np.concatenate([np.arange(0, 256, 29), np.arange(4096, N, 5), [N - 1]]))
    sel = np.unique(np.concatenate([(rows[:, None] * N + np.arange(N)[None, :]).ravel(),
                                    (np.arange(M)[:, None] * N + cols[None, :]).ravel()])).astype(np.int64)
    y, _ = oracle.gemm(A, B, C, 1.0, 1.0, tA, tB, dt=dt, sel=sel)
    g, w = got.ravel()[sel], rne(y, dt)
    bad = np.flatnonzero(~(g == w))
    assert bad.size == 0, "%d differ, first at flat %d: got %r want %r" % (len(bad), sel[bad[0]], g[bad[0]], w[bad[0]])


MATMUL_SHAPES = [
    ((5,), (5,)), ((3,), (3, 4)), ((4, 3), (3,)), ((2, 3, 4), (4, 5)), ((4, 5), (2, 5, 3)),
    ((2, 1, 3, 4), (5, 4, 2)), ((1, 6, 2), (3, 1, 2, 7)), ((7,), (2, 3, 7, 2)), ((2, 3, 4, 5), (5,)),
    ((3, 1, 70, 40), (1, 4, 40, 90)), ((2, 3, 2, 130, 72), (3, 1, 72, 66)), ((5, 200, 64), (64, 136)),
    ((2, 2, 2, 2, 33, 17), (2, 1, 2, 1, 17, 9)), ((0, 3), (3, 4)), ((4, 0), (0, 3)),
]


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32", "f64"])
@pytest.mark.parametrize("sa,sb", MATMUL_SHAPES)
def test_matmul_broadcast(dt, sa, sb):
    rng = np.random.default_rng(abs(hash((sa, sb))) % 2**31)
    A, B = draw(rng, sa, dt), draw(rng, sb, dt)
    Y = om.matmul(dev(A, dt), dev(B, dt))
    torch.cuda.synchronize()
    y, t = oracle.matmul(A, B, dt=dt)
    assert tuple(Y.shape) == y.shape
    check_close(host_f64(Y), y, t, dt, "matmul %s %s x %s" % (dt, sa, sb))


def test_matmul_bf16_batched_large_tile_path():
    """The broadcast-batch structure at 1/2 scale in M, N, K: 128 batches, 256x256 tiles, n-contiguous B."""
    c = synth.matmul_bf16_bcast(seed=11, scale=2)
    A, B = c["A"], c["B"]
    Y = om.matmul(dev(A, "bf16"), dev(B, "bf16"))
    torch.cuda.synchronize()
    y, t = oracle.matmul(A, B, dt="bf16")
    check_close(host_f32(Y), y, t, "bf16", "matmul batched 256-tile")


def test_matmul_small_integers_exact_batched():
    rng = np.random.default_rng(99)
    A = synth.store(synth.small_ints(rng, (4, 1, 130, 64)), "bf16")
    B = synth.store(synth.small_ints(rng, (1, 3, 64, 136)), "bf16")
    Y = om.matmul(dev(A, "bf16"), dev(B, "bf16"))
    torch.cuda.synchronize()
    y, _ = oracle.matmul(A, B, dt="bf16")
    assert np.array_equal(host_f64(Y), y)


def test_printed_examples_on_gpu(golden):
    """The pages' fp32 MatMul and Gemm examples through the GPU path."""
    from tests.test_oracle_examples import arr, half_ulps
    for ex in golden("matmul"):
        A, B = arr(ex["inputs"]["A"]), arr(ex["inputs"]["B"])
        Y = om.matmul(dev(A), dev(B))
        torch.cuda.synchronize()
        exp = arr(ex["outputs"]["Y"]).astype(np.float64)
        y, t = oracle.matmul(A, B)
        assert tuple(Y.shape) == exp.shape, ex["cite"]
        check_close(host_f64(Y), y, t, "f32", ex["cite"])
        assert np.all(np.abs(host_f64(Y) - exp) <= 1e-5 * t + 1e-6 + half_ulps(ex["outputs"]["Y"])), ex["cite"]
    for ex in golden("gemm"):
        at = ex["attrs"]
        alpha, beta = float(at.get("alpha", "1.0")), float(at.get("beta", "1.0"))
        tA, tB = int(at.get("transA", "0")), int(at.get("transB", "0"))
        A, B = arr(ex["inputs"]["A"]), arr(ex["inputs"]["B"])
        C = arr(ex["inputs"]["C"]) if "C" in ex["inputs"] else None
        Y = om.gemm(dev(A), dev(B), dev(C) if C is not None else None, alpha, beta, tA, tB)
        torch.cuda.synchronize()
        y, t = oracle.gemm(A, B, C, alpha, beta, tA, tB)
        cm = abs(beta) * np.abs(np.broadcast_to(C, y.shape)) if C is not None else 0
        check_close(host_f64(Y), y, abs(alpha) * t + cm, "f32", ex["cite"])


def test_gemm_on_side_stream_and_reuse():
    """Work is enqueued on the caller's stream; a second call on the same buffers is consistent."""
    rng = np.random.default_rng(5)
    A, B = draw(rng, (200, 96), "bf16"), draw(rng, (96, 150), "bf16")
    dA, dB = dev(A, "bf16"), dev(B, "bf16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Y1 = om.gemm(dA, dB, None, 1.0, 0.0)
        Y2 = om.gemm(dA, dB, None, 1.0, 0.0)
    s.synchronize()
    assert torch.equal(Y1, Y2)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("tA,tB", [(0, 1), (0, 0), (1, 0), (1, 1)])
@pytest.mark.parametrize("cform", ["none", "row", "matrix"])
def test_full_tile_modes_exact(dt, tA, tB, cform):
    """Every tile whole (the epilogue without bounds checks, staged through
    LDS): no C, a bias row, and a full C (general epilogue).  Small integers
    make every sum exact, so every output must match bit for bit."""
    rng = np.random.default_rng(300 + 2 * tA + tB + len(cform))
    M, N, K = 4096, 4096, 64
    # |sum| <= 64 + 8: every partial sum and result is an integer exact in bf16
    A = synth.store(synth.small_ints(rng, (K, M) if tA else (M, K), -1, 1), dt)
    B = synth.store(synth.small_ints(rng, (N, K) if tB else (K, N), -1, 1), dt)
    C = None
    if cform == "row":
        C = synth.store(synth.small_ints(rng, (N,), -8, 8), dt)
    elif cform == "matrix":
        C = synth.store(synth.small_ints(rng, (M, N), -8, 8), dt)
    Y = om.gemm(dev(A, dt), dev(B, dt), dev(C, dt) if C is not None else None, 1.0, 1.0, tA, tB)
    torch.cuda.synchronize()
    y, _ = oracle.gemm(A, B, C, 1.0, 1.0, tA, tB, dt=dt)
    got = host_f32(Y)
    assert np.array_equal(got, y), np.argwhere(got != y)[:5]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("tA,tB", [(0, 1), (0, 0), (1, 0), (1, 1)])
@pytest.mark.parametrize("K", [192, 320])
def test_full_tile_odd_stage_counts(dt, tA, tB, K):
    """Whole 256x256 tiles with an odd number of 64-k stages (3 and 5): the
    K loop runs stages in pairs, the last pair's second stage on zeros."""
    rng = np.random.default_rng(400 + 2 * tA + tB + K)
    M, N = 4096, 4096
    A = synth.store(synth.normal(rng, (K, M) if tA else (M, K), 0.05), dt)
    B = synth.store(synth.normal(rng, (N, K) if tB else (K, N), 0.05), dt)
    C = synth.store(synth.uniform(rng, (N,), -0.1, 0.1), dt)
    Y = om.gemm(dev(A, dt), dev(B, dt), dev(C, dt), 0.75, 1.25, tA, tB)
    torch.cuda.synchronize()
    y, t = oracle.gemm(A, B, C, 0.75, 1.25, tA, tB, dt=dt)
    check_close(host_f32(Y), y, 0.75 * t + 1.25 * np.abs(oracle.decode(C, dt))[None, :], dt,
                "gemm full tiles K=%d tA=%d tB=%d" % (K, tA, tB))


SPLITK = [  # (A shape, B shape, transA, transB): few output tiles, long K -> split-K path
    ((64, 8192), (8192, 4096), 0, 0), ((64, 8192), (4096, 8192), 0, 1), ((8192, 96), (8192, 1024), 1, 0),
    ((200, 4104), (4104, 320), 0, 0), ((1, 6144), (6144, 2048), 0, 0),
]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("sa,sb,tA,tB", SPLITK)
def test_gemm_split_k(dt, sa, sb, tA, tB):
    """Long-K, few-tile shapes: partial products over K ranges, reduced in a
    second kernel with the alpha / beta / C epilogue (ragged last K range for
    K = 4104)."""
    rng = np.random.default_rng(sum(sa) + sum(sb) + tA + tB)
    A = synth.store(synth.normal(rng, sa, 0.05), dt)
    B = synth.store(synth.normal(rng, sb, 0.05), dt)
    N = sb[0] if tB else sb[1]
    C = synth.store(synth.uniform(rng, (N,), -0.1, 0.1), dt)
    Y = om.gemm(dev(A, dt), dev(B, dt), dev(C, dt), 0.5, -1.5, tA, tB)
    torch.cuda.synchronize()
    M = Y.shape[0]
    y, t = oracle.gemm(A, B, C, 0.5, -1.5, tA, tB, dt=dt)
    c64 = oracle.decode(C, dt)
    check_close(host_f64(Y), y, 0.5 * t + 1.5 * np.abs(c64)[None, :], dt, "split-K %s %s x %s" % (dt, sa, sb))


SKINNY = [  # M, N, K: M <= 16 rows against B stored (N, K) -> the B-streaming skinny kernels
    (1, 8192, 8192), (5, 8200, 3000), (16, 8192, 1024),                        # single pass (>= 512 x 16 columns)
    (12, 8200, 3000), (9, 8240, 2056),               # single pass, 32-column workgroups, ragged N and K
    (16, 4096, 4104), (7, 4100, 2056), (16, 64, 1024), (2, 4104, 14336), (16, 1000, 9000),  # single pass, 8 waves
    (3, 100, 1000), (1, 1, 20000), (16, 1000, 20000), (4, 2056, 16392),  # K split over workgroups
]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("M,N,K", SKINNY)
def test_gemm_skinny_stream(dt, M, N, K):
    """Decode-like Gemm, transB=1: B streamed in the MFMA operand layout, K split
    over workgroups (ragged last range, N tails, a single column), reduced with
    the alpha / beta / C epilogue."""
    rng = np.random.default_rng(M * 131 + N + K)
    A = synth.store(synth.normal(rng, (M, K)), dt)
    B = synth.store(synth.normal(rng, (N, K), 0.02), dt)
    C = synth.store(synth.uniform(rng, (M, N), -0.1, 0.1), dt)
    Y = om.gemm(dev(A, dt), dev(B, dt), dev(C, dt), 0.75, 1.25, 0, 1)
    torch.cuda.synchronize()
    y, t = oracle.gemm(A, B, C, 0.75, 1.25, 0, 1, dt=dt)
    cabs = np.abs(oracle.decode(C, dt)).reshape(M, N)
    check_close(host_f64(Y), y, 0.75 * t + 1.25 * cabs, dt, "skinny %s M=%d N=%d K=%d" % (dt, M, N, K))


SKINNY_NMAJ = [  # MatMul with a few rows against B stored (K, N): the vector-ALU streaming kernel
    # 16- or 32-column workgroups of 4 waves over all of K
    ((1, 8192), (8192, 8192)), ((8192,), (8192, 4096)), ((3, 2048), (2048, 4104)), ((2, 1024), (1024, 8200)),
    ((2, 1, 1024), (2, 1024, 2048)), ((4, 4096), (4096, 4096)), ((2, 1, 4096), (2, 4096, 2048)),
    # fewer column groups: 16-column workgroups of 8 waves (ragged last group, a batch)
    ((1, 4096), (4096, 2048)), ((2, 8192), (8192, 1032)), ((4, 4096), (4096, 520)), ((2, 1, 8192), (2, 8192, 1000)),
    # 3-4 rows, K > 4096, and few columns with long K: K split over workgroups + reduction
    ((4, 7680), (7680, 4096)), ((1, 12288), (12288, 1024)),
]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("sa,sb", SKINNY_NMAJ)
def test_matmul_skinny_nmajor(dt, sa, sb):
    rng = np.random.default_rng(sum(sa) + sum(sb))
    A = synth.store(synth.normal(rng, sa), dt)
    B = synth.store(synth.normal(rng, sb, 0.02), dt)
    Y = om.matmul(dev(A, dt), dev(B, dt))
    torch.cuda.synchronize()
    y, t = oracle.matmul(A, B, dt=dt)
    assert tuple(Y.shape) == y.shape
    check_close(host_f64(Y), y, t, dt, "skinny n-major %s %s x %s" % (dt, sa, sb))


@pytest.mark.parametrize("N", [4096, 1032])  # 4 waves per workgroup / 8 (few column groups)
def test_gemm_skinny_nmajor_epilogue_exact(N):
    """Gemm transB=0 with 2 rows, C per row and column, small integers: bit-exact."""
    rng = np.random.default_rng(12)
    M, K = 2, 4096
    A = synth.store(rng.integers(-1, 2, (M, K)).astype(np.float32) * (np.arange(K) % 16 == 0), "bf16")
    B = synth.store(rng.integers(-1, 2, (K, N)).astype(np.float32), "bf16")
    C = synth.store(rng.integers(-8, 9, (M, N)).astype(np.float32), "bf16")
    Y = om.gemm(dev(A, "bf16"), dev(B, "bf16"), dev(C, "bf16"), 1.0, 2.0, 0, 0)
    torch.cuda.synchronize()
    y, _ = oracle.gemm(A, B, C, 1.0, 2.0, 0, 0, dt="bf16")
    assert np.array_equal(host_f64(Y), y)


@pytest.mark.parametrize("K", [2048, 20480])  # single pass (8 waves) / K split over workgroups
@pytest.mark.parametrize("M", [1, 5, 16])
def test_gemm_skinny_exact(M, K):
    """Small integers (entries in {-1, 0, 1}, |partial sums| <= 256): bit-exact."""
    rng = np.random.default_rng(M)
    N = 320
    A = synth.store(rng.integers(-1, 2, (M, K)).astype(np.float32) * (np.arange(K) % (K // 256) == 0), "bf16")
    B = synth.store(rng.integers(-1, 2, (N, K)).astype(np.float32), "bf16")
    Y = om.gemm(dev(A, "bf16"), dev(B, "bf16"), None, 1.0, 0.0, 0, 1)
    torch.cuda.synchronize()
    y, _ = oracle.gemm(A, B, None, 1.0, 0.0, 0, 1, dt="bf16")
    assert np.array_equal(host_f64(Y), y)


@pytest.mark.parametrize("M", [1, 8, 9, 16])
def test_gemm_skinny_single_pass_exact(M):
    """The single-pass kernel on both sides of its 8-row switch (16 or 32
    columns per workgroup), a ragged last column group and a K tail: small
    integers, so both sides sum exactly and round once to bf16: bit-exact."""
    rng = np.random.default_rng(40 + M)
    K, N = 2056, 8216
    A = synth.store(rng.integers(-1, 2, (M, K)).astype(np.float32) * (np.arange(K) % 8 == 0), "bf16")
    B = synth.store(rng.integers(-1, 2, (N, K)).astype(np.float32), "bf16")
    C = synth.store(rng.integers(-8, 9, (N,)).astype(np.float32), "bf16")
    Y = om.gemm(dev(A, "bf16"), dev(B, "bf16"), dev(C, "bf16"), 1.0, 2.0, 0, 1)
    torch.cuda.synchronize()
    y, _ = oracle.gemm(A, B, C, 1.0, 2.0, 0, 1, dt="bf16")
    assert np.array_equal(host_f64(Y), y)


def test_split_k_workspace_two_streams_exact():
    """Split-K calls (tile path, skinny path, n-contiguous B) issued on two
    streams without waits between them, the workspace growing on the way:
    every output bit-exact (small integers, exact fp32 sums) against the
    oracle.  The library orders calls that share its split-K workspace."""
    rng = np.random.default_rng(951)
    cases = [  # (M, N, K, transB): workspace sizes grow and shrink along the list
        (8, 4096, 4096, 0), (24, 4096, 4096, 1), (16, 1000, 20480, 1), (4, 2056, 16392, 1), (32, 2048, 8192, 0),
        (8, 4096, 4096, 0), (16, 1000, 20480, 1),
    ]
    data, outs = [], []
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for i, (M, N, K, tB) in enumerate(cases):
        step = max(1, K // 256)
        A = synth.store(rng.integers(-1, 2, (M, K)).astype(np.float32) * (np.arange(K) % step == 0), "bf16")
        B = synth.store(rng.integers(-1, 2, (N, K) if tB else (K, N)).astype(np.float32), "bf16")
        data.append((A, B, tB))
        dA, dB = dev(A, "bf16"), dev(B, "bf16")
        torch.cuda.synchronize()
        with torch.cuda.stream(streams[i % 2]):
            Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
            om.gemm(dA, dB, None, 1.0, 0.0, 0, tB, Y)
        outs.append((Y, dA, dB))
    torch.cuda.synchronize()
    for (A, B, tB), (Y, _, _) in zip(data, outs):
        y, _ = oracle.gemm(A, B, None, 1.0, 0.0, 0, tB, dt="bf16")
        assert np.array_equal(host_f64(Y), y), (A.shape, B.shape, tB)


def test_matmul_split_k_decode_batch_exact():
    """A batch of single-token rows against one weight matrix (batch folds into
    M = 8): split-K, small integers, fp16 output exact."""
    rng = np.random.default_rng(901)
    A = synth.store(synth.small_ints(rng, (8, 1, 8192), -1, 1), "f16")
    B = synth.store(synth.small_ints(rng, (8192, 3072), -1, 1), "f16")
    Y = om.matmul(dev(A, "f16"), dev(B, "f16"))
    torch.cuda.synchronize()
    y, _ = oracle.matmul(A, B, dt="f16")
    assert tuple(Y.shape) == (8, 1, 3072)
    assert np.abs(y).max() < 2048
    assert np.array_equal(host_f64(Y), y)


def test_gemm_f64_full_size_sampled():
    """The fp64 Gemm at its benchmark size (4096^3, B stored (N, K), a C row),
    in the launch configuration the benchmark times: sampled outputs against
    the oracle's fp64 sums."""
    rng = np.random.default_rng(64)
    n = 4096
    A = synth.store(synth.normal(rng, (n, n)), "f64")
    B = synth.store(synth.normal(rng, (n, n)), "f64")
    C = synth.store(synth.normal(rng, (n,)), "f64")
    Y = om.gemm(dev(A, "f64"), dev(B, "f64"), dev(C, "f64"), 1.0, 1.0, 0, 1)
    torch.cuda.synchronize()
    sel = sample_indices(n * n, 3000, 11)
    y, t = oracle.gemm(A, B, C, 1.0, 1.0, 0, 1, dt="f64", sel=sel)
    check_close(host_f64(Y).ravel()[sel], y, t + np.abs(C[sel % n]), "f64", "gemm f64 4096^3 sampled")
