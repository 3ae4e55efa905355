"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/omm.h declares, and rejects invalid arguments on the host (before any
launch).  No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "omm.h")

om = pytest.importorskip("onnx_matmul_family_amd._omm")

if not os.path.exists(om.LIB_PATH):
    from onnx_matmul_family_amd import build as _build
    _build.build()


def declared_symbols():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(omm_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = om.lib()
    names = declared_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    L = om.lib()
    assert L.omm_version() >= 100
    for code in range(0, -9, -1):
        s = om.status_string(code)
        assert s and s != "unknown status", code
    assert om.status_string(-99) == "unknown status"


FAKE = 0x100000  # never dereferenced: every call below fails validation first


def T(shape, dt, data=FAKE):
    t = om.OmmTensor()
    t.data = data
    t.dtype = dt
    t.ndim = len(shape)
    for i, s in enumerate(shape):
        t.shape[i] = s
    return t


F32, F16, BF16, F64, I8, U8, I32, I64 = range(8)


def out_shape(fn, *args):
    nd = ctypes.c_int32(0)
    sh = (ctypes.c_int64 * 8)()
    rc = fn(*args, ctypes.byref(nd), sh)
    return rc, tuple(sh[i] for i in range(nd.value))


@pytest.mark.parametrize("sa,sb,exp", [
    ((3,), (3,), ()), ((4,), (2, 4, 3), (2, 3)), ((2, 3), (3, 4), (2, 4)), ((2, 3, 4, 5), (5,), (2, 3, 4)),
    ((2, 2, 3), (1, 3, 4), (2, 2, 4)), ((2, 3, 4), (4, 5), (2, 3, 5)), ((8, 1, 5, 6), (1, 16, 6, 7), (8, 16, 5, 7)),
    ((0, 3), (3, 4), (0, 4)), ((3, 1, 2, 3), (0, 3, 2), (3, 0, 2, 2)),
])
def test_matmul_output_shape(sa, sb, exp):
    L = om.lib()
    rc, sh = out_shape(L.omm_matmul_output_shape, ctypes.byref(T(sa, BF16)), ctypes.byref(T(sb, BF16)))
    assert rc == 0 and sh == exp


@pytest.mark.parametrize("sa,sb,code", [((2, 3), (4, 5), -3), ((2, 2, 3), (3, 3, 4), -4), ((3,), (4,), -3),
                                        ((), (3,), -3)])
def test_matmul_shape_errors(sa, sb, code):
    L = om.lib()
    rc, _ = out_shape(L.omm_matmul_output_shape, ctypes.byref(T(sa, BF16)), ctypes.byref(T(sb, BF16)))
    assert rc == code


def test_matmul_argument_errors():
    L = om.lib()
    A, B, Y = T((4, 8), BF16), T((8, 5), BF16), T((4, 5), BF16)
    assert L.omm_matmul(None, ctypes.byref(B), ctypes.byref(Y), None) == -1
    assert L.omm_matmul(ctypes.byref(A), ctypes.byref(T((8, 5), F16)), ctypes.byref(Y), None) == -2
    assert L.omm_matmul(ctypes.byref(T((4, 8), I32)), ctypes.byref(T((8, 5), I32)),
                        ctypes.byref(T((4, 5), I32)), None) == -5
    assert L.omm_matmul(ctypes.byref(A), ctypes.byref(B), ctypes.byref(T((4, 6), BF16)), None) == -3
    assert L.omm_matmul(ctypes.byref(T((4, 8), BF16, 0)), ctypes.byref(B), ctypes.byref(Y), None) == -1
    # empty output: valid, nothing launched
    assert L.omm_matmul(ctypes.byref(T((0, 8), BF16)), ctypes.byref(B), ctypes.byref(T((0, 5), BF16)), None) == 0


def test_gemm_noalloc_rejects_oversized_scratch():
    """A decode-like bf16 Gemm (16 rows, K = 131328, N = 8176) whose split-K
    partials (65 K ranges x 16 x 8176 x 4 bytes) exceed the 32 MiB static
    scratch: OMM_ERR_SCRATCH, found on the host before any launch."""
    L = om.lib()
    M, N, K = 16, 8176, 131328
    A, B, Y = T((M, K), BF16), T((N, K), BF16), T((M, N), BF16)
    assert 65 * M * N * 4 > 32 * 1024 * 1024
    assert L.omm_gemm_noalloc(ctypes.byref(A), ctypes.byref(B), None, 1.0, 0.0, 0, 1, ctypes.byref(Y), None) == -8
    assert "scratch" in om.status_string(-8)
    # argument errors come first, as for omm_gemm
    assert L.omm_gemm_noalloc(None, ctypes.byref(B), None, 1.0, 0.0, 0, 1, ctypes.byref(Y), None) == -1
    assert L.omm_gemm_noalloc(ctypes.byref(A), ctypes.byref(B), None, 1.0, 0.0, 0, 0, ctypes.byref(Y), None) == -3


@pytest.mark.parametrize("cshape,ok", [((), True), ((1,), True), ((5,), True), ((1, 5), True), ((4, 1), True),
                                       ((4, 5), True), ((4,), False), ((5, 4), False), ((1, 4, 5), False)])
def test_gemm_c_forms(cshape, ok):
    L = om.lib()
    A, B, Y = T((4, 8), F32), T((8, 5), F32), T((4, 5), F32)
    rc = L.omm_gemm(ctypes.byref(A), ctypes.byref(B), ctypes.byref(T(cshape, F32)), 1.0, 1.0, 0, 0,
                    ctypes.byref(T((4, 6), F32)), None)
    assert rc == -3  # a wrong Y shape fails before C is looked at
    if not ok:  # valid C forms would launch: only the rejected ones are called here
        rc = L.omm_gemm(ctypes.byref(A), ctypes.byref(B), ctypes.byref(T(cshape, F32)), 1.0, 1.0, 0, 0,
                        ctypes.byref(Y), None)
        assert rc == -4


@pytest.mark.parametrize("tA,tB,sa,sb,exp", [(0, 0, (3, 4), (4, 5), (3, 5)), (1, 0, (4, 3), (4, 5), (3, 5)),
                                             (0, 1, (3, 4), (5, 4), (3, 5)), (1, 1, (4, 3), (5, 4), (3, 5))])
def test_gemm_output_shape(tA, tB, sa, sb, exp):
    L = om.lib()
    rc, sh = out_shape(L.omm_gemm_output_shape, ctypes.byref(T(sa, F32)), ctypes.byref(T(sb, F32)), tA, tB)
    assert rc == 0 and sh == exp
    rc, _ = out_shape(L.omm_gemm_output_shape, ctypes.byref(T(sa, F32)), ctypes.byref(T(sb, F32)), 1 - tA, tB)
    assert rc == -3


def test_qlinear_argument_errors():
    L = om.lib()
    a, b, y = T((4, 8), I8), T((8, 5), I8), T((4, 5), I8)
    s1, z1 = T((), F32), T((), I8)
    args = lambda **kw: [ctypes.byref(kw.get(k, d)) for k, d in
                         (("a", a), ("as_", s1), ("az", z1), ("b", b), ("bs", s1), ("bz", z1),
                          ("ys", s1), ("yz", z1), ("y", y))]
    assert L.omm_qlinear_matmul(*args(a=T((4, 8), F32)), None) == -2          # a not 8-bit
    assert L.omm_qlinear_matmul(*args(az=T((), U8)), None) == -2             # zp dtype != a dtype
    assert L.omm_qlinear_matmul(*args(y=T((4, 5), U8)), None) == -2          # y dtype != y_zp dtype
    assert L.omm_qlinear_matmul(*args(as_=T((), F16)), None) == -2           # scales of mixed dtypes
    assert L.omm_qlinear_matmul(*args(as_=T((), BF16), bs=T((), BF16), ys=T((), BF16)), None) == -2
    assert L.omm_qlinear_matmul(*args(as_=T((4,), F32)), None) == -4         # scale / zp shapes differ
    assert L.omm_qlinear_matmul(*args(as_=T((5,), F32), az=T((5,), I8)), None) == -4   # not M
    assert L.omm_qlinear_matmul(*args(bs=T((1, 4), F32), bz=T((1, 4), I8)), None) == -4  # not N
    assert L.omm_qlinear_matmul(*args(ys=T((2,), F32)), None) == -5          # y_scale must be one element
    assert L.omm_qlinear_matmul(*args(y=T((4, 4), I8)), None) == -3
    assert L.omm_qlinear_matmul(*args(a=T((0, 8), I8), y=T((0, 5), I8)), None) == 0  # empty


def test_grouped_argument_errors():
    L = om.lib()
    inp, w, idx, out = T((6, 8), BF16), T((3, 8, 5), BF16), T((6, 2), I32), T((6, 2, 5), BF16)
    rc, sh = out_shape(L.omm_grouped_matmul_output_shape, ctypes.byref(inp), ctypes.byref(w), ctypes.byref(idx))
    assert rc == 0 and sh == (6, 2, 5)
    ws = L.omm_grouped_matmul_workspace_size(6, 2, 3)
    assert ws > 0 and ws % 256 == 0
    assert L.omm_grouped_matmul_workspace_size(16384, 8, 64) >= 4 * 16384 * 8
    call = lambda **kw: L.omm_grouped_matmul(
        ctypes.byref(kw.get("inp", inp)), ctypes.byref(kw.get("w", w)), ctypes.byref(kw.get("idx", idx)),
        kw.get("bias", None), ctypes.byref(kw.get("out", out)), kw.get("ws", FAKE), kw.get("wsb", ws), None)
    assert call(idx=T((6, 2), F32)) == -2
    assert call(w=T((3, 8, 5), F16)) == -2
    assert call(w=T((3, 7, 5), BF16)) == -3
    assert call(idx=T((5, 2), I32)) == -3
    assert call(out=T((6, 2, 4), BF16)) == -3
    assert call(bias=ctypes.byref(T((3, 4), BF16))) == -3
    assert call(ws=None) == -6
    assert call(wsb=ws - 1) == -6
    assert call(ws=FAKE + 8) == -6  # not 256-byte aligned
    assert L.omm_grouped_matmul_check(None, None, ctypes.byref(ctypes.c_int64())) == -1


def test_grouped_dequant_argument_errors():
    L = om.lib()
    inp, q, idx, out = T((6, 8), BF16), T((3, 8, 5), I8), T((6, 2), I32), T((6, 2, 5), BF16)
    sc, zp = T((3, 2, 5), BF16), T((3, 2, 5), I8)  # block_size 4 -> 2 blocks along K = 8
    ws = L.omm_grouped_matmul_workspace_size(6, 2, 3)
    call = lambda **kw: L.omm_grouped_matmul_dequant(
        ctypes.byref(kw.get("inp", inp)), ctypes.byref(kw.get("q", q)), ctypes.byref(kw.get("sc", sc)),
        kw.get("zp", ctypes.byref(zp)), kw.get("bs", 4), ctypes.byref(kw.get("idx", idx)), kw.get("bias", None),
        ctypes.byref(kw.get("out", out)), kw.get("ws", FAKE), kw.get("wsb", ws), None)
    assert call(q=T((3, 8, 5), BF16)) == -2          # weights must be int8 / uint8
    assert call(sc=T((3, 2, 5), F16)) == -2          # scale of the input's type
    assert call(zp=ctypes.byref(T((3, 2, 5), U8))) == -2  # zero point of the weights' type
    assert call(out=T((6, 2, 5), F16)) == -2
    assert call(bs=0) == -3
    assert call(bs=3) == -3                          # ceil(8 / 3) = 3 blocks, scale has 2
    assert call(sc=T((3, 1, 5), BF16)) == -3
    assert call(zp=ctypes.byref(T((3, 2, 4), I8))) == -3
    assert call(q=T((3, 7, 5), I8)) == -3
    assert call(bias=ctypes.byref(T((3, 4), BF16))) == -3
    assert call(inp=T((6, 8), I8), q=T((3, 8, 5), I8)) == -2
    assert call(ws=None) == -6
    assert call(sc=T((3, 2, 5), F64), inp=T((6, 8), F64), out=T((6, 2, 5), F64)) == -5


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        om.describe(torch.zeros(3, 3))
