"""Python handle on the plain-C CPU oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product library never does.
It shares no code with the GPU path.  Inputs are numpy arrays; bfloat16 data
is passed as uint16 bit patterns together with ``dt="bf16"``.

Every function returns the oracle's exact-definition result: float operators
give the unrounded fp64 value ``y`` and ``t = sum_k |a*b|`` (used for the
tolerance), QLinearMatMul gives the quantised output and the int32 accumulator.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# OMM_ORACLE_LIB lets the mutation tests load a deliberately broken build
LIB = os.environ.get("OMM_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "oracle.c")

F32, F16, BF16, F64, I8, U8, I32, I64 = range(8)
_CODES = {"f32": F32, "f16": F16, "bf16": BF16, "f64": F64, "i8": I8, "u8": U8, "i32": I32, "i64": I64}
_NP = {np.dtype(np.float32): F32, np.dtype(np.float16): F16, np.dtype(np.float64): F64,
       np.dtype(np.int8): I8, np.dtype(np.uint8): U8, np.dtype(np.int32): I32, np.dtype(np.int64): I64}
_ERR = {-1: "shape mismatch", -2: "not broadcastable", -3: "unsupported dtype", -4: "index outside [0, G)"}


class OracleError(ValueError):
    def __init__(self, code):
        super().__init__("oracle: %s (%d)" % (_ERR.get(code, "error"), code))
        self.code = code


def build(verbose=False):
    """Compile oracle.c -> liboracle.so (plain gcc, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(LIB + ".tmp", LIB)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        vp, i64p, dp, ip = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)
        ci, cl, cf = ctypes.c_int, ctypes.c_int64, ctypes.c_float
        L.orc_matmul_shape.argtypes = [ci, i64p, ci, i64p, ip, i64p]
        L.orc_matmul.argtypes = [vp, ci, ci, i64p, vp, ci, i64p, cl, i64p, dp, dp, ci]
        L.orc_gemm.argtypes = [vp, i64p, vp, i64p, vp, ci, i64p, ci, cf, cf, ci, ci, cl, i64p, dp, dp, ci]
        L.orc_qlinear_matmul.argtypes = [vp, ci, ci, i64p, vp, ci, vp, ci, i64p,
                                         vp, ci, ci, i64p, vp, ci, vp, ci, i64p,
                                         vp, ci, vp, ci, cl, i64p, vp, vp, ci]
        L.orc_grouped_matmul.argtypes = [vp, vp, vp, ci, vp, ci, cl, cl, cl, cl, cl, cl, i64p, dp, dp, ci]
        L.orc_grouped_matmul_dq.argtypes = [vp, vp, ci, vp, vp, cl, vp, ci, vp, ci, cl, cl, cl, cl, cl, cl, i64p,
                                            dp, dp, ci]
        L.orc_round.argtypes = [ci, ctypes.c_double]
        L.orc_round.restype = ctypes.c_double
        L.orc_decode.argtypes = [ci, vp, cl]
        L.orc_decode.restype = ctypes.c_double
        _lib = L
    return _lib


def threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, n)


def _code(arr, dt):
    if dt is not None:
        return _CODES[dt]
    try:
        return _NP[arr.dtype]
    except KeyError:
        raise TypeError("oracle: pass dt= for numpy dtype %s" % arr.dtype)


def _shape(arr):
    sh = (ctypes.c_int64 * max(1, arr.ndim))(*arr.shape)
    return sh


def _ptr(arr):
    return ctypes.c_void_p(arr.ctypes.data) if arr is not None else None


def _sel(sel):
    if sel is None:
        return None, 0, None
    s = np.ascontiguousarray(sel, dtype=np.int64).ravel()
    return s, s.size, s.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def matmul_shape(a_shape, b_shape):
    L = lib()
    y_nd = ctypes.c_int(0)
    ysh = (ctypes.c_int64 * 8)()
    a = (ctypes.c_int64 * max(1, len(a_shape)))(*a_shape)
    b = (ctypes.c_int64 * max(1, len(b_shape)))(*b_shape)
    r = L.orc_matmul_shape(len(a_shape), a, len(b_shape), b, ctypes.byref(y_nd), ysh)
    if r:
        raise OracleError(r)
    return tuple(ysh[i] for i in range(y_nd.value))


def matmul(A, B, dt=None, sel=None, nthreads=None):
    """MatMul (numpy.matmul semantics). Returns (y, t) in float64."""
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    code = _code(A, dt)
    yshape = matmul_shape(A.shape, B.shape)
    s, ns, sp = _sel(sel)
    cnt = ns if s is not None else int(np.prod(yshape, dtype=np.int64))
    y = np.empty(cnt, np.float64)
    t = np.empty(cnt, np.float64)
    r = lib().orc_matmul(_ptr(A), code, A.ndim, _shape(A), _ptr(B), B.ndim, _shape(B),
                         ns, sp, _ptr(y), _ptr(t), nthreads or threads())
    if r:
        raise OracleError(r)
    if s is None:
        return y.reshape(yshape), t.reshape(yshape)
    return y, t


def gemm(A, B, C=None, alpha=1.0, beta=1.0, transA=0, transB=0, dt=None, sel=None, nthreads=None):
    """Gemm: alpha*A'B' + beta*C. Returns (y, t) in float64, shape (M, N)."""
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    if A.ndim != 2 or B.ndim != 2:
        raise OracleError(-1)
    code = _code(A, dt)
    M = A.shape[1] if transA else A.shape[0]
    N = B.shape[0] if transB else B.shape[1]
    if C is not None:
        C = np.ascontiguousarray(C)
    s, ns, sp = _sel(sel)
    cnt = ns if s is not None else M * N
    y = np.empty(cnt, np.float64)
    t = np.empty(cnt, np.float64)
    r = lib().orc_gemm(_ptr(A), _shape(A), _ptr(B), _shape(B), _ptr(C),
                       C.ndim if C is not None else 0, _shape(C) if C is not None else None,
                       code, float(alpha), float(beta), int(bool(transA)), int(bool(transB)),
                       ns, sp, _ptr(y), _ptr(t), nthreads or threads())
    if r:
        raise OracleError(r)
    if s is None:
        return y.reshape(M, N), t.reshape(M, N)
    return y, t


def qlinear_matmul(a, a_scale, a_zero_point, b, b_scale, b_zero_point, y_scale, y_zero_point,
                   sel=None, nthreads=None):
    """QLinearMatMul. Returns (y, acc32): y in y_zero_point's dtype, acc32 int32."""
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    a_scale, b_scale, y_scale = (np.ascontiguousarray(x) for x in (a_scale, b_scale, y_scale))
    a_zero_point, b_zero_point, y_zero_point = (np.ascontiguousarray(x) for x in
                                                (a_zero_point, b_zero_point, y_zero_point))
    if a_scale.shape != a_zero_point.shape or b_scale.shape != b_zero_point.shape:
        raise OracleError(-2)
    if a_zero_point.dtype != a.dtype or b_zero_point.dtype != b.dtype:
        raise OracleError(-3)
    yshape = matmul_shape(a.shape, b.shape)
    s, ns, sp = _sel(sel)
    cnt = ns if s is not None else int(np.prod(yshape, dtype=np.int64))
    y = np.empty(cnt, y_zero_point.dtype)
    acc = np.empty(cnt, np.int32)
    r = lib().orc_qlinear_matmul(
        _ptr(a), _code(a, None), a.ndim, _shape(a),
        _ptr(a_scale), _code(a_scale, None), _ptr(a_zero_point), a_scale.ndim, _shape(a_scale),
        _ptr(b), _code(b, None), b.ndim, _shape(b),
        _ptr(b_scale), _code(b_scale, None), _ptr(b_zero_point), b_scale.ndim, _shape(b_scale),
        _ptr(y_scale), _code(y_scale, None), _ptr(y_zero_point), _code(y_zero_point, None),
        ns, sp, _ptr(y), _ptr(acc), nthreads or threads())
    if r:
        raise OracleError(r)
    if s is None:
        return y.reshape(yshape), acc.reshape(yshape)
    return y, acc


def grouped_matmul(inp, weights, group_indices, bias=None, dt=None, sel=None, nthreads=None):
    """GroupedMatMul. Returns (y, t) in float64, shape (M, S, N)."""
    inp, weights = np.ascontiguousarray(inp), np.ascontiguousarray(weights)
    idx = np.ascontiguousarray(group_indices)
    if bias is not None:
        bias = np.ascontiguousarray(bias)
    M, K = inp.shape
    G, K2, N = weights.shape
    M2, S = idx.shape
    if K2 != K or M2 != M or (bias is not None and bias.shape != (G, N)):
        raise OracleError(-1)
    s, ns, sp = _sel(sel)
    cnt = ns if s is not None else M * S * N
    y = np.empty(cnt, np.float64)
    t = np.empty(cnt, np.float64)
    r = lib().orc_grouped_matmul(_ptr(inp), _ptr(weights), _ptr(idx), _code(idx, None), _ptr(bias),
                                 _code(inp, dt), M, K, G, N, S, ns, sp, _ptr(y), _ptr(t),
                                 nthreads or threads())
    if r:
        raise OracleError(r)
    if s is None:
        return y.reshape(M, S, N), t.reshape(M, S, N)
    return y, t


def grouped_matmul_dequant(inp, qweights, scale, zero_point, block_size, group_indices, bias=None, dt=None,
                           sel=None, nthreads=None):
    """GroupedMatMul over DequantizeLinear weights (blocked along K, per column).

    qweights (G, K, N) int8/uint8; scale (G, ceil(K/bs), N) of the float type;
    zero_point None or like scale with qweights' dtype.  Returns (y, t) in
    float64, shape (M, S, N)."""
    inp, qw = np.ascontiguousarray(inp), np.ascontiguousarray(qweights)
    scale = np.ascontiguousarray(scale)
    idx = np.ascontiguousarray(group_indices)
    zp = None if zero_point is None else np.ascontiguousarray(zero_point)
    if bias is not None:
        bias = np.ascontiguousarray(bias)
    M, K = inp.shape
    G, K2, N = qw.shape
    M2, S = idx.shape
    nkb = (K + block_size - 1) // block_size if block_size > 0 else -1
    if (K2 != K or M2 != M or scale.shape != (G, nkb, N) or (zp is not None and zp.shape != scale.shape)
            or (zp is not None and zp.dtype != qw.dtype) or (bias is not None and bias.shape != (G, N))):
        raise OracleError(-1)
    s, ns, sp = _sel(sel)
    cnt = ns if s is not None else M * S * N
    y = np.empty(cnt, np.float64)
    t = np.empty(cnt, np.float64)
    r = lib().orc_grouped_matmul_dq(_ptr(inp), _ptr(qw), _code(qw, None), _ptr(scale), _ptr(zp), block_size,
                                    _ptr(idx), _code(idx, None), _ptr(bias), _code(inp, dt), M, K, G, N, S, ns, sp,
                                    _ptr(y), _ptr(t), nthreads or threads())
    if r:
        raise OracleError(r)
    if s is None:
        return y.reshape(M, S, N), t.reshape(M, S, N)
    return y, t


def round_to(values, dt):
    """The oracle's own rounding of real values to float type dt (nearest, ties to even)."""
    L = lib()
    return np.array([L.orc_round(_CODES[dt], float(v)) for v in np.ravel(values)])


def decode(arr, dt):
    """The oracle's own element decoder (fp16 / bf16 / fp32 / fp64 -> double)."""
    arr = np.ascontiguousarray(arr)
    L = lib()
    return np.array([L.orc_decode(_CODES[dt], _ptr(arr), i) for i in range(arr.size)])
