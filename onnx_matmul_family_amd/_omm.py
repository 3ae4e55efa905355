"""Thin ctypes binding of libomm.so (include/omm.h): argument marshalling only.

Each function takes torch tensors that already live on the GPU, describes them
to the C ABI (pointer, dtype, shape) and enqueues the call on torch's current
stream.  Outputs that are not passed in are allocated with torch at the shape
the library reports.  Every computation happens in the library's HIP kernels;
there is no fallback: if libomm.so is missing or a tensor is not a contiguous
GPU tensor, the call raises.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# OMM_LIB names another build of the same library (the sanitizer build of the host code)
LIB_PATH = os.environ.get("OMM_LIB") or os.path.join(HERE, "libomm.so")

MAX_DIMS = 8
_DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.float64: 3,
       torch.int8: 4, torch.uint8: 5, torch.int32: 6, torch.int64: 7}
_TORCH = {v: k for k, v in _DT.items()}


class OmmTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * MAX_DIMS)]


class OmmError(RuntimeError):
    def __init__(self, code, what):
        self.code = code
        super().__init__("%s: %s (status %d)" % (what, status_string(code), code))


_lib = None


def lib():
    """The loaded libomm.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libomm.so is not built (run: python -m onnx_matmul_family_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(OmmTensor)
        vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        i32p, i64p = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
        L.omm_status_string.restype = ctypes.c_char_p
        L.omm_status_string.argtypes = [ci]
        L.omm_version.restype = ci
        L.omm_matmul_output_shape.argtypes = [P, P, i32p, i64p]
        L.omm_matmul.argtypes = [P, P, P, vp]
        L.omm_gemm_output_shape.argtypes = [P, P, ci, ci, i32p, i64p]
        L.omm_gemm.argtypes = [P, P, P, cf, cf, ci, ci, P, vp]
        L.omm_gemm_noalloc.argtypes = [P, P, P, cf, cf, ci, ci, P, vp]
        L.omm_qlinear_matmul_output_shape.argtypes = [P, P, i32p, i64p]
        L.omm_qlinear_matmul.argtypes = [P, P, P, P, P, P, P, P, P, vp]
        L.omm_grouped_matmul_workspace_size.restype = ctypes.c_size_t
        L.omm_grouped_matmul_workspace_size.argtypes = [ctypes.c_int64] * 3
        L.omm_grouped_matmul_output_shape.argtypes = [P, P, P, i32p, i64p]
        L.omm_grouped_matmul.argtypes = [P, P, P, P, P, vp, ctypes.c_size_t, vp]
        L.omm_grouped_matmul_check.argtypes = [vp, vp, i64p]
        L.omm_grouped_matmul_dequant.argtypes = [P, P, P, P, ctypes.c_int64, P, P, P, vp, ctypes.c_size_t, vp]
        _lib = L
    return _lib


def status_string(code):
    return lib().omm_status_string(int(code)).decode()


def describe(x):
    """omm_tensor for a contiguous GPU tensor (shape and dtype only, no copy)."""
    if not isinstance(x, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not x.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not x.is_contiguous():
        raise ValueError("tensor must be contiguous (row-major)")
    if x.dim() > MAX_DIMS:
        raise ValueError("at most %d dims" % MAX_DIMS)
    t = OmmTensor()
    t.data = x.data_ptr() if x.numel() > 0 else 0
    t.dtype = _DT[x.dtype]
    t.ndim = x.dim()
    for i, s in enumerate(x.shape):
        t.shape[i] = s
    return t


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _shape(fn, *args):
    nd = ctypes.c_int32(0)
    sh = (ctypes.c_int64 * MAX_DIMS)()
    rc = fn(*args, ctypes.byref(nd), sh)
    if rc:
        raise OmmError(rc, fn.__name__)
    return tuple(sh[i] for i in range(nd.value))


def _check(rc, what):
    if rc:
        raise OmmError(rc, what)


def matmul(A, B, Y=None, stream=None):
    """MatMul: numpy.matmul semantics (bf16 / fp16 / fp32)."""
    L = lib()
    tA, tB = describe(A), describe(B)
    if Y is None:
        Y = torch.empty(_shape(L.omm_matmul_output_shape, ctypes.byref(tA), ctypes.byref(tB)),
                        dtype=A.dtype, device=A.device)
    tY = describe(Y)
    _check(L.omm_matmul(ctypes.byref(tA), ctypes.byref(tB), ctypes.byref(tY), _stream(stream)), "omm_matmul")
    return Y


def gemm(A, B, C=None, alpha=1.0, beta=1.0, transA=0, transB=0, Y=None, stream=None):
    """Gemm: Y = alpha * A' B' + beta * C."""
    L = lib()
    tA, tB = describe(A), describe(B)
    if Y is None:
        Y = torch.empty(_shape(L.omm_gemm_output_shape, ctypes.byref(tA), ctypes.byref(tB), int(transA),
                               int(transB)), dtype=A.dtype, device=A.device)
    tY = describe(Y)
    pC = ctypes.byref(describe(C)) if C is not None else None
    _check(L.omm_gemm(ctypes.byref(tA), ctypes.byref(tB), pC, float(alpha), float(beta), int(transA), int(transB),
                      ctypes.byref(tY), _stream(stream)), "omm_gemm")
    return Y


def gemm_noalloc(A, B, C, alpha, beta, transA, transB, Y, stream=None):
    """Gemm into a preallocated Y through omm_gemm_noalloc: the library
    allocates nothing (split-K partials in its static per-GPU scratch)."""
    L = lib()
    tA, tB, tY = describe(A), describe(B), describe(Y)
    pC = ctypes.byref(describe(C)) if C is not None else None
    _check(L.omm_gemm_noalloc(ctypes.byref(tA), ctypes.byref(tB), pC, float(alpha), float(beta), int(transA),
                              int(transB), ctypes.byref(tY), _stream(stream)), "omm_gemm_noalloc")
    return Y


def qlinear_matmul(a, a_scale, a_zero_point, b, b_scale, b_zero_point, y_scale, y_zero_point, y=None, stream=None):
    """QLinearMatMul: int8/uint8 in, int8/uint8 out (y_zero_point's dtype)."""
    L = lib()
    ts = [describe(x) for x in (a, a_scale, a_zero_point, b, b_scale, b_zero_point, y_scale, y_zero_point)]
    if y is None:
        y = torch.empty(_shape(L.omm_qlinear_matmul_output_shape, ctypes.byref(ts[0]), ctypes.byref(ts[3])),
                        dtype=y_zero_point.dtype, device=a.device)
    ty = describe(y)
    _check(L.omm_qlinear_matmul(*[ctypes.byref(t) for t in ts], ctypes.byref(ty), _stream(stream)),
           "omm_qlinear_matmul")
    return y


def grouped_matmul_workspace_size(M, S, G):
    return int(lib().omm_grouped_matmul_workspace_size(int(M), int(S), int(G)))


def grouped_matmul(input, weights, group_indices, bias=None, output=None, workspace=None, stream=None):
    """GroupedMatMul: output[m, i] = input[m] @ weights[group_indices[m, i]] (+ bias[g]).

    `workspace` is a uint8 GPU tensor of at least grouped_matmul_workspace_size
    bytes; one is allocated when omitted.  Returns (output, workspace)."""
    L = lib()
    ti, tw, tx = describe(input), describe(weights), describe(group_indices)
    if output is None:
        output = torch.empty(_shape(L.omm_grouped_matmul_output_shape, ctypes.byref(ti), ctypes.byref(tw),
                                    ctypes.byref(tx)), dtype=input.dtype, device=input.device)
    to = describe(output)
    M, S, G = group_indices.shape[0], group_indices.shape[1], weights.shape[0]
    need = grouped_matmul_workspace_size(M, S, G)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=input.device)
    pb = ctypes.byref(describe(bias)) if bias is not None else None
    _check(L.omm_grouped_matmul(ctypes.byref(ti), ctypes.byref(tw), ctypes.byref(tx), pb, ctypes.byref(to),
                                ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(stream)),
           "omm_grouped_matmul")
    return output, workspace


def grouped_matmul_dequant(input, qweights, w_scale, w_zero_point, block_size, group_indices, bias=None,
                           output=None, workspace=None, stream=None):
    """GroupedMatMul over DequantizeLinear(qweights, w_scale, w_zero_point) blocked along K:
    w[g, k, n] = T((q - zp) * scale) with the scale / zero point of block k // block_size.
    Returns (output, workspace)."""
    L = lib()
    ti, tq, tx, ts = describe(input), describe(qweights), describe(group_indices), describe(w_scale)
    if output is None:
        output = torch.empty(_shape(L.omm_grouped_matmul_output_shape, ctypes.byref(ti), ctypes.byref(tq),
                                    ctypes.byref(tx)), dtype=input.dtype, device=input.device)
    to = describe(output)
    M, S, G = group_indices.shape[0], group_indices.shape[1], qweights.shape[0]
    need = grouped_matmul_workspace_size(M, S, G)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=input.device)
    pz = ctypes.byref(describe(w_zero_point)) if w_zero_point is not None else None
    pb = ctypes.byref(describe(bias)) if bias is not None else None
    _check(L.omm_grouped_matmul_dequant(ctypes.byref(ti), ctypes.byref(tq), ctypes.byref(ts), pz, int(block_size),
                                        ctypes.byref(tx), pb, ctypes.byref(to), ctypes.c_void_p(workspace.data_ptr()),
                                        workspace.numel(), _stream(stream)),
           "omm_grouped_matmul_dequant")
    return output, workspace


def grouped_matmul_check(workspace, stream=None):
    """Number of (m, i) pairs of the last grouped call on `workspace` with an index outside [0, G)."""
    n = ctypes.c_int64(0)
    _check(lib().omm_grouped_matmul_check(ctypes.c_void_p(workspace.data_ptr()), _stream(stream), ctypes.byref(n)),
           "omm_grouped_matmul_check")
    return n.value
