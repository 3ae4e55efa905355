"""ONNX MatMul-family operators for AMD Instinct MI355X (gfx950).

MatMul, Gemm, QLinearMatMul and GroupedMatMul as hand-written HIP kernels
behind the C ABI in include/omm.h (libomm.so); this package is the thin
Python binding (`_omm`), the build step (`build`) and the seeded input
generators (`synth`).  The binding is imported lazily so that the generators
and the build step work on machines without a GPU.
"""

_BINDING = ("matmul", "gemm", "gemm_noalloc", "qlinear_matmul", "grouped_matmul", "grouped_matmul_dequant",
            "grouped_matmul_check", "grouped_matmul_workspace_size", "describe", "lib", "status_string", "OmmError",
            "OmmTensor")


def __getattr__(name):
    if name in _BINDING:
        from . import _omm
        return getattr(_omm, name)
    raise AttributeError(name)
