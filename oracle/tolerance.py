"""The parity criterion between a GPU result and the oracle (test infrastructure).

With y the oracle's unrounded fp64 value and t = sum_k |a_ik * b_kj|:
  fp32 outputs:        |y_gpu - y| <= 1e-5 * t + 1e-6
  bf16 / fp16 outputs: |y_gpu - y| <= 1e-2 * t + 1e-3
  fp64 outputs (no bound is stated for them): the GPU sums the same products
  in another order, each fp64 operation off by at most 2^-53 relative, so
  |err| <= K * 2^-53 * t, under 1e-12 * t for every K tested (K <= 4096).
Integer results (QLinearMatMul, int32 accumulators) compare exactly.
"""
import numpy as np

TOL = {"f32": (1e-5, 1e-6), "bf16": (1e-2, 1e-3), "f16": (1e-2, 1e-3), "f64": (1e-12, 1e-300)}


def check_close(got, y, t, dt, what=""):
    """Assert |got - y| <= rtol * t + atol elementwise; report the worst offender."""
    rt, at = TOL[dt]
    got = np.asarray(got, np.float64).ravel()
    y = np.asarray(y, np.float64).ravel()
    t = np.asarray(t, np.float64).ravel()
    assert got.shape == y.shape, (what, got.shape, y.shape)
    err = np.abs(got - y)
    tol = rt * t + at
    bad = ~(err <= tol)  # NaN counts as bad
    if bad.any():
        i = int(np.argmax(np.where(bad, err / tol, 0)))
        raise AssertionError("%s: %d / %d outside tolerance; worst at %d: got %r want %r (t=%r, tol=%r)"
                             % (what, int(bad.sum()), bad.size, i, got[i], y[i], t[i], tol[i]))
