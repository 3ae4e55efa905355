"""The CPU oracle against the worked examples printed on the operator pages.

Fixtures under tests/golden/ were transcribed from the pages by
tests/golden/extract_examples.py; each example carries its citation (page
title and example name).  The printed float values are numpy's shortest
round-trip representation of the fp32 result, so the tolerance is the fp32
bound 1e-5 * sum_k|a*b| + 1e-6 plus half a unit in the last printed digit.
"""
import numpy as np
import pytest

import oracle

NP_DT = {"float32": np.float32, "float16": np.float16, "float64": np.float64,
         "int8": np.int8, "uint8": np.uint8, "int32": np.int32, "int64": np.int64}


def arr(field):
    return np.array(field["text"], dtype=NP_DT[field["dtype"]]).reshape(field["shape"])


def printed_half_ulp(tok):
    mant, _, exp = tok.lower().partition("e")
    dec = len(mant.split(".")[1]) if "." in mant else 0
    e = int(exp) if exp else 0
    return 0.5 * 10.0 ** (-(dec - e))


def half_ulps(field):
    return np.array([printed_half_ulp(t) for t in field["text"]]).reshape(field["shape"])


def ids(exs):
    return [e["name"] for e in exs]


def _load(name):
    import json
    import os
    p = os.path.join(os.path.dirname(__file__), "golden", name + "_examples.json")
    with open(p) as f:
        return json.load(f)["examples"]


MATMUL = _load("matmul")
GEMM = _load("gemm")
QLIN = _load("qlinearmatmul")
GROUPED = _load("groupedmatmul")


def test_fixture_counts():
    assert (len(MATMUL), len(GEMM), len(QLIN), len(GROUPED)) == (9, 12, 12, 8)


@pytest.mark.parametrize("ex", MATMUL, ids=ids(MATMUL))
def test_matmul_printed(ex):
    A, B = arr(ex["inputs"]["A"]), arr(ex["inputs"]["B"])
    Yf = ex["outputs"]["Y"]
    y, t = oracle.matmul(A, B)
    assert list(y.shape) == Yf["shape"], ex["cite"]
    exp = arr(Yf).astype(np.float64)
    tol = 1e-5 * t + 1e-6 + half_ulps(Yf)
    assert np.all(np.abs(y - exp) <= tol), (ex["cite"], np.max(np.abs(y - exp)))


@pytest.mark.parametrize("ex", GEMM, ids=ids(GEMM))
def test_gemm_printed(ex):
    ins = ex["inputs"]
    at = ex["attrs"]
    # attribute defaults where an example does not set them: alpha=beta=1, trans=0
    alpha = float(at.get("alpha", "1.0"))
    beta = float(at.get("beta", "1.0"))
    tA, tB = int(at.get("transA", "0")), int(at.get("transB", "0"))
    A, B = arr(ins["A"]), arr(ins["B"])
    C = arr(ins["C"]) if "C" in ins else None
    Yf = ex["outputs"]["Y"]
    y, t = oracle.gemm(A, B, C, alpha, beta, tA, tB)
    assert list(y.shape) == Yf["shape"], ex["cite"]
    exp = arr(Yf).astype(np.float64)
    cmag = abs(beta) * np.abs(np.broadcast_to(C, y.shape)) if C is not None else 0.0
    tol = 1e-5 * (abs(alpha) * t + cmag) + 1e-6 + half_ulps(Yf)
    assert np.all(np.abs(y - exp) <= tol), (ex["cite"], np.max(np.abs(y - exp)))


def test_gemm_defaults_are_needed():
    """The examples fix alpha=beta=1 (not 0) when unset: beta=0 would fail matrix_bias."""
    ex = [e for e in GEMM if e["name"] == "test_cc_gemm_default_matrix_bias"][0]
    A, B, C = (arr(ex["inputs"][k]) for k in "ABC")
    y0, _ = oracle.gemm(A, B, C, 1.0, 0.0)
    assert np.max(np.abs(y0 - arr(ex["outputs"]["Y"]))) > 0.1


@pytest.mark.parametrize("ex", QLIN, ids=ids(QLIN))
def test_qlinear_printed(ex):
    i = ex["inputs"]
    y, acc = oracle.qlinear_matmul(arr(i["a"]), arr(i["a_scale"]), arr(i["a_zero_point"]),
                                   arr(i["b"]), arr(i["b_scale"]), arr(i["b_zero_point"]),
                                   arr(i["y_scale"]), arr(i["y_zero_point"]))
    exp = arr(ex["outputs"]["y"])
    assert y.dtype == exp.dtype and y.shape == exp.shape, ex["cite"]
    assert np.array_equal(y, exp), (ex["cite"], y, exp)


def _grouped_inputs(ex, T=None, Tind=None):
    def mk(f, dflt):
        dt = f["dtype"]
        dt = {"T": T, "Tind": Tind}.get(dt, dt) or dflt
        if f["values"] == "arange":
            v = np.arange(f["count"])
        else:
            v = np.array(f["values"], dtype=np.float64)
        return v.astype(NP_DT[dt]).reshape(f["shape"])
    ins = ex["inputs"]
    inp = mk(ins["input"], "float32")
    w = mk(ins["weights"], "float32")
    idx = mk(ins["group_indices"], "int64")
    bias = mk(ins["bias"], "float32") if ("bias" in ins and "bias" in ex["node_inputs"]) else None
    return inp, w, idx, bias


# Outputs worked by hand from output[m, i] = input[m] @ weights[g] (+ bias[g]),
# g = group_indices[m, i]; the page computes them with a helper it does not print.
HAND = {
    "default": [[[2, 0]], [[1, 2]], [[1, 1]], [[0, 1]]],
    "_without_bias_explicit_empty_input": [[[2, 0]], [[1, 2]], [[1, 1]], [[0, 1]]],
    "_with_bias": [[[1.1, 0.2], [0.3, 1.0]], [[0.5, 0.5], [0.1, 1.2]]],
    "_additional_types": [[[1.5, 3.0], [3.5, 3.0]], [[5.5, 5.0], [3.5, 5.0]]],
    "_single_group": [[[9, 12, 15]], [[19, 26, 33]], [[29, 40, 51]]],
    "_with_unused_group": [[[4, 7]], [[8, 15]], [[100, 111]], [[136, 151]]],
}


def _grouped_cases():
    out = []
    for ex in GROUPED:
        for T in ex.get("T_values", [None]):
            for Tind in ex.get("Tind_values", [None]):
                out.append(pytest.param(ex, T, Tind, id="%s-%s-%s" % (ex["name"], T, Tind)))
    return out


@pytest.mark.parametrize("ex,T,Tind", _grouped_cases())
def test_grouped_examples(ex, T, Tind):
    inp, w, idx, bias = _grouped_inputs(ex, T, Tind)
    M, S = idx.shape
    G, K, N = w.shape
    y, t = oracle.grouped_matmul(inp, w, idx, bias)
    assert y.shape == (M, S, N), ex["cite"]
    # the decomposition the page names: Gather the selected weights, then MatMul
    sel = w.astype(np.float64)[idx.reshape(-1)].reshape(M, S, K, N)
    dec = np.matmul(inp.astype(np.float64)[:, None, None, :], sel)[:, :, 0, :]
    if bias is not None:
        dec = dec + bias.astype(np.float64)[idx]
    assert np.allclose(y, dec, rtol=0, atol=1e-12), ex["cite"]
    if ex["name"] in HAND:
        hb = np.array(HAND[ex["name"]], dtype=np.float64)
        # bias values are stored in T: compare against the stored bias, not the decimal
        tol = 1e-3 if T == "float16" else 1e-6
        assert np.allclose(y, hb, rtol=0, atol=tol), (ex["cite"], y, hb)
