"""Planted mistakes in the oracle must be caught by its pins.

Each case below rewrites one plausible slip into a copy of oracle/oracle.c (a
dropped term, a flipped sign, a wrong index, a transposed operand, the wrong
rounding), builds that copy into a private library, and runs the pin suites
(printed examples + properties) against it in a fresh interpreter.  The suites
must fail for every mutant.  CPU only; nothing here touches the GPU path.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = ["tests/test_oracle_examples.py", "tests/test_oracle_properties.py", "tests/test_oracle_dequant.py"]

MUTANTS = {
    # MatMul
    "matmul_drops_last_k": ("for (int64_t k = 0; k < g.K; k++) {\n            double p",
                            "for (int64_t k = 0; k + 1 < g.K; k++) {\n            double p"),
    "matmul_b_transposed": ("orc_ldf(b, dt, bo + k * g.N + n)", "orc_ldf(b, dt, bo + n * g.K + k)"),
    "matmul_no_1d_promotion_drop": ("g->drop_m = 1;", "g->drop_m = 0;"),
    "matmul_bad_batch_broadcast": ("if (da != db && da != 1 && db != 1) return ORC_EBCAST;",
                                   "if (da != db) return ORC_EBCAST;"),
    # Gemm
    "gemm_ignores_transA": ("transA ? k * M + m : m * K + k", "m * K + k"),
    "gemm_beta_sign": ("v += (double)beta *", "v -= (double)beta *"),
    "gemm_alpha_dropped": ("double v = (double)alpha * s;", "double v = s;"),
    "gemm_c_axes_swapped": ("(cM == 1 ? 0 : m) * cN + (cN == 1 ? 0 : n)",
                            "(cN == 1 ? 0 : n) * cM + (cM == 1 ? 0 : m)"),
    # QLinearMatMul
    "qlinear_b_zero_point_sign": ("- zb);", "+ zb);"),
    "qlinear_a_zero_point_dropped": ("(orc_ldi(a, a_dt, ao + m * g.K + k) - za)", "orc_ldi(a, a_dt, ao + m * g.K + k)"),
    "qlinear_round_half_away": ("float rr = rintf(x);", "float rr = roundf(x);"),
    "qlinear_truncates": ("float rr = rintf(x);", "float rr = truncf(x);"),
    "qlinear_no_int32_wrap": ("int32_t acc_w = (int32_t)(uint32_t)(uint64_t)acc;", "double acc_w = (double)acc;"),
    "qlinear_column_param_by_row": ("bpo = n * bpn", "bpo = m * bpn"),
    "qlinear_no_upper_saturation": ("if (q > hi) q = hi;", ""),
    "qlinear_zero_point_not_added": ("int64_t q = (int64_t)rr + zy;", "int64_t q = (int64_t)rr;"),
    "qlinear_requant_in_double": ("float x = xf * mult;", "float x = (float)((double)acc_w * sa * sb / sy);"),
    "qlinear_requant_other_order": ("float mult = prod / sy;", "float mult = sa * (sb / sy);"),
    # GroupedMatMul
    "grouped_bias_dropped": ("if (bias) s += orc_ldf(bias", "if (0) s += orc_ldf(bias", "int orc_grouped_matmul(const void* input"),
    "grouped_first_selection_only": ("orc_ldi(idx, idx_dt, mi)", "orc_ldi(idx, idx_dt, m * S)", "int orc_grouped_matmul(const void* input"),
    "grouped_weights_transposed": ("(grp * K + k) * N + n", "(grp * N + n) * K + k", "int orc_grouped_matmul(const void* input"),
    "grouped_bias_of_group_zero": ("orc_ldf(bias, dt, grp * N + n)", "orc_ldf(bias, dt, n)", "int orc_grouped_matmul(const void* input"),
    # GroupedMatMul over DequantizeLinear weights
    "dq_bias_dropped": ("if (bias) s += orc_ldf(bias", "if (0) s += orc_ldf(bias", "int orc_grouped_matmul_dq("),
    "dq_first_selection_only": ("orc_ldi(idx, idx_dt, mi)", "orc_ldi(idx, idx_dt, m * S)", "int orc_grouped_matmul_dq("),
    "dq_zero_point_dropped": ("double z = zp ? (double)orc_ldi(zp, q_dt, po) : 0.0;", "double z = 0.0;"),
    "dq_zero_point_added": ("orc_round_to((q - z) *", "orc_round_to((q + z) *"),
    "dq_block_index_wraps": ("int64_t po = (grp * nkb + k / bs) * N + n;", "int64_t po = (grp * nkb + k % nkb) * N + n;"),
    "dq_scale_n_major": ("int64_t po = (grp * nkb + k / bs) * N + n;", "int64_t po = (grp * N + n) * nkb + k / bs;"),
    "dq_weights_transposed": ("orc_ldi(qw, q_dt, (grp * K + k) * N + n)", "orc_ldi(qw, q_dt, (grp * N + n) * K + k)"),
    "dq_weight_not_rounded": ("double w = orc_round_to((q - z) * orc_ldf(scale, dt, po), dt);",
                              "double w = (q - z) * orc_ldf(scale, dt, po);"),
    "round_ties_away": ("nearbyint(v / ulp)", "round(v / ulp)"),
    "round_no_subnormal_spacing": ("if (ue < emin) ue = emin;", ""),
    "round_no_overflow": ("if (fabs(r) > maxf) return v > 0 ? INFINITY : -INFINITY;", ""),
    "round_bf16_one_bit_more": ("case ORC_BF16: p = 8;", "case ORC_BF16: p = 9;"),
    # element decoding
    "bf16_decode_shift": ("(uint32_t)h << 16", "(uint32_t)h << 15"),
    "fp16_subnormal_scale": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
}


def _site(name):
    """(old, new, start): the mutation replaces the first `old` at or after the
    first occurrence of `start` (a marker naming the function it belongs to)."""
    m = MUTANTS[name]
    return m if len(m) == 3 else (m[0], m[1], None)


def _mutate(src, name):
    old, new, start = _site(name)
    base = 0 if start is None else src.index(start)
    at = src.index(old, base)
    if start is None:
        assert src.count(old) == 1, "mutation site for %s not found exactly once" % name
    return src[:at] + new + src[at + len(old):]


def _run_mutant(name, old, new, tmp):
    src = open(SRC).read()
    path = os.path.join(tmp, name + ".c")
    with open(path, "w") as f:
        f.write(_mutate(src, name))
    lib = os.path.join(tmp, "lib_" + name + ".so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
                           "-shared", "-w", "-o", lib, path, "-lm"])
    env = dict(os.environ, OMM_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    failed = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED")]
    return r.returncode, failed


def test_every_mutant_is_caught():
    with tempfile.TemporaryDirectory() as tmp, cf.ThreadPoolExecutor(max_workers=4) as ex:
        futs = {name: ex.submit(_run_mutant, name, None, None, tmp) for name in MUTANTS}
        survivors = []
        for name, fut in futs.items():
            rc, failed = fut.result()
            if rc == 0:
                survivors.append(name)
        assert not survivors, "planted mistakes not caught by any pin: %s" % survivors


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutation_site_present(name):
    src = open(SRC).read()
    assert _mutate(src, name) != src
