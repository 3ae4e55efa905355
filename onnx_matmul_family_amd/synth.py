"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and stores them in the operators'
storage types; it holds none of the operators' arithmetic.  Every draw uses
numpy's PCG64 ``default_rng(seed)``; float inputs are drawn in fp32 and, for
bfloat16 / float16 storage, rounded to nearest-even once, so one host copy
feeds both the CPU oracle and the GPU.

bfloat16 arrays are numpy ``uint16`` bit patterns (numpy has no bfloat16).
"""
import numpy as np


def bf16_bits(x):
    """fp32 -> bfloat16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b):
    """bfloat16 bit pattern -> fp32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def store(x, dt):
    """Store fp32 draws in the named float type ('f32', 'f16', 'bf16', 'f64')."""
    if dt == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dt == "f16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16)
    if dt == "bf16":
        return bf16_bits(x)
    if dt == "f64":
        return np.ascontiguousarray(x, dtype=np.float64)
    raise ValueError(dt)


def normal(rng, shape, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def uniform(rng, shape, lo, hi):
    x = rng.random(size=shape, dtype=np.float32)
    return (x * np.float32(hi - lo) + np.float32(lo)).astype(np.float32)


def small_ints(rng, shape, lo=-2, hi=2):
    """Small integers as floats: every product and partial sum is exact in fp32."""
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def int8_uniform(rng, shape, lo=-128, hi=127, dtype=np.int8):
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(dtype)


def distinct_groups(rng, M, S, G, dtype=np.int32):
    """For each of M tokens, S distinct group ids drawn uniformly from [0, G)."""
    if S == 0 or M == 0:
        return np.zeros((M, S), dtype=dtype)
    keys = rng.random((M, G))
    return np.argsort(keys, axis=1)[:, :S].astype(dtype)


# --------------------------------------------------------------------------
# The five benchmark workloads (shapes, distributions and seeds as specified).

WORKLOADS = {
    "gemm_f32_64x32x48": "Gemm fp32, transA=1 transB=1, A[48,64] B[32,48] C[1,32], alpha=0.75 beta=1.5, N(0,1), seed 0",
    "matmul_bf16_bcast": "MatMul bf16, A[8,1,512,1024] x B[1,16,1024,768] -> Y[8,16,512,768], U(-1,1), seed 1",
    "gemm_bf16_8192": "Gemm bf16 M=N=K=8192, transB=1, C[8192], alpha=beta=1, A/B N(0,0.02), C U(-0.1,0.1), seed 2",
    "qlinear_i8_4096": "QLinearMatMul int8 4096^3, per-row a / per-column b scales U(0.002,0.01), zps U[-16,16], y_scale 0.05, y_zp 0, seed 3",
    "grouped_bf16_moe": "GroupedMatMul bf16, M=16384 K=4096 N=2048 G=64 S=8 int32 indices, input N(0,1), weights N(0,0.02), bias U(-0.1,0.1), seed 4",
}


def gemm_f32_64x32x48(seed=0):
    rng = np.random.default_rng(seed)
    A = normal(rng, (48, 64))
    B = normal(rng, (32, 48))
    C = normal(rng, (1, 32))
    return dict(A=A, B=B, C=C, alpha=0.75, beta=1.5, transA=1, transB=1, dt="f32")


def matmul_bf16_bcast(seed=1, scale=1):
    """scale > 1 divides M, N and K by it (smaller parity cases of the same structure)."""
    rng = np.random.default_rng(seed)
    M, K, N = 512 // scale, 1024 // scale, 768 // scale
    A = store(uniform(rng, (8, 1, M, K), -1.0, 1.0), "bf16")
    B = store(uniform(rng, (1, 16, K, N), -1.0, 1.0), "bf16")
    return dict(A=A, B=B, dt="bf16")


def gemm_bf16_8192(seed=2, size=8192):
    rng = np.random.default_rng(seed)
    A = store(normal(rng, (size, size), 0.02), "bf16")
    B = store(normal(rng, (size, size), 0.02), "bf16")      # stored [N, K]
    C = store(uniform(rng, (size,), -0.1, 0.1), "bf16")
    return dict(A=A, B=B, C=C, alpha=1.0, beta=1.0, transA=0, transB=1, dt="bf16")


def qlinear_i8_4096(seed=3, size=4096):
    rng = np.random.default_rng(seed)
    a = int8_uniform(rng, (size, size))
    b = int8_uniform(rng, (size, size))
    a_scale = uniform(rng, (size, 1), 0.002, 0.01)
    b_scale = uniform(rng, (1, size), 0.002, 0.01)
    a_zp = int8_uniform(rng, (size, 1), -16, 16)
    b_zp = int8_uniform(rng, (1, size), -16, 16)
    y_scale = np.array(0.05, dtype=np.float32)
    y_zp = np.array(0, dtype=np.int8)
    return dict(a=a, a_scale=a_scale, a_zero_point=a_zp, b=b, b_scale=b_scale, b_zero_point=b_zp,
                y_scale=y_scale, y_zero_point=y_zp)


def grouped_bf16_moe(seed=4, M=16384, K=4096, N=2048, G=64, S=8):
    rng = np.random.default_rng(seed)
    inp = store(normal(rng, (M, K)), "bf16")
    weights = store(normal(rng, (G, K, N), 0.02), "bf16")
    bias = store(uniform(rng, (G, N), -0.1, 0.1), "bf16")
    idx = distinct_groups(rng, M, S, G, np.int32)
    return dict(input=inp, weights=weights, group_indices=idx, bias=bias, dt="bf16")


# Weight-only quantised experts (GroupedMatMul fed by DequantizeLinear): the
# grouped workload's shapes with int8 weights, one bf16 scale and int8 zero
# point per 128 k and column (scales U(1e-4, 3e-4): dequantised weights of
# about the same spread as the bf16 workload's N(0, 0.02)).
GROUPED_DQ_WORKLOAD = ("GroupedMatMul over int8 weights (DequantizeLinear blocked along K, block 128), bf16, "
                       "M=16384 K=4096 N=2048 G=64 S=8, q U[-128,127], zp U[-8,8], scale U(1e-4,3e-4), seed 5")


def grouped_dq_int8_moe(seed=5, M=16384, K=4096, N=2048, G=64, S=8, bs=128):
    rng = np.random.default_rng(seed)
    nkb = -(-K // bs)
    inp = store(normal(rng, (M, K)), "bf16")
    q = rng.integers(-128, 127, size=(G, K, N), dtype=np.int8, endpoint=True)
    scale = store(uniform(rng, (G, nkb, N), 1e-4, 3e-4), "bf16")
    zp = rng.integers(-8, 8, size=(G, nkb, N), dtype=np.int8, endpoint=True)
    bias = store(uniform(rng, (G, N), -0.1, 0.1), "bf16")
    idx = distinct_groups(rng, M, S, G, np.int32)
    return dict(input=inp, qweights=q, scale=scale, zero_point=zp, block_size=bs, group_indices=idx, bias=bias,
                dt="bf16")


# fp32 / fp64 GroupedMatMul (the page's type list includes float and double):
# a mid-size expert layer, 4096 tokens x 4 of 16 experts, K = N = 1024.
GROUPED_FP_WORKLOAD = ("GroupedMatMul %s, M=4096 K=1024 N=1024 G=16 S=4 int32 indices, input N(0,1), "
                       "weights N(0,0.02), bias U(-0.1,0.1), seed 7")


def grouped_fp_moe(dt, seed=7, M=4096, K=1024, N=1024, G=16, S=4):
    rng = np.random.default_rng(seed)
    if dt == "f64":
        inp = rng.standard_normal((M, K))
        weights = rng.standard_normal((G, K, N)) * 0.02
        bias = rng.uniform(-0.1, 0.1, (G, N))
    else:
        inp = store(normal(rng, (M, K)), dt)
        weights = store(normal(rng, (G, K, N), 0.02), dt)
        bias = store(uniform(rng, (G, N), -0.1, 0.1), dt)
    idx = distinct_groups(rng, M, S, G, np.int32)
    return dict(input=inp, weights=weights, group_indices=idx, bias=bias, dt=dt)
