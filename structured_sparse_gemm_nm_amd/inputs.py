"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws numbers and stores them in the element formats; it holds
none of the method's arithmetic (no pruning, packing or products), so that the
oracle and the GPU path can both consume its bytes without sharing code.

Recipe: numpy PCG64 ``default_rng(seed)``; normal draws are fp64, scaled by
sigma, rounded to fp32 and then to the element format with round-to-nearest-even
(numpy's float16 cast for fp16, the bit-level rule below for bf16); the
out-of-cache GEMV workload (2^30 elements) draws fp32 normals directly
('normal32'), which halves the host memory and time of the draw. Integer draws
are uniform over the closed range.

The workloads mirror the shapes of the pages' examples: the BERT-Large GEMMs of
the cuSPARSELt blog (Table 1; batch 32 x seq 128 tokens), a transposable 2:4
training pair (pytorch issue 126420), int8 with int32 accumulation (the blog's
type list) and M = 32 groups (apex PR 1631, nmSPARSE).
"""
import numpy as np


def _fp32_to_bf16_bits(x32):
    """fp32 -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def normal(shape, seed, sigma=1.0, dtype="f16"):
    """N(0, sigma^2) draws as raw element bits (uint16) for 'f16' / 'bf16'."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(size=shape) * sigma).astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return _fp32_to_bf16_bits(x).reshape(shape)
    raise ValueError(dtype)


def normal32(shape, seed, sigma=1.0, dtype="f16"):
    """As normal(), but drawn as fp32 (for very large operands)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return _fp32_to_bf16_bits(x).reshape(shape)
    raise ValueError(dtype)


def uniform_int(shape, seed, lo, hi, dtype=np.int8):
    """Uniform integers in [lo, hi]."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(dtype)


def as_float(raw, dtype):
    """View helper for printing/plots only (fp16 bits -> float16 view)."""
    return raw.view(np.float16) if dtype == "f16" else raw


# Workload table. Seeds follow 1000*config + role. Shapes are (m, n, k) of
# D[m x n] = op(A)[m x k] op(B)[k x n]. 'b_draw' is the shape the B values are
# drawn in: 'nk' for token-major activations (n tokens x k features, as a
# model stores them), 'kn' for a plain k x n operand; op_b picks how the
# product consumes them ('T': the n x k array as stored, 'N': its k x n
# transpose, materialised).
WORKLOADS = {
    # small case: 256x256 fp16 weight, 64 columns
    "c1_fp16_256": dict(dtype="f16", N=2, M=4, m=256, n=64, k=256, op_a="N", op_b="N",
                        a=("normal", 1001, 1.0), b=("normal", 1002, 1.0), alpha=1.0, beta=0.0),
    # BERT-Large GEMMs, 4096 tokens (batch 32 x seq 128), weights N(0, 0.02)
    "c2_fc1": dict(dtype="f16", N=2, M=4, m=4096, n=4096, k=1024, a=("normal", 2001, 0.02),
                   b=("normal", 2011, 1.0), b_draw="nk", op_a="N", op_b="T", alpha=1.0, beta=0.0),
    "c2_fc2": dict(dtype="f16", N=2, M=4, m=1024, n=4096, k=4096, a=("normal", 2002, 0.02),
                   b=("normal", 2014, 1.0), b_draw="nk", op_a="N", op_b="T", alpha=1.0, beta=0.0),
    "c2_proj": dict(dtype="f16", N=2, M=4, m=1024, n=4096, k=1024, a=("normal", 2003, 0.02),
                    b=("normal", 2011, 1.0), b_draw="nk", op_a="N", op_b="T", alpha=1.0, beta=0.0),
    # bf16 training pair, transposable 2:4 weight 11008 x 4096
    "c3_fwd": dict(dtype="bf16", N=2, M=4, m=11008, n=8192, k=4096, op_a="N", op_b="T",
                   a=("normal", 3001, 0.02), b=("normal", 3002, 1.0), b_draw="nk", alpha=1.0, beta=0.0, tile=True),
    "c3_bwd": dict(dtype="bf16", N=2, M=4, m=4096, n=8192, k=11008, op_a="T", op_b="T",
                   a=("normal", 3001, 0.02), b=("normal", 3003, 1.0), b_draw="nk", alpha=1.0, beta=0.0, tile=True),
    # the training-pair shapes in fp16 (large-shape fp16 measurement)
    "x1_fwd": dict(dtype="f16", N=2, M=4, m=11008, n=8192, k=4096, op_a="N", op_b="T",
                   a=("normal", 3101, 0.02), b=("normal", 3102, 1.0), b_draw="nk", alpha=1.0, beta=0.0, tile=True),
    "x1_bwd": dict(dtype="f16", N=2, M=4, m=4096, n=8192, k=11008, op_a="T", op_b="T",
                   a=("normal", 3101, 0.02), b=("normal", 3103, 1.0), b_draw="nk", alpha=1.0, beta=0.0, tile=True),
    # the cuSPARSELt blog's Table 1 shapes (BERT-Large, sequence 128 x batch 128 =
    # 16384 tokens), for side-by-side context with the blog's figures; D is
    # column-major as in the blog's runs (D^T = tokens x features, row-major)
    "x3_qkv": dict(dtype="f16", N=2, M=4, m=3072, n=16384, k=1024, a=("normal", 7001, 0.02),
                   b=("normal", 7011, 1.0), b_draw="nk", op_a="N", op_b="T", alpha=1.0, beta=0.0, order_cd="col"),
    "x3_proj": dict(dtype="f16", N=2, M=4, m=1024, n=16384, k=1024, a=("normal", 7002, 0.02),
                    b=("normal", 7011, 1.0), b_draw="nk", op_a="N", op_b="T", alpha=1.0, beta=0.0, order_cd="col"),
    "x3_fc1": dict(dtype="f16", N=2, M=4, m=4096, n=16384, k=1024, a=("normal", 7003, 0.02),
                   b=("normal", 7011, 1.0), b_draw="nk", op_a="N", op_b="T", alpha=1.0, beta=0.0, order_cd="col"),
    "x3_fc2": dict(dtype="f16", N=2, M=4, m=1024, n=16384, k=4096, a=("normal", 7004, 0.02),
                   b=("normal", 7014, 1.0), b_draw="nk", op_a="N", op_b="T", alpha=1.0, beta=0.0, order_cd="col"),
    # int8 with int32 accumulate, beta = 1
    "c4_int8": dict(dtype="i8", N=2, M=4, m=4096, n=4096, k=4096, op_a="N", op_b="N",
                    a=("int", 4001, -127, 127), b=("int", 4002, -127, 127), c=("int32", 4003, -2**20, 2**20),
                    alpha=1.0, beta=1.0),
    # general N:M GEMV beyond the Infinity Cache: m = k = 32768 at 4:32
    # (compressed values 268 MB + metadata 84 MB)
    "x2_4of32_n1": dict(dtype="f16", N=4, M=32, m=32768, n=1, k=32768, op_a="N", op_b="N",
                        a=("normal32", 8001, 1.0), b=("normal", 8002, 1.0), alpha=1.0, beta=0.0),
    "x2_4of32_n8": dict(dtype="f16", N=4, M=32, m=32768, n=8, k=32768, op_a="N", op_b="N",
                        a=("normal32", 8001, 1.0), b=("normal", 8003, 1.0), alpha=1.0, beta=0.0),
    # general N:M with M = 32
    "c5_4of32_n1": dict(dtype="f16", N=4, M=32, m=4096, n=1, k=4096, op_a="N", op_b="N",
                        a=("normal", 5001, 1.0), b=("normal", 5002, 1.0), alpha=1.0, beta=0.0),
    "c5_4of32_n8": dict(dtype="f16", N=4, M=32, m=4096, n=8, k=4096, op_a="N", op_b="N",
                        a=("normal", 5001, 1.0), b=("normal", 5003, 1.0), alpha=1.0, beta=0.0),
    "c5_4of32_n4096": dict(dtype="f16", N=4, M=32, m=4096, n=4096, k=4096, op_a="N", op_b="N",
                           a=("normal", 5001, 1.0), b=("normal", 5004, 1.0), alpha=1.0, beta=0.0),
    "c5_8of32_n1": dict(dtype="f16", N=8, M=32, m=4096, n=1, k=4096, op_a="N", op_b="N",
                        a=("normal", 5001, 1.0), b=("normal", 5002, 1.0), alpha=1.0, beta=0.0),
    "c5_8of32_n8": dict(dtype="f16", N=8, M=32, m=4096, n=8, k=4096, op_a="N", op_b="N",
                        a=("normal", 5001, 1.0), b=("normal", 5003, 1.0), alpha=1.0, beta=0.0),
    "c5_8of32_n4096": dict(dtype="f16", N=8, M=32, m=4096, n=4096, k=4096, op_a="N", op_b="N",
                           a=("normal", 5001, 1.0), b=("normal", 5004, 1.0), alpha=1.0, beta=0.0),
    # vector-wise N:M (16 consecutive rows share each group's kept offsets) on the
    # M = 32 shapes: the variant whose gather of B rows is shared by a row block
    "c5vw_4of32_n1": dict(dtype="f16", N=4, M=32, m=4096, n=1, k=4096, op_a="N", op_b="N", vector_rows=16,
                          a=("normal", 5001, 1.0), b=("normal", 5002, 1.0), alpha=1.0, beta=0.0),
    "c5vw_4of32_n8": dict(dtype="f16", N=4, M=32, m=4096, n=8, k=4096, op_a="N", op_b="N", vector_rows=16,
                          a=("normal", 5001, 1.0), b=("normal", 5003, 1.0), alpha=1.0, beta=0.0),
    "c5vw_4of32_n4096": dict(dtype="f16", N=4, M=32, m=4096, n=4096, k=4096, op_a="N", op_b="N", vector_rows=16,
                             a=("normal", 5001, 1.0), b=("normal", 5004, 1.0), alpha=1.0, beta=0.0),
    "c5vw_8of32_n1": dict(dtype="f16", N=8, M=32, m=4096, n=1, k=4096, op_a="N", op_b="N", vector_rows=16,
                          a=("normal", 5001, 1.0), b=("normal", 5002, 1.0), alpha=1.0, beta=0.0),
    "c5vw_8of32_n8": dict(dtype="f16", N=8, M=32, m=4096, n=8, k=4096, op_a="N", op_b="N", vector_rows=16,
                          a=("normal", 5001, 1.0), b=("normal", 5003, 1.0), alpha=1.0, beta=0.0),
    "c5vw_8of32_n4096": dict(dtype="f16", N=8, M=32, m=4096, n=4096, k=4096, op_a="N", op_b="N", vector_rows=16,
                             a=("normal", 5001, 1.0), b=("normal", 5004, 1.0), alpha=1.0, beta=0.0),
}


def stored_shape_a(w):
    return (w["m"], w["k"]) if w.get("op_a", "N") == "N" else (w["k"], w["m"])


def stored_shape_b(w):
    return (w["k"], w["n"]) if w.get("op_b", "N") == "N" else (w["n"], w["k"])


_LARGE = {}   # the most recent large draw (>= 2^28 elements), reused when asked for again


def draw(spec, shape, dtype):
    key = (tuple(spec), tuple(shape), dtype)
    if int(np.prod(shape)) >= (1 << 28):
        if key not in _LARGE:
            _LARGE.clear()
            _LARGE[key] = _draw(spec, shape, dtype)
        return _LARGE[key]
    return _draw(spec, shape, dtype)


def _draw(spec, shape, dtype):
    kind = spec[0]
    if kind == "normal":
        return normal(shape, spec[1], spec[2], dtype)
    if kind == "normal32":
        return normal32(shape, spec[1], spec[2], dtype)
    if kind == "int":
        return uniform_int(shape, spec[1], spec[2], spec[3], np.int8)
    if kind == "int32":
        return uniform_int(shape, spec[1], spec[2], spec[3], np.int32)
    raise ValueError(kind)


def workload_inputs(name, op_b=None):
    """Dense stored A (before pruning), B stored for op_b, and C (or None)."""
    w = WORKLOADS[name]
    ob = op_b or w.get("op_b", "N")
    a = draw(w["a"], stored_shape_a(w), w["dtype"])
    if w.get("b_draw", "kn") == "nk":
        b = draw(w["b"], (w["n"], w["k"]), w["dtype"])
        b = b if ob == "T" else np.ascontiguousarray(b.T)
    else:
        b = draw(w["b"], (w["k"], w["n"]), w["dtype"])
        b = b if ob == "N" else np.ascontiguousarray(b.T)
    c = draw(w["c"], (w["m"], w["n"]), w["dtype"]) if "c" in w else None
    return a, b, c
