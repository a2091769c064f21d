"""ctypes wrapper around liboracle.so (oracle.c) — TEST INFRASTRUCTURE ONLY.

Arrays are numpy. 16-bit floating formats travel as their raw bits (uint16),
int8 as int8. Every routine works on the *logical* op(A) (m rows, k columns,
groups along k); for op_a == 'T' the stored k x m matrix is transposed here
(a numpy view change, no arithmetic) before and after the C routine.

What is computed, and from which page:
  prune_1d      -- apex PR "[sparse] update support for arbitrary N:M settings
                   sparse", extension 1 (mn_1d_greedy): top-N |w| per group of M.
  *_vw          -- the same PR, extension 2: vector-wise N:M (V rows share the
                   kept offsets; vector score |sum of its values|).
  prune_tile    -- pytorch issue "backpropagation for sparse semi-structured",
                   maintainer reply: 2:4 in both directions on 4x4 tiles.
  check_*       -- cuSPARSELt blog, the prune-check snippet (non-zero = invalid).
  compress /
  decompress    -- cuSPARSELt blog, Figure 2 text: kept values + index metadata.
  gemm_*        -- cuSPARSELt blog: D = alpha*op(A)*op(B) + beta*C (int8
                   output: the exact integer saturated to int8).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

DT = {"f16": 0, "bf16": 1, "i8": 2}
ESIZE = {"f16": 2, "bf16": 2, "i8": 1}
NP_RAW = {"f16": np.uint16, "bf16": np.uint16, "i8": np.int8}


def build(force=False):
    """Compile oracle.c into liboracle.so with plain gcc (no FMA contraction)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                               "-o", _SO, _SRC, "-lm"])
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_SO)
        P, I64, I, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.or_f16_to_f64.restype = D; L.or_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.or_bf16_to_f64.restype = D; L.or_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.or_decode.argtypes = [P, I, I64, P]
        L.or_prune_1d.argtypes = [P, I, I64, I64, I, I, P, P]
        L.or_prune_tile.argtypes = [P, I, I64, I64, P, P]
        L.or_tile_patterns.restype = I; L.or_tile_patterns.argtypes = [P]
        L.or_check_1d.restype = I64; L.or_check_1d.argtypes = [P, I, I64, I64, I, I]
        L.or_check_tile.restype = I64; L.or_check_tile.argtypes = [P, I, I64, I64]
        L.or_meta_bits.restype = I; L.or_meta_bits.argtypes = [I]
        L.or_compress.argtypes = [P, I, I64, I64, I, I, P, I64, P, I64]
        L.or_decompress.argtypes = [P, I64, P, I64, I, I64, I64, I, I, P]
        L.or_gemm_f64.argtypes = [P, P, P, P, I64, I64, I64, D, D]
        L.or_gemm_f64_points.argtypes = [P, P, P, P, I64, P, P, I64, D, D]
        L.or_gemm_i64.argtypes = [P, P, P, P, I64, I64, I64, I64, I64]
        L.or_threads.restype = I; L.or_threads.argtypes = []
        L.or_spmm_compressed_f64.argtypes = [P, I64, P, I64, I, I64, I64, I, I, P, I64, P, P, D, D]
        L.or_prune_vw.argtypes = [P, I, I64, I64, I, I, I, P, P]
        L.or_check_vw.restype = I64; L.or_check_vw.argtypes = [P, I, I64, I64, I, I, I]
        L.or_compress_vw.argtypes = [P, I, I64, I64, I, I, I, P, I64, P, I64]
        L.or_decompress_vw.argtypes = [P, I64, P, I64, I, I64, I64, I, I, I, P]
        L.or_spmm_compressed_vw_f64.argtypes = [P, I64, P, I64, I, I64, I64, I, I, I, P, I64, P]
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype=None):
    a = np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))
    return a


def _logical(a, op):
    """Stored matrix -> logical op(A) (contiguous copy)."""
    return np.ascontiguousarray(a.T if op == "T" else a)


def _stored(x, op):
    return np.ascontiguousarray(x.T if op == "T" else x)


# ---------------------------------------------------------------- decoding

def decode(raw, dtype):
    """Raw element bits -> float64 (oracle's own IEEE decoders)."""
    raw = _c(raw, NP_RAW[dtype])
    out = np.empty(raw.shape, np.float64)
    lib().or_decode(_ptr(raw), DT[dtype], raw.size, _ptr(out))
    return out


def threads():
    """OpenMP threads the oracle's parallel loops use."""
    return lib().or_threads()


def meta_bits(M):
    return lib().or_meta_bits(M)


# ---------------------------------------------------------------- layout sizes

def values_ld(k, N, M, dtype):
    """Row stride (elements) of the compressed values: k*N/M rounded up to 16 bytes."""
    per = 16 // ESIZE[dtype]
    n = k * N // M
    return (n + per - 1) // per * per


def meta_ld(k, N, M):
    """Row stride (bytes) of the metadata: ceil(k/M * N * b / 8) rounded up to 16."""
    nbytes = ((k // M) * N * meta_bits(M) + 7) // 8
    return (nbytes + 15) // 16 * 16


# ---------------------------------------------------------------- prune / check

def prune_1d(a, dtype, N, M, op="N"):
    """Returns (pruned stored matrix, keep mask as uint8 in stored layout)."""
    x = _logical(_c(a, NP_RAW[dtype]), op)
    rows, cols = x.shape
    assert cols % M == 0
    out = np.empty_like(x)
    keep = np.empty(x.shape, np.uint8)
    lib().or_prune_1d(_ptr(x), DT[dtype], rows, cols, N, M, _ptr(out), _ptr(keep))
    return _stored(out, op), _stored(keep, op)


def prune_tile(a, dtype):
    """Transposable 2:4 on 4x4 tiles of the stored matrix. Returns (pruned, keep)."""
    x = _c(a, NP_RAW[dtype])
    rows, cols = x.shape
    assert rows % 4 == 0 and cols % 4 == 0
    out = np.empty_like(x)
    keep = np.empty(x.shape, np.uint8)
    lib().or_prune_tile(_ptr(x), DT[dtype], rows, cols, _ptr(out), _ptr(keep))
    return out, keep


def tile_patterns():
    """The oracle's 90 candidate tile patterns as (90, 4) pair indices."""
    pat = np.zeros((90, 4), np.int32)
    n = lib().or_tile_patterns(_ptr(pat))
    assert n == 90
    return pat


def check_1d(a, dtype, N, M, op="N"):
    x = _logical(_c(a, NP_RAW[dtype]), op)
    return int(lib().or_check_1d(_ptr(x), DT[dtype], x.shape[0], x.shape[1], N, M))


def check_tile(a, dtype):
    x = _c(a, NP_RAW[dtype])
    return int(lib().or_check_tile(_ptr(x), DT[dtype], x.shape[0], x.shape[1]))


def mask_bits(keep):
    """Keep mask (uint8, rows x cols) -> packed bitmask: uint32 words, LSB first,
    each row starting at a fresh word (ceil(cols/32) words per row)."""
    rows, cols = keep.shape
    words = (cols + 31) // 32
    padded = np.zeros((rows, words * 32), np.uint8)
    padded[:, :cols] = keep
    return np.packbits(padded, axis=1, bitorder="little").view(np.uint32).reshape(rows, words)


# ---------------------------------------------------------------- compress / decompress

def compress(a, dtype, N, M, op="N"):
    """Returns (values rows x values_ld raw, meta rows x meta_ld uint8)."""
    x = _logical(_c(a, NP_RAW[dtype]), op)
    rows, cols = x.shape
    vld, mld = values_ld(cols, N, M, dtype), meta_ld(cols, N, M)
    vals = np.empty((rows, vld), NP_RAW[dtype])
    meta = np.empty((rows, mld), np.uint8)
    lib().or_compress(_ptr(x), DT[dtype], rows, cols, N, M, _ptr(vals), vld, _ptr(meta), mld)
    return vals, meta


def decompress(vals, meta, dtype, m, k, N, M, op="N"):
    """Inverse of compress; returns the stored dense matrix (m x k for 'N', k x m for 'T')."""
    vals = _c(vals, NP_RAW[dtype]); meta = _c(meta, np.uint8)
    out = np.empty((m, k), NP_RAW[dtype])
    lib().or_decompress(_ptr(vals), vals.shape[1], _ptr(meta), meta.shape[1], DT[dtype], m, k, N, M, _ptr(out))
    return _stored(out, op)


# ---------------------------------------------------------------- vector-wise N:M

def prune_vw(a, dtype, V, N, M):
    """Vector-wise N:M on logical op(A) (m x k, m a multiple of V): every block of
    V consecutive rows keeps, in each group of M columns, the N columns whose
    score |sum of the V values| is largest (apex PR extension 2's vector score),
    ties to the lower offset. Returns (pruned, keep mask as uint8)."""
    x = _c(a, NP_RAW[dtype])
    rows, cols = x.shape
    assert rows % V == 0 and cols % M == 0
    out = np.empty_like(x)
    keep = np.empty(x.shape, np.uint8)
    lib().or_prune_vw(_ptr(x), DT[dtype], rows, cols, V, N, M, _ptr(out), _ptr(keep))
    return out, keep


def check_vw(a, dtype, V, N, M):
    """Number of (V-row block, group) pairs whose rows use more than N offsets."""
    x = _c(a, NP_RAW[dtype])
    return int(lib().or_check_vw(_ptr(x), DT[dtype], x.shape[0], x.shape[1], V, N, M))


def compress_vw(a, dtype, V, N, M):
    """Returns (values rows x values_ld, meta (rows / V) x meta_ld)."""
    x = _c(a, NP_RAW[dtype])
    rows, cols = x.shape
    vld, mld = values_ld(cols, N, M, dtype), meta_ld(cols, N, M)
    vals = np.empty((rows, vld), NP_RAW[dtype])
    meta = np.empty((rows // V, mld), np.uint8)
    lib().or_compress_vw(_ptr(x), DT[dtype], rows, cols, V, N, M, _ptr(vals), vld, _ptr(meta), mld)
    return vals, meta


def decompress_vw(vals, meta, dtype, m, k, V, N, M):
    vals = _c(vals, NP_RAW[dtype]); meta = _c(meta, np.uint8)
    out = np.empty((m, k), NP_RAW[dtype])
    lib().or_decompress_vw(_ptr(vals), vals.shape[1], _ptr(meta), meta.shape[1], DT[dtype], m, k, V, N, M, _ptr(out))
    return out


def spmm_compressed_vw_f64(vals, meta, dtype, m, k, V, N, M, B):
    """The sparse loop on the vector-wise form: D = A_hat @ B in fp64, reading (values, metadata)."""
    vals = _c(vals, NP_RAW[dtype]); meta = _c(meta, np.uint8); B = _c(B, np.float64)
    n = B.shape[1]
    D = np.empty((m, n), np.float64)
    lib().or_spmm_compressed_vw_f64(_ptr(vals), vals.shape[1], _ptr(meta), meta.shape[1], DT[dtype], m, k, V, N, M,
                                    _ptr(B), n, _ptr(D))
    return D


# ---------------------------------------------------------------- products

def gemm_f64(A, B, alpha=1.0, beta=0.0, C=None):
    """D = alpha*A@B + beta*C, fp64 triple loop; A (m,k), B (k,n) float64 logical operands."""
    A = _c(A, np.float64); B = _c(B, np.float64)
    m, k = A.shape; n = B.shape[1]
    D = np.empty((m, n), np.float64)
    Cc = _c(C, np.float64) if (C is not None and beta != 0.0) else None
    lib().or_gemm_f64(_ptr(A), _ptr(B), _ptr(Cc), _ptr(D), m, n, k, float(alpha), float(beta))
    return D


def gemm_f64_points(A, Bt, pi, pj, alpha=1.0, beta=0.0, Cpts=None):
    """Selected outputs D[pi[p], pj[p]]; A (m,k), Bt = op(B)^T (n,k) float64."""
    A = _c(A, np.float64); Bt = _c(Bt, np.float64)
    pi = _c(pi, np.int64); pj = _c(pj, np.int64)
    out = np.empty(pi.size, np.float64)
    Cc = _c(Cpts, np.float64) if (Cpts is not None and beta != 0.0) else None
    lib().or_gemm_f64_points(_ptr(A), _ptr(Bt), _ptr(Cc), _ptr(out), A.shape[1], _ptr(pi), _ptr(pj), pi.size,
                             float(alpha), float(beta))
    return out


def gemm_i64(A, B, alpha=1, beta=0, C=None):
    """Exact integer D = alpha*A@B + beta*C for int8 A (m,k), B (k,n), int32 C."""
    A = _c(A, np.int8); B = _c(B, np.int8)
    m, k = A.shape; n = B.shape[1]
    D = np.empty((m, n), np.int64)
    Cc = _c(C, np.int32) if C is not None else None
    lib().or_gemm_i64(_ptr(A), _ptr(B), _ptr(Cc), _ptr(D), m, n, k, int(alpha), int(beta))
    return D


def gemm_i8_saturated(A, B, alpha=1, beta=0, C=None):
    """int8 output (cuSPARSELt blog: int8 inputs and outputs with int32
    accumulation): the exact integer alpha*A@B + beta*C, int8 C widened
    exactly, saturated to [-128, 127] (saturation is the reading taken for
    the int8 store)."""
    Cw = np.asarray(C, np.int32) if C is not None else None
    return np.clip(gemm_i64(A, B, alpha, beta, Cw), -128, 127).astype(np.int8)


def spmm_compressed_f64(vals, meta, dtype, m, k, N, M, B, alpha=1.0, beta=0.0, C=None):
    """The sparse loop: fp64 product read directly from (values, metadata)."""
    vals = _c(vals, NP_RAW[dtype]); meta = _c(meta, np.uint8); B = _c(B, np.float64)
    n = B.shape[1]
    D = np.empty((m, n), np.float64)
    Cc = _c(C, np.float64) if (C is not None and beta != 0.0) else None
    lib().or_spmm_compressed_f64(_ptr(vals), vals.shape[1], _ptr(meta), meta.shape[1], DT[dtype], m, k, N, M,
                                 _ptr(B), n, _ptr(Cc), _ptr(D), float(alpha), float(beta))
    return D


def tolerance(absA, absB, alpha=1.0, beta=0.0, C=None):
    """Elementwise bound for fp16/bf16 outputs: 1e-2*(|alpha|*(|A|@|B|) + |beta|*|C|) + 1e-3."""
    t = abs(alpha) * gemm_f64(absA, absB)
    if C is not None and beta != 0.0:
        t = t + abs(beta) * np.abs(C)
    return 1e-2 * t + 1e-3
