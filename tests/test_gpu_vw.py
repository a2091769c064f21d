"""GPU parity of vector-wise N:M (V consecutive rows share each group's kept
offsets) against the CPU oracle: prune (with the keep mask), prune check,
compress and decompress bit-exact on padded rows, and the product on the
vector-wise matrix-core kernel and on the fallbacks (general gather, small n)
within tolerance (bit-exact for int8)."""
import numpy as np
import pytest
import torch

import oracle
import structured_sparse_gemm_nm_amd as nm
from structured_sparse_gemm_nm_amd import inputs
from tests.gpu_helpers import Guarded, dev, host, sync

pytestmark = pytest.mark.gpu

RAW = {"f16": np.uint16, "bf16": np.uint16, "i8": np.int8}
TRAW = {"f16": torch.int16, "bf16": torch.int16, "i8": torch.int8}


def values(dtype, shape, seed, ties=False):
    if ties:
        rng = np.random.default_rng(seed)
        if dtype == "i8":
            return rng.integers(-3, 4, size=shape).astype(np.int8)
        x = rng.choice(np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 2.0], np.float32), size=shape)
        return x.astype(np.float16).view(np.uint16) if dtype == "f16" else inputs._fp32_to_bf16_bits(x).reshape(shape)
    if dtype == "i8":
        return inputs.uniform_int(shape, seed, -127, 127)
    return inputs.normal(shape, seed, 1.0, dtype)


ELEM_CASES = [
    # (V, N, M, m, k): k past whole 256-column chunks, several blocks, wide and narrow groups
    (16, 4, 32, 32, 544), (16, 8, 32, 48, 1024), (32, 2, 4, 64, 260), (2, 3, 8, 10, 264),
    (4, 5, 16, 12, 272), (16, 31, 32, 16, 320), (256, 1, 4, 256, 32), (8, 1, 4, 24, 100),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("case", ELEM_CASES, ids=["V%d-%d:%d-%dx%d" % c for c in ELEM_CASES])
@pytest.mark.parametrize("ties", [False, True])
def test_vw_elementwise(dtype, case, ties):
    V, N, M, m, k = case
    es = 1 if dtype == "i8" else 2
    lda = -(-k // (16 // es)) * (16 // es) + 16 // es              # padded rows, 16-byte starts
    full = values(dtype, (m, lda), 300 + V + N + M + k, ties)
    a = np.ascontiguousarray(full[:, :k])
    plan = nm.nm_plan_init(m, 32, k, N, M, dtype=dtype, lda=lda, vector_rows=V)
    sentinel = np.full((m, lda), 0x5A if es == 1 else 0x5A5A, dtype=RAW[dtype])
    # prune + keep mask
    ref, keep = oracle.prune_vw(a, dtype, V, N, M)
    out = Guarded((m, lda), TRAW[dtype], fill=dev(sentinel))
    mask = Guarded((plan.mask_bytes // 4,), torch.int32)
    nm.nm_prune(plan, dev(full), out.t, "1d", mask.t)
    sync()
    out.check(); mask.check()
    got = host(out.t, RAW[dtype])
    assert np.array_equal(got[:, :k], ref)
    assert np.array_equal(got[:, k:], sentinel[:, k:])
    assert np.array_equal(host(mask.t, np.uint32).reshape(m, -1), oracle.mask_bits(keep))
    # check: raw input and pruned
    cnt = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    nm.nm_prune_check(plan, dev(full), "1d", cnt)
    sync()
    assert int(cnt.item()) == oracle.check_vw(a, dtype, V, N, M)
    pf = full.copy(); pf[:, :k] = ref
    nm.nm_prune_check(plan, dev(pf), "1d", cnt)
    sync()
    assert int(cnt.item()) == 0
    # compress (one metadata row per block) and decompress of the oracle's form
    vref, mref = oracle.compress_vw(a, dtype, V, N, M)
    assert plan.meta_bytes == (m // V) * plan.meta_ld
    vals = Guarded((m, plan.values_ld), TRAW[dtype], fill=torch.full((m, plan.values_ld), -1, dtype=TRAW[dtype]))
    meta = Guarded((m // V, plan.meta_ld), torch.uint8, fill=torch.full((m // V, plan.meta_ld), 0xEE, dtype=torch.uint8))
    nm.nm_compress(plan, dev(full), vals.t, meta.t)
    sync()
    vals.check(); meta.check()
    assert np.array_equal(host(vals.t, RAW[dtype]), vref)
    assert np.array_equal(host(meta.t, np.uint8), mref)
    dec = Guarded((m, lda), TRAW[dtype], fill=dev(sentinel))
    nm.nm_decompress(plan, dev(vref), dev(mref), dec.t)
    sync()
    dec.check()
    got = host(dec.t, RAW[dtype])
    assert np.array_equal(got[:, :k], oracle.decompress_vw(vref, mref, dtype, m, k, V, N, M))
    assert np.array_equal(got[:, k:], sentinel[:, k:])


def run_vw_product(dtype, V, N, M, m, n, k, op_b, alpha, beta, seed, expect):
    a = values(dtype, (m, k), seed)
    ahat, _ = oracle.prune_vw(a, dtype, V, N, M)
    vref, mref = oracle.compress_vw(a, dtype, V, N, M)
    b_log = values(dtype, (k, n), seed + 1)
    b_st = b_log if op_b == "N" else np.ascontiguousarray(b_log.T)
    c = None
    if beta != 0:
        c = (inputs.uniform_int((m, n), seed + 2, -2**20, 2**20, np.int32) if dtype == "i8"
             else values(dtype, (m, n), seed + 2))
    plan = nm.nm_plan_init(m, n, k, N, M, op_b=op_b, dtype=dtype, vector_rows=V)
    assert plan.kernel_name == expect, plan.kernel_name
    odt, raw = (torch.int32, np.int32) if dtype == "i8" else (torch.int16, np.uint16)
    d = Guarded((m, n), odt)
    nm.nm_spmm(plan, alpha, dev(vref), dev(mref), dev(b_st), beta, dev(c) if c is not None else None, d.t)
    sync()
    d.check()
    got = host(d.t, raw)
    if dtype == "i8":
        ref = oracle.gemm_i64(ahat, b_log, int(alpha), int(beta), c)
        assert np.array_equal(got.astype(np.int64), ref)
        return plan
    A = oracle.decode(ahat, dtype); B = oracle.decode(b_log, dtype)
    C = oracle.decode(c, dtype) if c is not None else None
    ref = oracle.gemm_f64(A, B, alpha, beta, C)
    tol = oracle.tolerance(np.abs(A), np.abs(B), alpha, beta, C)
    g = oracle.decode(got, dtype)
    assert np.isfinite(g).all()
    bad = np.abs(g - ref) > tol
    assert not bad.any(), (np.argwhere(bad)[:5], np.abs(g - ref)[bad][:5])
    return plan


MFMA_CASES = [
    # (V, N, M, m, n, k): 4:32 and 8:32 (the M = 32 configurations), 2:4 and 1:8, V = 16 and 32
    (16, 4, 32, 256, 128, 512), (16, 8, 32, 512, 256, 1024), (32, 4, 32, 256, 256, 512),
    (16, 2, 4, 256, 128, 512), (16, 1, 8, 256, 384, 1024), (64, 8, 32, 512, 128, 768),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("case", MFMA_CASES, ids=["V%d-%d:%d-%dx%dx%d" % c for c in MFMA_CASES])
@pytest.mark.parametrize("ab", [(1.0, 0.0), (2.0, -1.0)])
def test_vw_spmm_mfma(dtype, case, ab):
    V, N, M, m, n, k = case
    kl = 256 if dtype == "i8" else 128
    if k % kl:
        pytest.skip("k-step of this type does not divide k")
    if dtype == "i8" and 256 * N // M < 32:
        pytest.skip("int8 needs at least 32 kept k per step")
    alpha, beta = ab
    if dtype != "i8" and beta != 0:
        alpha, beta = 0.75, -0.5
    plan = run_vw_product(dtype, V, N, M, m, n, k, "N", alpha, beta, 4000 + V + N + m + k, "spmm_vw_mfma")
    assert "vw_gemm_kernel" in plan.spmm_kernel


FALLBACK_CASES = [
    # (V, N, M, m, n, k, op_b, kernel): B stored n x k, ragged tiles, V below 16, N not a power of two, small n
    (16, 4, 32, 256, 128, 512, "T", "spmm_gather_mfma"),
    (16, 4, 32, 272, 80, 544, "N", "spmm_gather_mfma"),
    (2, 2, 4, 64, 96, 128, "N", "spmm_gather_mfma"),
    (16, 3, 8, 256, 128, 256, "N", "spmm_gather_mfma"),
    (16, 8, 32, 256, 1, 1024, "N", "spmm_skinny"),
    (32, 4, 32, 256, 8, 1024, "T", "spmm_skinny"),
    (4, 2, 4, 100, 16, 96, "N", "spmm_skinny"),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("case", FALLBACK_CASES, ids=["V%d-%d:%d-%dx%dx%d-%s" % c[:7] for c in FALLBACK_CASES])
def test_vw_spmm_fallbacks(dtype, case):
    V, N, M, m, n, k, op_b, kern = case
    if m % V:
        pytest.skip("m must be a multiple of V")
    alpha, beta = (1.0, 1.0) if dtype == "i8" else (0.5, 0.25)
    run_vw_product(dtype, V, N, M, m, n, k, op_b, alpha, beta, 5000 + V + N + n, kern)
