"""The allocation-free product: nm_spmm_noalloc (split-k partial sums in the
library's static device scratch) against nm_spmm with a caller workspace, on
two calls in a row, the second with a smaller problem; also checked against
the oracle. Runs alone in a fresh process and after the other GPU tests."""
import numpy as np
import pytest
import torch

import oracle
import structured_sparse_gemm_nm_amd as nm
from structured_sparse_gemm_nm_amd import inputs
from tests.gpu_helpers import Guarded, dev, host, sync

pytestmark = pytest.mark.gpu


def _case(dtype, m, n, k, splits, seed, beta):
    if dtype == "i8":
        a = inputs.uniform_int((m, k), seed, -127, 127)
        b = inputs.uniform_int((n, k), seed + 1, -127, 127)
        c = inputs.uniform_int((m, n), seed + 2, -2**20, 2**20, np.int32) if beta else None
    else:
        a = inputs.normal((m, k), seed, 1.0, dtype)
        b = inputs.normal((n, k), seed + 1, 1.0, dtype)
        c = inputs.normal((m, n), seed + 2, 1.0, dtype) if beta else None
    ahat, _ = oracle.prune_1d(a, dtype, 2, 4)
    v, meta = oracle.compress(a, dtype, 2, 4)
    plan = nm.nm_plan_init(m, n, k, 2, 4, op_b="T", dtype=dtype)
    nm.nm_plan_set_split_k(plan, splits)
    return plan, ahat, v, meta, b, c


@pytest.mark.parametrize("dtype", ["f16", "i8"])
def test_noalloc_matches_workspace_product_twice(dtype):
    raw, odt = (np.int32, torch.int32) if dtype == "i8" else (np.uint16, torch.int16)
    alpha = 1.0 if dtype == "i8" else 0.75
    beta = 1.0 if dtype == "i8" else -0.5
    # first call: 4 k ranges over 512 x 1024 (8 MiB of partial sums); second: 3 over 256 x 256
    for (m, n, k, splits, seed) in [(512, 1024, 2048, 4, 11), (256, 256, 768, 3, 12)]:
        plan, ahat, v, meta, b, c = _case(dtype, m, n, k, splits, seed, beta)
        need = nm.nm_spmm_workspace_size(plan)
        assert 0 < need <= nm.NM_NOALLOC_SCRATCH_BYTES
        dv, dm, db = dev(v), dev(meta), dev(b)
        dc = dev(c) if c is not None else None
        d_ws = Guarded((m, n), odt)
        nm.nm_spmm(plan, alpha, dv, dm, db, beta, dc, d_ws.t, workspace=torch.empty(need, dtype=torch.uint8,
                                                                                        device="cuda"))
        d_na = Guarded((m, n), odt)
        nm.nm_spmm_noalloc(plan, alpha, dv, dm, db, beta, dc, d_na.t)
        sync()
        d_ws.check(); d_na.check()
        got = host(d_na.t, raw)
        assert np.array_equal(got, host(d_ws.t, raw)), (m, n, k)
        if dtype == "i8":
            ref = oracle.gemm_i64(ahat, np.ascontiguousarray(b.T), int(alpha), int(beta), c)
            assert np.array_equal(got.astype(np.int64), ref)
        else:
            A = oracle.decode(ahat, dtype); B = oracle.decode(np.ascontiguousarray(b.T), dtype)
            C = oracle.decode(c, dtype)
            ref = oracle.gemm_f64(A, B, alpha, beta, C)
            tol = oracle.tolerance(np.abs(A), np.abs(B), alpha, beta, C)
            assert (np.abs(oracle.decode(got, dtype) - ref) <= tol).all()


def test_noalloc_without_split_and_too_large():
    # no workspace needed: the same as nm_spmm
    plan, ahat, v, meta, b, c = _case("f16", 256, 256, 512, 1, 21, 0.0)
    d1 = Guarded((256, 256), torch.int16)
    d2 = Guarded((256, 256), torch.int16)
    nm.nm_spmm(plan, 1.0, dev(v), dev(meta), dev(b), 0.0, None, d1.t)
    nm.nm_spmm_noalloc(plan, 1.0, dev(v), dev(meta), dev(b), 0.0, None, d2.t)
    sync()
    assert np.array_equal(host(d1.t, np.uint16), host(d2.t, np.uint16))
    # a split whose partial sums exceed the scratch is refused before launching
    big = nm.nm_plan_init(2048, 2048, 4096, 2, 4, op_b="T", dtype="f16")
    nm.nm_plan_set_split_k(big, 4)
    assert nm.nm_spmm_workspace_size(big) > nm.NM_NOALLOC_SCRATCH_BYTES
    with pytest.raises(nm.NmError) as e:
        nm.nm_spmm_noalloc(big, 1.0, dev(v), dev(meta), dev(b), 0.0, None, d2.t)
    assert e.value.status == nm.NM_ERR_SHAPE and "scratch" in str(e.value)
