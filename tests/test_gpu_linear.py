"""The runtime-sparsified linear layer (forward and backward through the C ABI)
against the oracle: W_hat = the oracle's transposable tile prune of W,
Y = X W_hat^T, dX = dY W_hat, dW = dY^T X, each in fp64 and within the
fp16/bf16 bound |D - D_ref| <= 1e-2 (|A| |B|)_ij + 1e-3."""
import numpy as np
import pytest
import torch

import oracle
from structured_sparse_gemm_nm_amd import inputs
from structured_sparse_gemm_nm_amd.linear import SemiStructuredSparseLinear
from tests.gpu_helpers import host, sync

pytestmark = pytest.mark.gpu

TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


def to_torch(raw, dtype):
    return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).cuda().view(TORCH[dtype])


def check(dtype, got, A, B):
    ref = oracle.gemm_f64(A, B)
    tol = oracle.tolerance(np.abs(A), np.abs(B))
    g = oracle.decode(host(got.contiguous().view(torch.int16), np.uint16), dtype)
    assert np.isfinite(g).all()
    err = np.abs(g - ref)
    assert (err <= tol).all(), (err.max(), np.argmax(err - tol))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(96, 128, 192), (64, 264, 136)])
def test_sparse_linear_forward_backward(dtype, shape):
    tokens, in_f, out_f = shape
    w = inputs.normal((out_f, in_f), 9001 + in_f, 0.02, dtype)
    x = inputs.normal((tokens, in_f), 9002 + in_f, 1.0, dtype)
    dy = inputs.normal((tokens, out_f), 9003 + in_f, 1.0, dtype)
    layer = SemiStructuredSparseLinear(in_f, out_f, dtype=TORCH[dtype], weight=to_torch(w, dtype))
    xt = to_torch(x, dtype).view(2, tokens // 2, in_f).requires_grad_(True)
    y = layer(xt)
    assert y.shape == (2, tokens // 2, out_f)
    y.backward(to_torch(dy, dtype).view(2, tokens // 2, out_f))
    sync()
    w_hat, _ = oracle.prune_tile(w, dtype)
    W = oracle.decode(w_hat, dtype)
    X = oracle.decode(x, dtype)
    DY = oracle.decode(dy, dtype)
    check(dtype, y.reshape(tokens, out_f), X, np.ascontiguousarray(W.T))
    check(dtype, xt.grad.reshape(tokens, in_f), DY, W)
    check(dtype, layer.weight.grad, np.ascontiguousarray(DY.T), X)
    # the weight itself is untouched (runtime sparsification works on a copy)
    assert np.array_equal(host(layer.weight.detach().view(torch.int16), np.uint16), w)


def test_sparse_linear_rejects_bad_shapes():
    with pytest.raises(ValueError):
        SemiStructuredSparseLinear(100, 64)
    layer = SemiStructuredSparseLinear(64, 64)
    with pytest.raises(ValueError):
        layer(torch.zeros((6, 64), dtype=torch.float16, device="cuda"))
