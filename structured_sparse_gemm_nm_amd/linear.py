"""A runtime-sparsified linear layer over the C ABI.

The pytorch issue "backpropagation for sparse semi-structured" (maintainer
reply) describes the use this serves: a drop-in replacement for a linear layer
whose weight is made 2:4 on 4x4 tiles, so that both the forward product W x
and the backward product W^T dL/dy run on the 2:4 instructions, with the
weight pruned and compressed again at run time every step.

Per forward, with W the dense (out x in) weight and X the (tokens x in) input:

- nm_prune TILE4X4: W_hat, two kept per row and per column of every 4x4 tile;
- nm_compress twice: W_hat along in (op_a = N) for the forward and along out
  (op_a = T) for the backward;
- nm_spmm: Y^T = W_hat X^T written column-major, i.e. Y (tokens x out)
  row-major.

Backward, with dY the (tokens x out) output gradient:

- nm_spmm: dX^T = W_hat^T dY^T written column-major, i.e. dX row-major;
- nm_dense_gemm: dW = dY^T X, the dense gradient of the pruned product, handed
  to the dense weight as it is (the pages describe no masking of the weight
  gradient; the next forward prunes again), or, with mask_weight_grad=True,
  masked with the forward's keep mask (nm_mask_apply), so that pruned weights
  receive no gradient.

Every step runs in the library's kernels; this module only allocates the
outputs with torch and marshals pointers. Shapes: in and out multiples of 8
(4x4 tiles and 16-byte rows of 16-bit elements), tokens a multiple of 4 (the
reduction length of the weight-gradient product).
"""
import torch

from . import nm_compress, nm_dense_gemm, nm_mask_apply, nm_plan_init, nm_prune, nm_spmm

_DTYPE_NAMES = {torch.float16: "f16", torch.bfloat16: "bf16"}


class _Plans:
    """The four plans of one (out, in, tokens, dtype) shape (host-only objects)."""

    def __init__(self, out_f, in_f, tokens, dtype):
        self.fwd = nm_plan_init(out_f, tokens, in_f, 2, 4, op_a="N", op_b="T", dtype=dtype, order_cd="col")
        self.bwd = nm_plan_init(in_f, tokens, out_f, 2, 4, op_a="T", op_b="T", dtype=dtype, order_cd="col")
        self.dw = nm_plan_init(out_f, in_f, tokens, 2, 4, op_a="T", op_b="N", dtype=dtype)


_PLAN_CACHE = {}


def _plans(out_f, in_f, tokens, dtype):
    key = (out_f, in_f, tokens, dtype)
    p = _PLAN_CACHE.get(key)
    if p is None:
        p = _PLAN_CACHE[key] = _Plans(out_f, in_f, tokens, dtype)
    return p


def _check_operands(x2d, weight):
    """The library takes raw device addresses: refuse host tensors, mixed devices
    and dtype mismatches before anything is launched."""
    if weight.dtype not in _DTYPE_NAMES:
        raise ValueError("weight must be torch.float16 or torch.bfloat16, got %s" % weight.dtype)
    if x2d.dtype != weight.dtype:
        raise ValueError("input dtype %s differs from the weight dtype %s" % (x2d.dtype, weight.dtype))
    if not (x2d.is_cuda and weight.is_cuda):
        raise ValueError("input and weight must be GPU tensors")
    if x2d.device != weight.device:
        raise ValueError("input (%s) and weight (%s) are on different devices" % (x2d.device, weight.device))
    if x2d.dim() != 2 or weight.dim() != 2 or x2d.shape[1] != weight.shape[1]:
        raise ValueError("expected x (tokens x in) and weight (out x in)")
    if not (x2d.is_contiguous() and weight.is_contiguous()):
        raise ValueError("input and weight must be contiguous")


class SparseLinearFunction(torch.autograd.Function):
    """Y = X W_hat^T with W_hat the transposable 2:4 pruning of W (see the module docstring)."""

    @staticmethod
    def forward(ctx, x2d, weight, mask_weight_grad=False):
        _check_operands(x2d, weight)
        out_f, in_f = weight.shape
        tokens = x2d.shape[0]
        plans = _plans(out_f, in_f, tokens, _DTYPE_NAMES[weight.dtype])
        w_hat = torch.empty_like(weight)
        keep = plans.fwd.empty_mask() if mask_weight_grad else None
        nm_prune(plans.fwd, weight, w_hat, "tile", keep)
        v_fwd, m_fwd = plans.fwd.empty_values(), plans.fwd.empty_meta()
        nm_compress(plans.fwd, w_hat, v_fwd, m_fwd)
        v_bwd, m_bwd = plans.bwd.empty_values(), plans.bwd.empty_meta()
        nm_compress(plans.bwd, w_hat, v_bwd, m_bwd)
        y = torch.empty((tokens, out_f), dtype=weight.dtype, device=weight.device)
        nm_spmm(plans.fwd, 1.0, v_fwd, m_fwd, x2d, 0.0, None, y)
        ctx.save_for_backward(x2d, v_bwd, m_bwd, keep if keep is not None else torch.empty(0, device=x2d.device))
        ctx.plans = plans
        ctx.shape = (tokens, out_f, in_f)
        ctx.mask_weight_grad = mask_weight_grad
        return y

    @staticmethod
    def backward(ctx, dy):
        x2d, v_bwd, m_bwd, keep = ctx.saved_tensors
        tokens, out_f, in_f = ctx.shape
        if dy.dtype != x2d.dtype or not dy.is_cuda or dy.device != x2d.device or tuple(dy.shape) != (tokens, out_f):
            raise ValueError("output gradient must be a (tokens x out) GPU tensor of the layer's dtype and device")
        dy = dy.contiguous()
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dx = torch.empty((tokens, in_f), dtype=dy.dtype, device=dy.device)
            nm_spmm(ctx.plans.bwd, 1.0, v_bwd, m_bwd, dy, 0.0, None, dx)
        if ctx.needs_input_grad[1]:
            dw = torch.empty((out_f, in_f), dtype=dy.dtype, device=dy.device)
            nm_dense_gemm(ctx.plans.dw, 1.0, dy, x2d, 0.0, None, dw)
            if ctx.mask_weight_grad:
                nm_mask_apply(ctx.plans.fwd, keep, dw)
        return dx, dw, None


class SemiStructuredSparseLinear(torch.nn.Module):
    """Linear layer without bias whose dense weight is pruned to transposable 2:4
    and compressed at every forward; forward and input-gradient products run on
    the 2:4 SpMM, the weight gradient on the dense product."""

    def __init__(self, in_features, out_features, dtype=torch.float16, device="cuda", weight=None,
                 mask_weight_grad=False):
        super().__init__()
        self.mask_weight_grad = bool(mask_weight_grad)
        if dtype not in _DTYPE_NAMES:
            raise ValueError("dtype must be torch.float16 or torch.bfloat16")
        if weight is None and torch.device(device).type != "cuda":
            raise ValueError("the layer runs on the GPU: device must be a cuda device")
        if in_features % 8 or out_features % 8:
            raise ValueError("in_features and out_features must be multiples of 8")
        self.in_features, self.out_features = in_features, out_features
        if weight is None:
            weight = torch.empty((out_features, in_features), dtype=dtype, device=device)
            torch.nn.init.normal_(weight, std=0.02)
        elif tuple(weight.shape) != (out_features, in_features) or weight.dtype != dtype:
            raise ValueError("weight must be (out_features, in_features) of the layer's dtype")
        if not weight.is_cuda:
            raise ValueError("the weight must live on the GPU (the library's kernels read it in place)")
        self.weight = torch.nn.Parameter(weight.contiguous())

    def forward(self, x):
        if x.shape[-1] != self.in_features:
            raise ValueError("last dimension of x must be in_features")
        x2d = x.reshape(-1, self.in_features).contiguous()
        if x2d.shape[0] % 4:
            raise ValueError("the number of tokens must be a multiple of 4")
        _check_operands(x2d, self.weight)
        y = SparseLinearFunction.apply(x2d, self.weight, self.mask_weight_grad)
        return y.reshape(*x.shape[:-1], self.out_features)
