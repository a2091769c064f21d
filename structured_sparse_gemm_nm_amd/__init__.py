"""Python binding for libnmsparse (N:M structured-sparse GEMM on MI355X).

Argument marshalling only: torch tensors become device pointers
(``tensor.data_ptr()``) and the current HIP stream becomes a ``void*``; every
step of the path runs in the library's HIP kernels. The names mirror the C ABI
in include/nmsparse.h, whose comments define each operation.

The binding refuses to run without the built library: there is no CPU or
PyTorch fallback.
"""
import ctypes
import os

import torch  # loaded first so the library binds to torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnmsparse.so")

NM_OK, NM_ERR_INVALID_ARG, NM_ERR_SHAPE, NM_ERR_ALIGN, NM_ERR_UNSUPPORTED, NM_ERR_HIP = range(6)
NM_F16, NM_BF16, NM_I8, NM_I32 = range(4)
NM_OP_N, NM_OP_T = 0, 1
NM_PRUNE_1D, NM_PRUNE_TILE4X4 = 0, 1

DTYPES = {"f16": (NM_F16, NM_F16), "bf16": (NM_BF16, NM_BF16), "i8": (NM_I8, NM_I32)}
TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8, "i32": torch.int32}
MODES = {"1d": NM_PRUNE_1D, "tile": NM_PRUNE_TILE4X4}


class NmError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s (%s)" % (message, _status_name(status)))
        self.status = status


class nm_problem_t(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("nm_n", ctypes.c_int32), ("nm_m", ctypes.c_int32),
                ("op_a", ctypes.c_int32), ("op_b", ctypes.c_int32),
                ("type_ab", ctypes.c_int32), ("type_cd", ctypes.c_int32),
                ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldc", ctypes.c_int64), ("ldd", ctypes.c_int64),
                ("order_cd", ctypes.c_int32), ("vector_rows", ctypes.c_int32)]


_lib = None


def lib():
    """Load libnmsparse.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libnmsparse.so is not built (run __graft_entry__.build() or "
                               "python structured_sparse_gemm_nm_amd/build.py); no fallback exists")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        st = ctypes.c_int
        L.nm_plan_init.restype = st; L.nm_plan_init.argtypes = [ctypes.POINTER(P), ctypes.POINTER(nm_problem_t)]
        L.nm_plan_destroy.restype = st; L.nm_plan_destroy.argtypes = [P]
        L.nm_compressed_size.restype = st
        L.nm_compressed_size.argtypes = [P, ctypes.POINTER(S), ctypes.POINTER(S), ctypes.POINTER(I64), ctypes.POINTER(I64)]
        L.nm_mask_size.restype = st; L.nm_mask_size.argtypes = [P, ctypes.POINTER(S), ctypes.POINTER(I64)]
        L.nm_prune.restype = st; L.nm_prune.argtypes = [P, P, P, I32, P, P]
        L.nm_prune_check.restype = st; L.nm_prune_check.argtypes = [P, P, I32, P, P]
        L.nm_mask_apply.restype = st; L.nm_mask_apply.argtypes = [P, P, P, P]
        L.nm_compress.restype = st; L.nm_compress.argtypes = [P, P, P, P, P]
        L.nm_decompress.restype = st; L.nm_decompress.argtypes = [P, P, P, P, P]
        FP = ctypes.POINTER(ctypes.c_float)
        L.nm_spmm.restype = st; L.nm_spmm.argtypes = [P, FP, P, P, P, FP, P, P, P, P]
        L.nm_dense_gemm.restype = st; L.nm_dense_gemm.argtypes = [P, FP, P, P, FP, P, P, P]
        L.nm_plan_kernel_name.restype = ctypes.c_char_p; L.nm_plan_kernel_name.argtypes = [P]
        L.nm_plan_algorithm_count.restype = I32; L.nm_plan_algorithm_count.argtypes = [P]
        L.nm_plan_set_algorithm.restype = st; L.nm_plan_set_algorithm.argtypes = [P, I32]
        L.nm_plan_get_algorithm.restype = st; L.nm_plan_get_algorithm.argtypes = [P, ctypes.POINTER(I32)]
        L.nm_plan_spmm_kernel.restype = ctypes.c_char_p; L.nm_plan_spmm_kernel.argtypes = [P]
        L.nm_plan_set_split_k.restype = st; L.nm_plan_set_split_k.argtypes = [P, I32]
        L.nm_plan_get_split_k.restype = st
        L.nm_plan_get_split_k.argtypes = [P, ctypes.POINTER(I32), ctypes.POINTER(I32)]
        L.nm_spmm_workspace_size.restype = st; L.nm_spmm_workspace_size.argtypes = [P, ctypes.POINTER(S)]
        L.nm_spmm_noalloc.restype = st; L.nm_spmm_noalloc.argtypes = [P, FP, P, P, P, FP, P, P, P]
        L.nm_spmm_streams.restype = st
        L.nm_spmm_streams.argtypes = [P, FP, P, P, P, FP, P, P, P, ctypes.POINTER(P), I32]
        L.nm_status_string.restype = ctypes.c_char_p; L.nm_status_string.argtypes = [st]
        L.nm_last_error.restype = ctypes.c_char_p; L.nm_last_error.argtypes = []
        L.nm_version.restype = I32; L.nm_version.argtypes = []
        _lib = L
    return _lib


def _status_name(s):
    try:
        return lib().nm_status_string(s).decode()
    except Exception:
        return str(s)


def _check(status):
    if status != NM_OK:
        raise NmError(status, lib().nm_last_error().decode() or "nmsparse call failed")


def _ptr(x):
    """Tensor or int (raw device address) or None -> c_void_p."""
    if x is None:
        return None
    if isinstance(x, int):
        return ctypes.c_void_p(x)
    return ctypes.c_void_p(x.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


class Plan:
    """Owns an nm_plan_t. Attributes mirror the size queries."""

    def __init__(self, handle, problem, dtype):
        self.handle = handle
        self.problem = problem
        self.dtype = dtype
        vb, mb = ctypes.c_size_t(), ctypes.c_size_t()
        vl, ml = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().nm_compressed_size(handle, ctypes.byref(vb), ctypes.byref(mb), ctypes.byref(vl), ctypes.byref(ml)))
        self.values_bytes, self.meta_bytes = vb.value, mb.value
        self.values_ld, self.meta_ld = vl.value, ml.value
        kb, kl = ctypes.c_size_t(), ctypes.c_int64()
        _check(lib().nm_mask_size(handle, ctypes.byref(kb), ctypes.byref(kl)))
        self.mask_bytes, self.mask_ld_words = kb.value, kl.value
        self.kernel_name = lib().nm_plan_kernel_name(handle).decode()

    @property
    def m(self):
        return self.problem.m

    @property
    def n(self):
        return self.problem.n

    @property
    def k(self):
        return self.problem.k

    @property
    def spmm_kernel(self):
        """Device kernel nm_spmm launches for this plan (profiler naming)."""
        return lib().nm_plan_spmm_kernel(self.handle).decode()

    def destroy(self):
        if self.handle is not None:
            lib().nm_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    # allocation helpers (torch owns the memory; the library never allocates)
    def empty_values(self, device="cuda"):
        dt = TORCH_DTYPES[self.dtype]
        return torch.empty((self.m, self.values_ld), dtype=dt, device=device)

    @property
    def vector_rows(self):
        return max(1, self.problem.vector_rows)

    def empty_meta(self, device="cuda"):
        return torch.empty((self.m // self.vector_rows, self.meta_ld), dtype=torch.uint8, device=device)

    def empty_workspace(self, device="cuda"):
        """Workspace nm_spmm needs for this plan's split-k setting (None when it needs none)."""
        n = nm_spmm_workspace_size(self)
        return torch.empty((n,), dtype=torch.uint8, device=device) if n else None

    def empty_mask(self, device="cuda"):
        rows = self.problem.m if self.problem.op_a == NM_OP_N else self.problem.k
        return torch.empty((rows, self.mask_ld_words), dtype=torch.int32, device=device)


def nm_plan_init(m, n, k, nm_n=2, nm_m=4, op_a="N", op_b="N", dtype="f16", lda=None, ldb=None, ldc=None, ldd=None,
                 order_cd="row", out_dtype=None, vector_rows=0):
    """Validate a problem and return a Plan (host only). order_cd: "row" or "col" (C and D storage).
    out_dtype: C/D type when it differs from the default of `dtype` ("i8" with dtype "i8": saturated int8 D).
    vector_rows: V > 1 for vector-wise N:M (V consecutive rows share their kept offsets)."""
    ta, tc = DTYPES[dtype]
    if out_dtype is not None:
        tc = {"f16": NM_F16, "bf16": NM_BF16, "i8": NM_I8, "i32": NM_I32}[out_dtype]
    oa = NM_OP_T if op_a == "T" else NM_OP_N
    ob = NM_OP_T if op_b == "T" else NM_OP_N
    p = nm_problem_t()
    p.m, p.n, p.k = m, n, k
    p.nm_n, p.nm_m = nm_n, nm_m
    p.op_a, p.op_b = oa, ob
    p.type_ab, p.type_cd = ta, tc
    p.lda = lda if lda is not None else max(1, k if oa == NM_OP_N else m)
    p.ldb = ldb if ldb is not None else max(1, n if ob == NM_OP_N else k)
    if order_cd not in ("row", "col"):
        raise ValueError("order_cd must be 'row' or 'col'")
    cd_len = m if order_cd == "col" else n
    p.ldc = ldc if ldc is not None else max(1, cd_len)
    p.ldd = ldd if ldd is not None else max(1, cd_len)
    p.order_cd, p.vector_rows = (1 if order_cd == "col" else 0), int(vector_rows)
    h = ctypes.c_void_p()
    _check(lib().nm_plan_init(ctypes.byref(h), ctypes.byref(p)))
    return Plan(h, p, dtype)


def nm_plan_destroy(plan):
    plan.destroy()


def nm_compressed_size(plan):
    return plan.values_bytes, plan.meta_bytes, plan.values_ld, plan.meta_ld


def nm_mask_size(plan):
    return plan.mask_bytes, plan.mask_ld_words


def nm_prune(plan, dA, dA_pruned, mode="1d", d_mask=None, stream=None):
    _check(lib().nm_prune(plan.handle, _ptr(dA), _ptr(dA_pruned), MODES[mode], _ptr(d_mask), _stream(stream)))


def nm_mask_apply(plan, d_mask, dX, stream=None):
    _check(lib().nm_mask_apply(plan.handle, _ptr(d_mask), _ptr(dX), _stream(stream)))


def nm_prune_check(plan, dA, mode, d_violations, stream=None):
    _check(lib().nm_prune_check(plan.handle, _ptr(dA), MODES[mode], _ptr(d_violations), _stream(stream)))


def nm_compress(plan, dA, d_values, d_meta, stream=None):
    _check(lib().nm_compress(plan.handle, _ptr(dA), _ptr(d_values), _ptr(d_meta), _stream(stream)))


def nm_decompress(plan, d_values, d_meta, dA_out, stream=None):
    _check(lib().nm_decompress(plan.handle, _ptr(d_values), _ptr(d_meta), _ptr(dA_out), _stream(stream)))


def nm_spmm(plan, alpha, d_values, d_meta, dB, beta, dC, dD, stream=None, workspace=None):
    """workspace: device buffer of at least nm_spmm_workspace_size(plan) bytes (split-k plans)."""
    a, b = ctypes.c_float(alpha), ctypes.c_float(beta)
    _check(lib().nm_spmm(plan.handle, ctypes.byref(a), _ptr(d_values), _ptr(d_meta), _ptr(dB), ctypes.byref(b),
                         _ptr(dC), _ptr(dD), _ptr(workspace), _stream(stream)))


def nm_spmm_streams(plan, alpha, d_values, d_meta, dB, beta, dC, dD, streams, workspace=None):
    """nm_spmm with the rows of D split over `streams` (torch streams or raw handles)."""
    a, b = ctypes.c_float(alpha), ctypes.c_float(beta)
    arr = (ctypes.c_void_p * len(streams))(*[_stream(s_).value for s_ in streams])
    _check(lib().nm_spmm_streams(plan.handle, ctypes.byref(a), _ptr(d_values), _ptr(d_meta), _ptr(dB), ctypes.byref(b),
                                 _ptr(dC), _ptr(dD), _ptr(workspace), arr, len(streams)))


NM_NOALLOC_SCRATCH_BYTES = 32 << 20


def nm_spmm_noalloc(plan, alpha, d_values, d_meta, dB, beta, dC, dD, stream=None):
    """nm_spmm with the split-k partial sums in the library's static device scratch (no workspace)."""
    a, b = ctypes.c_float(alpha), ctypes.c_float(beta)
    _check(lib().nm_spmm_noalloc(plan.handle, ctypes.byref(a), _ptr(d_values), _ptr(d_meta), _ptr(dB),
                                 ctypes.byref(b), _ptr(dC), _ptr(dD), _stream(stream)))


def nm_plan_set_split_k(plan, splits):
    _check(lib().nm_plan_set_split_k(plan.handle, int(splits)))


def nm_plan_get_split_k(plan):
    """(requested, effective) split-k of the plan."""
    r, e = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().nm_plan_get_split_k(plan.handle, ctypes.byref(r), ctypes.byref(e)))
    return r.value, e.value


def nm_spmm_workspace_size(plan):
    n = ctypes.c_size_t()
    _check(lib().nm_spmm_workspace_size(plan.handle, ctypes.byref(n)))
    return n.value


def nm_dense_gemm(plan, alpha, dA, dB, beta, dC, dD, stream=None):
    a, b = ctypes.c_float(alpha), ctypes.c_float(beta)
    _check(lib().nm_dense_gemm(plan.handle, ctypes.byref(a), _ptr(dA), _ptr(dB), ctypes.byref(b), _ptr(dC), _ptr(dD),
                               _stream(stream)))


NM_ALG_AUTO, NM_ALG_TILE128, NM_ALG_TILE256X128, NM_ALG_TILE256, NM_ALG_COUNT = range(5)


def nm_plan_algorithm_count(plan):
    return lib().nm_plan_algorithm_count(plan.handle)


def nm_plan_set_algorithm(plan, alg):
    _check(lib().nm_plan_set_algorithm(plan.handle, int(alg)))


def nm_plan_get_algorithm(plan):
    a = ctypes.c_int32()
    _check(lib().nm_plan_get_algorithm(plan.handle, ctypes.byref(a)))
    return a.value


def nm_plan_spmm_kernel(plan):
    return plan.spmm_kernel


def nm_status_string(status):
    return lib().nm_status_string(status).decode()


def nm_last_error():
    return lib().nm_last_error().decode()


def nm_version():
    return lib().nm_version()
