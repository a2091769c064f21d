"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/nmsparse.h declares, validates problems and arguments before
anything is enqueued, and computes the compressed sizes of the documented layout."""
import ctypes
import os
import re

import pytest

import oracle
import structured_sparse_gemm_nm_amd as nm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nmsparse.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nm_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 14
    L = ctypes.CDLL(nm.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_status_strings_and_version():
    for s in range(6):
        assert nm.nm_status_string(s).startswith("NM_")
    assert nm.nm_version() >= 10000


def _init(**kw):
    base = dict(m=64, n=32, k=128, nm_n=2, nm_m=4, op_a="N", op_b="N", dtype="f16")
    base.update(kw)
    return nm.nm_plan_init(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(nm_m=5), nm.NM_ERR_INVALID_ARG),
    (dict(nm_m=64), nm.NM_ERR_INVALID_ARG),
    (dict(nm_n=0), nm.NM_ERR_INVALID_ARG),
    (dict(nm_n=4, nm_m=4), nm.NM_ERR_INVALID_ARG),
    (dict(k=130), nm.NM_ERR_SHAPE),
    (dict(nm_n=4, nm_m=32, k=48), nm.NM_ERR_SHAPE),
    (dict(m=-1), nm.NM_ERR_SHAPE),
    (dict(lda=100), nm.NM_ERR_SHAPE),            # lda < k
    (dict(lda=132), nm.NM_ERR_ALIGN),            # 264-byte rows are not 16-byte multiples
    (dict(ldb=36), nm.NM_ERR_ALIGN),             # B rows 32 elements, ld 36 -> 72 bytes
    (dict(ldc=20), nm.NM_ERR_SHAPE),             # ldc < n
])
def test_plan_init_rejects(kw, status):
    with pytest.raises(nm.NmError) as e:
        _init(**kw)
    assert e.value.status == status


def test_plan_init_rejects_bad_type_pair_and_order():
    p = nm.nm_problem_t()
    p.m, p.n, p.k, p.nm_n, p.nm_m = 16, 16, 16, 2, 4
    p.lda, p.ldb, p.ldc, p.ldd = 16, 16, 16, 16
    h = ctypes.c_void_p()
    p.type_ab, p.type_cd = nm.NM_F16, nm.NM_I32
    assert nm.lib().nm_plan_init(ctypes.byref(h), ctypes.byref(p)) == nm.NM_ERR_INVALID_ARG
    assert h.value is None
    p.type_cd = nm.NM_F16
    p.order_cd = 2
    assert nm.lib().nm_plan_init(ctypes.byref(h), ctypes.byref(p)) == nm.NM_ERR_INVALID_ARG
    p.order_cd = 0
    p.vector_rows = 7                                        # not a power of two
    assert nm.lib().nm_plan_init(ctypes.byref(h), ctypes.byref(p)) == nm.NM_ERR_INVALID_ARG
    p.vector_rows = 512                                      # above 256
    assert nm.lib().nm_plan_init(ctypes.byref(h), ctypes.byref(p)) == nm.NM_ERR_INVALID_ARG
    p.vector_rows = 32                                       # m = 16 is not a multiple of 32
    assert nm.lib().nm_plan_init(ctypes.byref(h), ctypes.byref(p)) == nm.NM_ERR_SHAPE
    p.vector_rows, p.op_a, p.lda = 16, nm.NM_OP_T, 16        # vector-wise needs op_a = N
    assert nm.lib().nm_plan_init(ctypes.byref(h), ctypes.byref(p)) == nm.NM_ERR_UNSUPPORTED
    p.vector_rows, p.op_a = 0, nm.NM_OP_N
    assert nm.lib().nm_plan_init(None, ctypes.byref(p)) == nm.NM_ERR_INVALID_ARG
    assert nm.lib().nm_plan_init(ctypes.byref(h), None) == nm.NM_ERR_INVALID_ARG


def test_column_major_cd_leading_dimensions():
    # column-major C/D: ld counts rows (>= m), and columns of >= 16 bytes start on 16-byte boundaries
    _init(m=24, n=40, order_cd="col")
    _init(m=24, n=40, ldc=32, ldd=40, order_cd="col")
    with pytest.raises(nm.NmError) as e:
        _init(m=24, n=40, ldd=16, order_cd="col")             # ldd < m
    assert e.value.status == nm.NM_ERR_SHAPE
    with pytest.raises(nm.NmError) as e:
        _init(m=24, n=40, ldd=28, order_cd="col")             # 56-byte column stride
    assert e.value.status == nm.NM_ERR_ALIGN
    _init(m=4, n=40, ldc=5, ldd=7, order_cd="col")            # 8-byte columns: any ld >= m
    with pytest.raises(ValueError):
        _init(m=4, n=4, order_cd="diagonal")


def test_small_rows_may_use_any_leading_dimension():
    # rows shorter than 16 bytes (n = 1, 4 fp16) need no alignment of ld
    _init(n=1, ldb=1, ldc=1, ldd=1)
    _init(n=4, ldb=5, ldc=6, ldd=7)


@pytest.mark.parametrize("dtype,N,M,k", [("f16", 2, 4, 4096), ("bf16", 2, 4, 11008), ("i8", 2, 4, 4096),
                                         ("f16", 4, 32, 4096), ("f16", 8, 32, 4096), ("f16", 3, 8, 96),
                                         ("i8", 5, 16, 48), ("f16", 1, 4, 4), ("bf16", 31, 32, 64)])
def test_compressed_sizes_match_layout_definition(dtype, N, M, k):
    plan = _init(m=7, n=3, k=k, nm_n=N, nm_m=M, dtype=dtype)
    assert plan.values_ld == oracle.values_ld(k, N, M, dtype)
    assert plan.meta_ld == oracle.meta_ld(k, N, M)
    es = 1 if dtype == "i8" else 2
    assert plan.values_bytes == 7 * plan.values_ld * es
    assert plan.meta_bytes == 7 * plan.meta_ld
    assert (plan.values_ld * es) % 16 == 0 and plan.meta_ld % 16 == 0


def test_mask_size():
    plan = _init(m=40, k=100 * 4, op_a="N")
    assert plan.mask_ld_words == (400 + 31) // 32 and plan.mask_bytes == 40 * plan.mask_ld_words * 4
    plan_t = _init(m=40, k=400, op_a="T", lda=40)
    assert plan_t.mask_ld_words == 2 and plan_t.mask_bytes == 400 * 2 * 4


def test_kernel_choice():
    assert _init(n=64).kernel_name == "spmm_smfmac_2of4"
    assert _init(n=8).kernel_name == "spmm_skinny"
    assert _init(n=64, nm_n=4, nm_m=32, k=128).kernel_name == "spmm_gather_mfma"


def test_calls_reject_bad_arguments_before_launching():
    plan = _init()
    L = nm.lib()
    one = ctypes.c_float(1.0)
    half = ctypes.c_float(0.5)
    P = ctypes.c_void_p
    fake = P(0x10000)             # never dereferenced: every call below fails validation first
    odd = P(0x10008)              # not 16-byte aligned
    assert L.nm_prune(plan.handle, fake, fake, 7, None, None) == nm.NM_ERR_INVALID_ARG
    assert L.nm_prune(plan.handle, None, fake, 0, None, None) == nm.NM_ERR_INVALID_ARG
    assert L.nm_prune(plan.handle, odd, fake, 0, None, None) == nm.NM_ERR_ALIGN
    assert L.nm_prune(None, fake, fake, 0, None, None) == nm.NM_ERR_INVALID_ARG
    assert L.nm_compress(plan.handle, fake, None, fake, None) == nm.NM_ERR_INVALID_ARG
    assert L.nm_decompress(plan.handle, fake, fake, odd, None) == nm.NM_ERR_ALIGN
    assert L.nm_prune_check(plan.handle, fake, 0, None, None) == nm.NM_ERR_INVALID_ARG
    spmm = L.nm_spmm
    assert spmm(plan.handle, None, fake, fake, fake, ctypes.byref(one), None, fake, None, None) == nm.NM_ERR_INVALID_ARG
    assert spmm(plan.handle, ctypes.byref(one), fake, fake, fake, ctypes.byref(one), None, fake, None, None) == nm.NM_ERR_INVALID_ARG  # beta != 0, C NULL
    splan = _init(m=256, n=256, k=1024, op_b="T")
    nm.nm_plan_set_split_k(splan, 2)
    zero = ctypes.byref(ctypes.c_float(0.0))
    assert spmm(splan.handle, ctypes.byref(one), fake, fake, fake, zero, None, fake, None, None) == nm.NM_ERR_INVALID_ARG  # workspace missing
    assert "workspace" in nm.nm_last_error()
    assert spmm(splan.handle, ctypes.byref(one), fake, fake, fake, zero, None, fake, odd, None) == nm.NM_ERR_ALIGN
    assert spmm(plan.handle, ctypes.byref(one), fake, odd, fake, ctypes.byref(ctypes.c_float(0.0)), None, fake, None, None) == nm.NM_ERR_ALIGN
    assert spmm(plan.handle, ctypes.byref(ctypes.c_float(float("nan"))), fake, fake, fake, ctypes.byref(one), fake, fake, None, None) == nm.NM_ERR_INVALID_ARG
    iplan = _init(dtype="i8")
    assert spmm(iplan.handle, ctypes.byref(half), fake, fake, fake, ctypes.byref(one), fake, fake, None, None) == nm.NM_ERR_INVALID_ARG
    tplan = _init(nm_n=1, nm_m=4)
    assert L.nm_prune(tplan.handle, fake, fake, nm.NM_PRUNE_TILE4X4, None, None) == nm.NM_ERR_INVALID_ARG
    t2 = _init(m=66, k=128)
    assert L.nm_prune(t2.handle, fake, fake, nm.NM_PRUNE_TILE4X4, None, None) == nm.NM_ERR_SHAPE
    assert nm.nm_last_error() != ""


def test_empty_problems_enqueue_nothing():
    # m = 0 or n = 0: valid plans, and the calls return before any device work
    for kw in (dict(m=0), dict(n=0)):
        plan = _init(**kw)
        nm.nm_spmm(plan, 1.0, None, None, None, 0.0, None, None, stream=0)
    plan = _init(m=0)
    nm.nm_compress(plan, None, None, None, stream=0)
    nm.nm_decompress(plan, None, None, None, stream=0)
    nm.nm_prune(plan, None, None, stream=0)


def test_sparse_linear_validates_on_host():
    # shape errors are raised before any device work
    import torch
    from structured_sparse_gemm_nm_amd.linear import SemiStructuredSparseLinear
    with pytest.raises(ValueError):
        SemiStructuredSparseLinear(100, 64)
    with pytest.raises(ValueError):
        SemiStructuredSparseLinear(64, 64, dtype=torch.float32)


def test_sparse_linear_refuses_host_tensors_and_dtype_mismatch(monkeypatch):
    """Host tensors, mixed devices and mixed dtypes are refused before any
    library call (the library would read a host address as device memory)."""
    import torch
    import structured_sparse_gemm_nm_amd.linear as lin
    from structured_sparse_gemm_nm_amd.linear import SemiStructuredSparseLinear, SparseLinearFunction

    def no_call(*a, **k):
        raise AssertionError("a library call was made")
    for name in ("nm_prune", "nm_compress", "nm_spmm", "nm_dense_gemm", "nm_plan_init"):
        monkeypatch.setattr(lin, name, no_call)
    w = torch.zeros((16, 32), dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        SparseLinearFunction.apply(torch.zeros((8, 32), dtype=torch.float16), w)
    with pytest.raises(ValueError, match="dtype"):
        SparseLinearFunction.apply(torch.zeros((8, 32), dtype=torch.float32), w)
    with pytest.raises(ValueError, match="dtype"):
        SparseLinearFunction.apply(torch.zeros((8, 32), dtype=torch.bfloat16), w)
    with pytest.raises(ValueError):
        SparseLinearFunction.apply(torch.zeros((8, 32), dtype=torch.float32), w.float())
    with pytest.raises(ValueError, match="cuda"):
        SemiStructuredSparseLinear(32, 16, device="cpu")
    with pytest.raises(ValueError, match="GPU"):
        SemiStructuredSparseLinear(32, 16, weight=w)


def test_algorithm_ids_validate_on_host():
    plan = _init()
    assert nm.nm_plan_algorithm_count(plan) == nm.NM_ALG_COUNT == 4
    assert nm.nm_plan_get_algorithm(plan) == nm.NM_ALG_AUTO
    for alg in range(nm.NM_ALG_COUNT):
        nm.nm_plan_set_algorithm(plan, alg)
        assert nm.nm_plan_get_algorithm(plan) == alg
    for bad in (-1, nm.NM_ALG_COUNT):
        with pytest.raises(nm.NmError) as e:
            nm.nm_plan_set_algorithm(plan, bad)
        assert e.value.status == nm.NM_ERR_INVALID_ARG
    assert nm.nm_plan_get_algorithm(plan) == nm.NM_ALG_COUNT - 1     # unchanged by the rejected ids


def test_split_k_settings_and_workspace_size():
    """Split-k is a host-side plan setting; the workspace size is one m x n plane
    of 4-byte partial sums per k range, only where the whole-tile 2:4 kernel runs."""
    plan = _init(m=256, n=256, k=1024, op_b="T")            # 16 k-steps of 64
    assert nm.nm_plan_get_split_k(plan) == (1, 1)
    assert nm.nm_spmm_workspace_size(plan) == 0
    nm.nm_plan_set_split_k(plan, 4)
    assert nm.nm_plan_get_split_k(plan) == (4, 4)
    assert nm.nm_spmm_workspace_size(plan) == 4 * 256 * 256 * 4
    nm.nm_plan_set_split_k(plan, 16)
    assert nm.nm_plan_get_split_k(plan) == (16, 16)
    for bad in (0, -1, 17):
        with pytest.raises(nm.NmError) as e:
            nm.nm_plan_set_split_k(plan, bad)
        assert e.value.status == nm.NM_ERR_INVALID_ARG
    assert nm.nm_plan_get_split_k(plan) == (16, 16)         # unchanged by the rejected values
    short = _init(m=256, n=256, k=192, op_b="T")            # 3 k-steps: the split is clamped
    nm.nm_plan_set_split_k(short, 8)
    assert nm.nm_plan_get_split_k(short) == (8, 3)
    assert nm.nm_spmm_workspace_size(short) == 3 * 256 * 256 * 4
    i8 = _init(m=256, n=256, k=1024, dtype="i8")            # int8 k-steps are 128 long: 8 of them
    nm.nm_plan_set_split_k(i8, 16)
    assert nm.nm_plan_get_split_k(i8) == (16, 8)
    # shapes the split does not apply to need no workspace
    for kw in (dict(m=200, n=144, k=336), dict(m=256, n=256, k=1024, nm_n=4, nm_m=32), dict(m=256, n=8, k=1024)):
        p = _init(**kw)
        nm.nm_plan_set_split_k(p, 4)
        assert nm.nm_plan_get_split_k(p)[1] == 1 and nm.nm_spmm_workspace_size(p) == 0, kw


def test_noalloc_refuses_splits_beyond_its_scratch():
    """nm_spmm_noalloc checks the split-k workspace against its static scratch
    before any device call (the fake pointers below are never touched)."""
    L = nm.lib()
    big = _init(m=2048, n=2048, k=4096, op_b="T")
    nm.nm_plan_set_split_k(big, 4)                            # 64 MiB of partial sums
    assert nm.nm_spmm_workspace_size(big) == 4 * 2048 * 2048 * 4 > nm.NM_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x10000)
    one, zero = ctypes.c_float(1.0), ctypes.c_float(0.0)
    st = L.nm_spmm_noalloc(big.handle, ctypes.byref(one), fake, fake, fake, ctypes.byref(zero), None, fake, None)
    assert st == nm.NM_ERR_SHAPE
    assert "scratch" in nm.nm_last_error()
    assert L.nm_spmm_noalloc(None, ctypes.byref(one), fake, fake, fake, ctypes.byref(zero), None, fake, None) \
        == nm.NM_ERR_INVALID_ARG
