"""GPU parity: every kernel behind the C ABI against the CPU oracle on seeded
inputs at sizes the oracle finishes in seconds, spanning several tiles and a
ragged tail. Masks, pruned matrices, values, metadata (padding included) and
int32 outputs must be bit-exact; fp16/bf16 outputs must satisfy
|D - D_ref| <= 1e-2 * (|alpha| (|A| |B|)_ij + |beta| |C_ij|) + 1e-3."""
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
NM_CASES = [(2, 4), (1, 4), (3, 4), (2, 8), (5, 16), (4, 32), (8, 32)]


def rand(dtype, shape, seed, sigma=1.0):
    if dtype == "i8":
        return inputs.uniform_int(shape, seed, -127, 127)
    return inputs.normal(shape, seed, sigma, dtype)


def stored(op, rows, cols):
    return (rows, cols) if op == "N" else (cols, rows)


TILE_ALG = {None: nm.NM_ALG_AUTO, "auto": nm.NM_ALG_AUTO, "128": nm.NM_ALG_TILE128,
            "256x128": nm.NM_ALG_TILE256X128, "256": nm.NM_ALG_TILE256}


def plan_for(dtype, m, n, k, N, M, op_a="N", op_b="N", tile=None, **kw):
    """A plan; `tile` pins the block tile through the plan's algorithm id."""
    plan = nm.nm_plan_init(m, n, k, N, M, op_a=op_a, op_b=op_b, dtype=dtype, **kw)
    nm.nm_plan_set_algorithm(plan, TILE_ALG[tile])
    return plan


# ------------------------------------------------------------------ prune / check / compress

@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("N,M", NM_CASES)
@pytest.mark.parametrize("op", ["N", "T"])
def test_prune_1d(dtype, N, M, op):
    m, k = 208, 544
    a = rand(dtype, stored(op, m, k), 10 + N * M)
    ref, keep = oracle.prune_1d(a, dtype, N, M, op)
    plan = plan_for(dtype, m, 8, k, N, M, op_a=op)
    da = dev(a)
    out = Guarded(a.shape, TRAW[dtype])
    mask = Guarded((plan.mask_bytes // 4,), torch.int32)
    nm.nm_prune(plan, da, out.t, "1d", mask.t)
    sync()
    out.check(); mask.check()
    assert np.array_equal(host(out.t, RAW[dtype]), ref)
    assert np.array_equal(host(mask.t, np.uint32).reshape(ref.shape[0], -1), oracle.mask_bits(keep))
    # in place
    nm.nm_prune(plan, da, da, "1d")
    sync()
    assert np.array_equal(host(da, RAW[dtype]), ref)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("shape", [(132, 272), (4, 4), (8, 1040)])
def test_prune_tile(dtype, shape):
    a = rand(dtype, shape, 77, 0.02)
    ref, keep = oracle.prune_tile(a, dtype)
    plan = plan_for(dtype, shape[0], 16, shape[1], 2, 4)
    out = Guarded(shape, TRAW[dtype])
    mask = Guarded((plan.mask_bytes // 4,), torch.int32)
    nm.nm_prune(plan, dev(a), out.t, "tile", mask.t)
    sync()
    out.check(); mask.check()
    assert np.array_equal(host(out.t, RAW[dtype]), ref)
    assert np.array_equal(host(mask.t, np.uint32).reshape(shape[0], -1), oracle.mask_bits(keep))
    # the tile result conforms in both directions; the original does not
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    nm.nm_prune_check(plan, out.t, "tile", cnt)
    sync()
    assert int(cnt.item()) == 0
    nm.nm_prune_check(plan, dev(a), "tile", cnt)
    sync()
    assert int(cnt.item()) == oracle.check_tile(a, dtype)


@pytest.mark.parametrize("dtype", ["f16", "i8"])
@pytest.mark.parametrize("N,M", NM_CASES)
@pytest.mark.parametrize("op", ["N", "T"])
def test_check_1d(dtype, N, M, op):
    m, k = 144, 352
    a = rand(dtype, stored(op, m, k), 5)
    a[:: 7] = 0                                           # some rows with no non-zeros at all
    plan = plan_for(dtype, m, 8, k, N, M, op_a=op)
    cnt = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    nm.nm_prune_check(plan, dev(a), "1d", cnt)
    sync()
    assert int(cnt.item()) == oracle.check_1d(a, dtype, N, M, op)
    p, _ = oracle.prune_1d(a, dtype, N, M, op)
    nm.nm_prune_check(plan, dev(p), "1d", cnt)
    sync()
    assert int(cnt.item()) == 0


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("N,M", NM_CASES + [(31, 32), (7, 8), (15, 16)])
@pytest.mark.parametrize("op", ["N", "T"])
def test_compress_decompress(dtype, N, M, op):
    m, k = 208, 544
    a = rand(dtype, stored(op, m, k), 20 + N + M)
    vref, mref = oracle.compress(a, dtype, N, M, op)
    plan = plan_for(dtype, m, 8, k, N, M, op_a=op)
    vals = Guarded((m, plan.values_ld), TRAW[dtype])
    meta = Guarded((m, plan.meta_ld), torch.uint8)
    nm.nm_compress(plan, dev(a), vals.t, meta.t)
    sync()
    vals.check(); meta.check()
    assert np.array_equal(host(vals.t, RAW[dtype]), vref)
    assert np.array_equal(host(meta.t, np.uint8), mref)
    # decompress the oracle's compressed form back to the stored layout
    dref = oracle.decompress(vref, mref, dtype, m, k, N, M, op)
    out = Guarded(a.shape, TRAW[dtype])
    nm.nm_decompress(plan, dev(vref), dev(mref), out.t)
    sync()
    out.check()
    assert np.array_equal(host(out.t, RAW[dtype]), dref)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("N,M", NM_CASES)
@pytest.mark.parametrize("path", ["row", "tile"])
def test_check_1d_ragged_padded(dtype, N, M, path, monkeypatch):
    """1-D prune check on padded rows (lda > k) with a ragged last 16-byte chunk,
    groups narrower and wider than 16 bytes, and planted violations."""
    if path == "tile":
        monkeypatch.setenv("NM_TILE_ELEMWISE", "1")
    es = 1 if dtype == "i8" else 2
    for m, groups in [(3, 1), (5, 67), (2, 261)]:
        k = groups * M
        lda = -(-k // (16 // es)) * (16 // es) + 16 // es
        full = rand(dtype, (m, lda), 900 + groups + M)
        a = np.ascontiguousarray(full[:, :k])
        plan = plan_for(dtype, m, 8, k, N, M, lda=lda)
        cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        nm.nm_prune_check(plan, dev(full), "1d", cnt)
        sync()
        assert int(cnt.item()) == oracle.check_1d(a, dtype, N, M), (m, k)
        p, _ = oracle.prune_1d(a, dtype, N, M)
        pf = full.copy()
        pf[:, :k] = p
        nm.nm_prune_check(plan, dev(pf), "1d", cnt)
        sync()
        assert int(cnt.item()) == 0, (m, k)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
def test_prune_tile_unaligned_short_rows(dtype):
    """Rows shorter than 16 bytes may use any leading dimension: ld = 5 leaves tile
    rows unaligned; padding columns untouched."""
    rows, cols, ld = 8, 4, 5
    full = rand(dtype, (rows, ld), 78, 0.02)
    a = np.ascontiguousarray(full[:, :cols])
    ref, _ = oracle.prune_tile(a, dtype)
    plan = plan_for(dtype, rows, 16, cols, 2, 4, lda=ld)
    out = Guarded((rows, ld), TRAW[dtype], fill=dev(full))
    nm.nm_prune(plan, dev(full), out.t, "tile")
    sync()
    out.check()
    got = host(out.t, RAW[dtype])
    assert np.array_equal(got[:, :cols], ref)
    assert np.array_equal(got[:, cols:], full[:, cols:])


def _lda_op_t(m, es, align):
    """A padded leading dimension: whole 16-byte rows plus one more piece, or rows
    that are 4-byte but not 8-byte aligned (lda * esize = 4 mod 8; plans allow
    that only for rows shorter than 16 bytes)."""
    if align == 16:
        return -(-m // (16 // es)) * (16 // es) + 16 // es
    lda = m + 1
    while (lda * es) % 8 != 4:
        lda += 1
    return lda


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("path,align", [("colT", 16), ("colT", 4), ("tile", 16)])
def test_compress_op_t_ragged_padded(dtype, path, align, monkeypatch):
    """2:4 compress and decompress with groups down stored columns (op_a = T), on
    padded stored rows: ragged column counts for the 8-byte lanes (rows 8-byte
    aligned) and the 4-byte ones (short rows 4-byte aligned only), a ragged last
    block of 32 stored rows (odd group counts), several blocks, and blocks
    staged through LDS (m >= 256) next to a ragged one."""
    if path == "tile":
        monkeypatch.setenv("NM_TILE_ELEMWISE", "1")
    es = 1 if dtype == "i8" else 2
    shapes = [(7, 4), (33, 100), (130, 268), (5, 36), (64, 96), (521, 268)]
    if align == 4:
        shapes = [(m, k) for m, k in [(7, 4), (5, 36), (3, 268), (7, 100), (13, 268)] if m * es < 16]
    for m, k in shapes:
        lda = _lda_op_t(m, es, align)
        full = rand(dtype, (k, lda), 700 + m + k)
        a = np.ascontiguousarray(full[:, :m])                  # stored k x m
        plan = plan_for(dtype, m, 8, k, 2, 4, op_a="T", lda=lda)
        vref, mref = oracle.compress(a, dtype, 2, 4, "T")
        vals = Guarded((m, plan.values_ld), TRAW[dtype], fill=torch.full((m, plan.values_ld), -1, dtype=TRAW[dtype]))
        meta = Guarded((m, plan.meta_ld), torch.uint8, fill=torch.full((m, plan.meta_ld), 0xEE, dtype=torch.uint8))
        nm.nm_compress(plan, dev(full), vals.t, meta.t)
        sync()
        vals.check(); meta.check()
        assert np.array_equal(host(vals.t, RAW[dtype]), vref), (m, k)
        assert np.array_equal(host(meta.t, np.uint8), mref), (m, k)
        sentinel = np.full((k, lda), 0x5A if es == 1 else 0x5A5A, dtype=RAW[dtype])
        out = Guarded((k, lda), TRAW[dtype], fill=dev(sentinel))
        nm.nm_decompress(plan, dev(vref), dev(mref), out.t)
        sync()
        out.check()
        got = host(out.t, RAW[dtype])
        assert np.array_equal(got[:, :m], oracle.decompress(vref, mref, dtype, m, k, 2, 4, "T")), (m, k)
        assert np.array_equal(got[:, m:], sentinel[:, m:]), (m, k)


ROW_NM = [(2, 4), (4, 32), (8, 32)]


def row_shapes(dtype, M):
    """(m, k) for the register path: one group; a ragged last 16-byte unit; a ragged
    last segment of 64 units; several whole segments plus a ragged one."""
    es = 1 if dtype == "i8" else 2
    gu = max(1, 16 // (M * es))                 # groups per 16-byte unit
    return [(3, M), (5, (gu * 64 + 1) * M), (4, 3 * M), (2, (gu * 64 * 3 + gu + 1) * M)]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("N,M", ROW_NM)
@pytest.mark.parametrize("path", ["row", "tile"])
def test_row_path_ragged(dtype, N, M, path, monkeypatch):
    """Prune, compress and decompress for op_a = N on padded rows (lda > k): the
    register path and, forced, the LDS tile path. Bytes between k and lda are the
    caller's and must be left alone."""
    if path == "tile":
        monkeypatch.setenv("NM_TILE_ELEMWISE", "1")
    es = 1 if dtype == "i8" else 2
    for (m, k) in row_shapes(dtype, M):
        lda = -(-k // (16 // es)) * (16 // es) + 16 // es
        full = rand(dtype, (m, lda), 600 + k + N)
        a = np.ascontiguousarray(full[:, :k])
        plan = plan_for(dtype, m, 8, k, N, M, lda=lda)
        ref, keep = oracle.prune_1d(a, dtype, N, M)
        sentinel = np.full((m, lda), 0x5A if es == 1 else 0x5A5A, dtype=RAW[dtype])
        out = Guarded((m, lda), TRAW[dtype], fill=dev(sentinel))
        mask = Guarded((plan.mask_bytes // 4,), torch.int32)
        nm.nm_prune(plan, dev(full), out.t, "1d", mask.t)
        sync()
        out.check(); mask.check()
        got = host(out.t, RAW[dtype])
        assert np.array_equal(got[:, :k], ref), (m, k)
        assert np.array_equal(got[:, k:], sentinel[:, k:]), (m, k)
        assert np.array_equal(host(mask.t, np.uint32).reshape(m, -1), oracle.mask_bits(keep)), (m, k)
        vref, mref = oracle.compress(a, dtype, N, M)
        vals = Guarded((m, plan.values_ld), TRAW[dtype], fill=torch.full((m, plan.values_ld), -1, dtype=TRAW[dtype]))
        meta = Guarded((m, plan.meta_ld), torch.uint8, fill=torch.full((m, plan.meta_ld), 0xEE, dtype=torch.uint8))
        nm.nm_compress(plan, dev(full), vals.t, meta.t)
        sync()
        vals.check(); meta.check()
        assert np.array_equal(host(vals.t, RAW[dtype]), vref), (m, k)
        assert np.array_equal(host(meta.t, np.uint8), mref), (m, k)
        dref = oracle.decompress(vref, mref, dtype, m, k, N, M)
        dec = Guarded((m, lda), TRAW[dtype], fill=dev(sentinel))
        nm.nm_decompress(plan, dev(vref), dev(mref), dec.t)
        sync()
        dec.check()
        got = host(dec.t, RAW[dtype])
        assert np.array_equal(got[:, :k], dref), (m, k)
        assert np.array_equal(got[:, k:], sentinel[:, k:]), (m, k)


# ------------------------------------------------------------------ ties, signed zeros, NaN

def tie_values(dtype, shape, seed):
    """Tie-heavy inputs: fp16/bf16 drawn from {0, -0, +-0.5, +-1, 2}, int8 from
    [-3, 3], so equal magnitudes (and +0 against -0) meet in most groups."""
    rng = np.random.default_rng(seed)
    if dtype == "i8":
        return rng.integers(-3, 4, size=shape).astype(np.int8)
    x = rng.choice(np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 2.0], np.float32), size=shape)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    return inputs._fp32_to_bf16_bits(x).reshape(shape)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("N,M", NM_CASES)
@pytest.mark.parametrize("op", ["N", "T"])
def test_ties_prune_check_compress_1d(dtype, N, M, op):
    """1-D prune, check and compress on tie-heavy inputs with signed zeros, bit for
    bit: ties go to the lower offset (select_topn for M <= 16, the selection
    network for M = 32 on the register path), +0 and -0 weigh the same."""
    m, k = 208, 544
    a = tie_values(dtype, stored(op, m, k), 31 + N * M)
    ref, keep = oracle.prune_1d(a, dtype, N, M, op)
    plan = plan_for(dtype, m, 8, k, N, M, op_a=op)
    out = Guarded(a.shape, TRAW[dtype])
    mask = Guarded((plan.mask_bytes // 4,), torch.int32)
    nm.nm_prune(plan, dev(a), out.t, "1d", mask.t)
    sync()
    out.check(); mask.check()
    assert np.array_equal(host(out.t, RAW[dtype]), ref)
    assert np.array_equal(host(mask.t, np.uint32).reshape(ref.shape[0], -1), oracle.mask_bits(keep))
    cnt = torch.full((1,), 777, dtype=torch.int32, device="cuda")
    nm.nm_prune_check(plan, dev(a), "1d", cnt)
    sync()
    assert int(cnt.item()) == oracle.check_1d(a, dtype, N, M, op)
    vref, mref = oracle.compress(a, dtype, N, M, op)
    vals = Guarded((m, plan.values_ld), TRAW[dtype])
    meta = Guarded((m, plan.meta_ld), torch.uint8)
    nm.nm_compress(plan, dev(a), vals.t, meta.t)
    sync()
    vals.check(); meta.check()
    assert np.array_equal(host(vals.t, RAW[dtype]), vref)
    assert np.array_equal(host(meta.t, np.uint8), mref)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
def test_ties_prune_tile(dtype):
    """Transposable tile prune on tie-heavy tiles, all-equal tiles (the first
    pattern must win), all-zero tiles and tiles of +0 / -0 only."""
    rows, cols = 64, 96
    a = tie_values(dtype, (rows, cols), 55)
    one = {"f16": 0x3C00, "bf16": 0x3F80, "i8": 1}[dtype]
    neg_zero = {"f16": 0x8000, "bf16": 0x8000, "i8": 0}[dtype]
    a[0:4, 0:4] = one                                   # all-equal magnitudes
    a[4:8, 4:8] = 0                                     # all zero
    a[8:12, 8:12] = neg_zero                            # all -0
    a[12:16, 12:16] = np.where(np.arange(16).reshape(4, 4) % 3 == 0, neg_zero, 0)   # +0 / -0 mix
    a[16:20, 16:20] = one
    a[17, 17] = a[19, 18] = (one | 0x8000) if dtype != "i8" else -1                 # equal magnitudes, signs differ
    ref, keep = oracle.prune_tile(a, dtype)
    first = [[1, 1, 0, 0], [1, 1, 0, 0], [0, 0, 1, 1], [0, 0, 1, 1]]
    for t in range(5):
        assert keep[4 * t:4 * t + 4, 4 * t:4 * t + 4].tolist() == first, t
    plan = plan_for(dtype, rows, 16, cols, 2, 4)
    out = Guarded(a.shape, TRAW[dtype])
    mask = Guarded((plan.mask_bytes // 4,), torch.int32)
    nm.nm_prune(plan, dev(a), out.t, "tile", mask.t)
    sync()
    out.check(); mask.check()
    assert np.array_equal(host(out.t, RAW[dtype]), ref)
    assert np.array_equal(host(mask.t, np.uint32).reshape(rows, -1), oracle.mask_bits(keep))
    cnt = torch.full((1,), 777, dtype=torch.int32, device="cuda")
    nm.nm_prune_check(plan, dev(a), "tile", cnt)
    sync()
    assert int(cnt.item()) == oracle.check_tile(a, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prune_tile_nan_and_inf(dtype):
    """Tiles holding NaN or Inf: a NaN-keeping candidate never wins, and with no
    ordered candidate (a NaN row, column or tile) the first pattern stays."""
    from tests.test_oracle_pins import nan_inf_tiles
    a = nan_inf_tiles(dtype)
    ref, keep = oracle.prune_tile(a, dtype)
    plan = plan_for(dtype, a.shape[0], 16, a.shape[1], 2, 4)
    out = Guarded(a.shape, TRAW[dtype])
    mask = Guarded((plan.mask_bytes // 4,), torch.int32)
    nm.nm_prune(plan, dev(a), out.t, "tile", mask.t)
    sync()
    out.check(); mask.check()
    assert np.array_equal(host(out.t, RAW[dtype]), ref)
    assert np.array_equal(host(mask.t, np.uint32).reshape(a.shape[0], -1), oracle.mask_bits(keep))
    cnt = torch.full((1,), 777, dtype=torch.int32, device="cuda")
    nm.nm_prune_check(plan, out.t, "tile", cnt)
    sync()
    assert int(cnt.item()) == 0


def wide_bf16_tiles(seed):
    """bf16 tiles whose magnitudes span up to the whole exponent range, so that
    fp64 sums of kept magnitudes round: random exponents over all finite values
    (subnormals included), tiles with one huge element that absorbs the rest (every
    candidate keeping it ties after rounding), and tiles whose exponent fields
    span 32 and 33 binades (the edge of the exactly keyed case)."""
    rng = np.random.default_rng(seed)
    rows, cols = 64, 128
    sign = rng.integers(0, 2, (rows, cols)).astype(np.uint16) << 15
    expo = rng.integers(0, 255, (rows, cols)).astype(np.uint16) << 7
    mant = rng.integers(0, 128, (rows, cols)).astype(np.uint16)
    a = sign | expo | mant
    small = (0x3F80 + rng.integers(0, 128, (16, 128))).astype(np.uint16)   # [1, 2)
    a[16:32] = small
    for t in range(32):
        r, c = 16 + 4 * (t % 4), 4 * (t // 4)
        a[r + (t % 3), c + (t % 4)] = 0x7180 + (t % 7)                         # about 2^100
    edge = (0x3F80 + rng.integers(0, 128, (32, 128))).astype(np.uint16)
    a[32:64] = edge
    for t in range(64):
        r, c = 32 + 4 * (t % 8), 4 * (t // 8)
        spread = 32 if t % 2 == 0 else 33
        a[r + (t % 4), c + ((t // 2) % 4)] = (0x3F80 + (spread << 7)) | (t % 128)
    return a


def test_prune_tile_wide_bf16_exponents():
    """Exponent spreads where fp64 sums round: the fixed-order score and its
    first maximum decide, as in the definition."""
    a = wide_bf16_tiles(31)
    ref, keep = oracle.prune_tile(a, "bf16")
    plan = plan_for("bf16", a.shape[0], 16, a.shape[1], 2, 4)
    out = Guarded(a.shape, TRAW["bf16"])
    mask = Guarded((plan.mask_bytes // 4,), torch.int32)
    nm.nm_prune(plan, dev(a), out.t, "tile", mask.t)
    sync()
    out.check(); mask.check()
    assert np.array_equal(host(out.t, RAW["bf16"]), ref)
    assert np.array_equal(host(mask.t, np.uint32).reshape(a.shape[0], -1), oracle.mask_bits(keep))


# ------------------------------------------------------------------ products

def ref_product(dtype, ahat_logical, b_logical, alpha, beta, c):
    if dtype == "i8":
        return oracle.gemm_i64(ahat_logical, b_logical, int(alpha), int(beta), c), None
    A = oracle.decode(ahat_logical, dtype)
    B = oracle.decode(b_logical, dtype)
    C = oracle.decode(c, dtype) if c is not None else None
    D = oracle.gemm_f64(A, B, alpha, beta, C)
    tol = oracle.tolerance(np.abs(A), np.abs(B), alpha, beta, C)
    return D, tol


def assert_close(dtype, got_raw, ref, tol):
    if dtype == "i8":
        assert np.array_equal(got_raw.astype(np.int64), ref), np.argwhere(got_raw.astype(np.int64) != ref)[:5]
        return
    got = oracle.decode(got_raw, dtype)
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), (np.argwhere(bad)[:5], err[bad][:5], tol[bad][:5])


def run_spmm(dtype, N, M, m, n, k, op_b, alpha, beta, seed, op_a="N", tile=None):
    a = rand(dtype, stored(op_a, m, k), seed)
    ahat_stored, _ = oracle.prune_1d(a, dtype, N, M, op_a)
    ahat = ahat_stored if op_a == "N" else np.ascontiguousarray(ahat_stored.T)
    vref, mref = oracle.compress(a, dtype, N, M, op_a)
    b_log = rand(dtype, (k, n), seed + 1)
    b_st = b_log if op_b == "N" else np.ascontiguousarray(b_log.T)
    c = None
    if beta != 0:
        c = (inputs.uniform_int((m, n), seed + 2, -2**20, 2**20, np.int32) if dtype == "i8"
             else rand(dtype, (m, n), seed + 2))
    plan = plan_for(dtype, m, n, k, N, M, op_a=op_a, op_b=op_b, tile=tile)
    odt = torch.int32 if dtype == "i8" else torch.int16
    d = Guarded((m, n), odt)
    nm.nm_spmm(plan, alpha, dev(vref), dev(mref), dev(b_st), beta, dev(c) if c is not None else None, d.t)
    sync()
    d.check()
    ref, tol = ref_product(dtype, ahat, b_log, alpha, beta, c)
    assert_close(dtype, host(d.t, np.int32 if dtype == "i8" else np.uint16), ref, tol)
    return plan


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("op_b", ["N", "T"])
@pytest.mark.parametrize("m,n,k", [(200, 144, 336), (128, 128, 64), (64, 272, 1040), (17, 48, 4), (256, 256, 128), (512, 256, 192),
                                   (256, 512, 640)])
@pytest.mark.parametrize("ab", [(1.0, 0.0), (2.0, -3.0)])
@pytest.mark.parametrize("tile", ["auto", "128", "256"])
def test_spmm_2of4(dtype, op_b, m, n, k, ab, tile):
    alpha, beta = ab
    if dtype != "i8":
        alpha, beta = (0.75, -1.25) if beta != 0 else (1.0, 0.0)
    plan = run_spmm(dtype, 2, 4, m, n, k, op_b, alpha, beta, 1000 + m + n + k, tile=tile)
    assert plan.kernel_name == "spmm_smfmac_2of4"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_spmm_identity_is_bit_exact(dtype):
    """B = I: each output is one exact product, so D equals the pruned A bit for bit;
    with one-hot rows this also pins the instruction's lane and offset mapping."""
    m, k = 96, 192
    a = rand(dtype, (m, k), 3)
    ahat, _ = oracle.prune_1d(a, dtype, 2, 4)
    v, meta = oracle.compress(a, dtype, 2, 4)
    one = np.float16(1).view(np.uint16) if dtype == "f16" else np.uint16(0x3F80)
    eye = np.zeros((k, k), np.uint16)
    np.fill_diagonal(eye, one)
    for op_b in ("N", "T"):
        plan = plan_for(dtype, m, k, k, 2, 4, op_b=op_b)
        d = torch.empty((m, k), dtype=torch.int16, device="cuda")
        nm.nm_spmm(plan, 1.0, dev(v), dev(meta), dev(eye), 0.0, None, d)
        sync()
        got = host(d, np.uint16).copy()
        got[(got & 0x7FFF) == 0] = 0                  # -0 and +0 both mean zero here
        assert np.array_equal(got, ahat)


def test_spmm_kernel_names_the_launched_kernel():
    # the name comes from the same host logic that launches (dry run)
    big = plan_for("f16", 4096, 4096, 1024, 2, 4, op_b="T").spmm_kernel
    # op_b = T with metadata staged four k-steps at a time: layout bits 1 | 4
    assert big.startswith("void nm::gemm_dma_kernel<0, 0, 256, 256,") and big.endswith(", 5>(nm::GemmArgs)"), big
    nn = plan_for("bf16", 1024, 4096, 4096, 2, 4, op_b="N").spmm_kernel
    assert nn.startswith("void nm::gemm_dma_kernel<1, 0, 128, 128,") and nn.endswith(", 2, 2, 4>(nm::GemmArgs)"), nn
    nn8 = plan_for("i8", 1024, 4096, 4096, 2, 4, op_b="N").spmm_kernel   # int8: eight waves, one tile per CU
    assert nn8.startswith("void nm::gemm_dma_kernel<2, 0, 128, 128,") and nn8.endswith(", 2, 4, 0>(nm::GemmArgs)"), nn8
    nt = plan_for("bf16", 1024, 4096, 4096, 2, 4, op_b="T").spmm_kernel
    # four waves, op_b = T, batched metadata: layout bits 1 | 4
    assert nt.startswith("void nm::gemm_dma_kernel<1, 0, 128, 128,") and nt.endswith(", 2, 2, 5>(nm::GemmArgs)"), nt
    i8 = plan_for("i8", 1024, 4096, 4096, 2, 4, op_b="T").spmm_kernel
    assert i8.startswith("void nm::gemm_dma_kernel<2, 0, 128, 128,") and i8.endswith(", 2, 2, 1>(nm::GemmArgs)"), i8
    ragged = plan_for("f16", 200, 144, 336, 2, 4).spmm_kernel
    assert ragged.startswith("void nm::gemm_kernel<0, 0,"), ragged
    assert "skinny2_kernel" in plan_for("f16", 100, 8, 1088, 2, 4).spmm_kernel
    assert "gemm_kernel<0, 2," in plan_for("f16", 150, 80, 544, 4, 32).spmm_kernel


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("N,M", [(1, 4), (3, 4), (2, 8), (5, 16), (2, 32), (4, 32), (8, 32), (16, 32)])
@pytest.mark.parametrize("op_b", ["N", "T"])
def test_spmm_gather(dtype, N, M, op_b):
    alpha, beta = (1.0, 1.0) if dtype == "i8" else (0.5, 0.25)
    plan = run_spmm(dtype, N, M, 150, 80, 544, op_b, alpha, beta, 2000 + N * M)
    assert plan.kernel_name == "spmm_gather_mfma"


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("N,M", [(2, 4), (4, 32), (8, 32), (3, 8)])
@pytest.mark.parametrize("n", [1, 3, 8, 16])
@pytest.mark.parametrize("op_b", ["N", "T"])
def test_spmm_skinny(dtype, N, M, n, op_b):
    alpha, beta = (1.0, 0.0) if n != 3 else ((1.0, -2.0) if dtype == "i8" else (1.5, 0.5))
    plan = run_spmm(dtype, N, M, 100, n, 1088, op_b, alpha, beta, 3000 + n)
    assert plan.kernel_name == "spmm_skinny"


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("N,M,n,k", [(2, 4, 1, 1088), (4, 32, 2, 1088), (2, 4, 4, 1088), (4, 32, 8, 4160)])
def test_spmm_skinny_tall(dtype, N, M, n, k):
    """At least 16384 rows: each wave takes several rows (16-bit types); 16400 rows
    leave a ragged last block and k = 4160 with n = 8 spans two staged chunks."""
    alpha, beta = (1.0, 1.0) if dtype == "i8" else (0.5, -0.25)
    plan = run_spmm(dtype, N, M, 16400, n, k, "N" if n != 2 else "T", alpha, beta, 5000 + n)
    assert plan.kernel_name == "spmm_skinny"
    rw = 4 if n <= 2 else 2                                 # rows per wave for N <= 4 kept values per group
    assert plan.spmm_kernel.endswith(", false, %d, %d>(nm::GemmArgs, int)" % (rw, N)), plan.spmm_kernel


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("N,M,m", [(2, 4, 200), (4, 32, 4200), (0, 0, 300)])
def test_skinny_double_buffered(dtype, N, M, m):
    """16-byte B records (n = 8 for 16-bit types, 16 for int8) with k past one
    LDS chunk: the next chunk is staged while the current one is read; k = 12352
    leaves a 64-wide last chunk, 4200 rows give blocks a second row group.
    N = 0 runs the dense comparator on the same path."""
    n, k = (16 if dtype == "i8" else 8), 12352
    if N:
        plan = run_spmm(dtype, N, M, m, n, k, "N", 1.0, 0.0, 6000 + m)
        assert plan.kernel_name == "spmm_skinny"
        return
    a = rand(dtype, (m, k), 61)
    b = rand(dtype, (k, n), 62)
    plan = plan_for(dtype, m, n, k, 2, 4)
    odt = torch.int32 if dtype == "i8" else torch.int16
    d = Guarded((m, n), odt)
    nm.nm_dense_gemm(plan, 1.0, dev(a), dev(b), 0.0, None, d.t)
    sync()
    d.check()
    ref, tol = ref_product(dtype, a, b, 1.0, 0.0, None)
    assert_close(dtype, host(d.t, np.int32 if dtype == "i8" else np.uint16), ref, tol)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("n,k", [(1, 4160), (8, 1040)])
def test_dense_skinny_tall(dtype, n, k):
    m = 16400
    a = rand(dtype, (m, k), 51)
    b = rand(dtype, (k, n), 52)
    plan = plan_for(dtype, m, n, k, 2, 4)
    odt = torch.int32 if dtype == "i8" else torch.int16
    d = Guarded((m, n), odt)
    nm.nm_dense_gemm(plan, 1.0, dev(a), dev(b), 0.0, None, d.t)
    sync()
    d.check()
    ref, tol = ref_product(dtype, a, b, 1.0, 0.0, None)
    assert_close(dtype, host(d.t, np.int32 if dtype == "i8" else np.uint16), ref, tol)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("op_a", ["N", "T"])
@pytest.mark.parametrize("op_b", ["N", "T"])
@pytest.mark.parametrize("m,n,k", [(272, 8, 208), (272, 144, 208), (272, 304, 208), (256, 256, 320), (512, 384, 192),
                                   (256, 512, 640)])
@pytest.mark.parametrize("tile", ["auto", "128", "256"])
def test_dense_gemm(dtype, op_a, op_b, m, n, k, tile):
    a_log = rand(dtype, (m, k), 41)
    a_st = a_log if op_a == "N" else np.ascontiguousarray(a_log.T)
    b_log = rand(dtype, (k, n), 42)
    b_st = b_log if op_b == "N" else np.ascontiguousarray(b_log.T)
    plan = plan_for(dtype, m, n, k, 2, 4, op_a=op_a, op_b=op_b, tile=tile)
    odt = torch.int32 if dtype == "i8" else torch.int16
    d = Guarded((m, n), odt)
    nm.nm_dense_gemm(plan, 1.0, dev(a_st), dev(b_st), 0.0, None, d.t)
    sync()
    d.check()
    ref, tol = ref_product(dtype, a_log, b_log, 1.0, 0.0, None)
    assert_close(dtype, host(d.t, np.int32 if dtype == "i8" else np.uint16), ref, tol)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("op_b", ["N", "T"])
@pytest.mark.parametrize("m,n,k,pad,tile", [(256, 256, 256, 64, "256"), (384, 256, 512, 32, "128"),
                                            (2304, 2048, 256, 0, "128"), (2304, 256, 256, 16, "256")])
def test_dense_op_a_t_full_tiles(dtype, op_b, m, n, k, pad, tile):
    """A stored k x m (op_a = T) with a padded leading dimension and beta != 0 on
    whole tiles: the copy-ring kernel's transposed-A staging, on both tile shapes
    and both ring depths (more 128 x 128 tiles than compute units takes the
    shallow ring)."""
    a_log = rand(dtype, (m, k), 51)
    lda = m + pad
    a_st = np.zeros((k, lda), dtype=a_log.dtype)
    a_st[:, :m] = a_log.T
    b_log = rand(dtype, (k, n), 52)
    b_st = b_log if op_b == "N" else np.ascontiguousarray(b_log.T)
    c = (inputs.uniform_int((m, n), 53, -2**20, 2**20, np.int32) if dtype == "i8" else rand(dtype, (m, n), 53))
    alpha, beta = (2.0, -1.0) if dtype == "i8" else (0.75, 0.5)
    plan = plan_for(dtype, m, n, k, 2, 4, op_a="T", op_b=op_b, lda=lda, tile=tile)
    odt = torch.int32 if dtype == "i8" else torch.int16
    d = Guarded((m, n), odt)
    nm.nm_dense_gemm(plan, alpha, dev(a_st), dev(b_st), beta, dev(c), d.t)
    sync()
    d.check()
    ref, tol = ref_product(dtype, a_log, b_log, alpha, beta, c)
    assert_close(dtype, host(d.t, np.int32 if dtype == "i8" else np.uint16), ref, tol)


@pytest.mark.parametrize("dtype", ["f16", "i8"])
@pytest.mark.parametrize("n", [4, 48])
def test_k_zero_gives_beta_c(dtype, n):
    m = 24
    c = inputs.uniform_int((m, n), 1, -100, 100, np.int32) if dtype == "i8" else rand(dtype, (m, n), 1)
    plan = plan_for(dtype, m, n, 0, 2, 4)
    odt = torch.int32 if dtype == "i8" else torch.int16
    d = torch.empty((m, n), dtype=odt, device="cuda")
    nm.nm_spmm(plan, 1.0, None, None, None, 2.0 if dtype == "i8" else 0.5, dev(c), d)
    sync()
    got = host(d, np.int32 if dtype == "i8" else np.uint16)
    if dtype == "i8":
        assert np.array_equal(got, 2 * c)
    else:
        assert np.array_equal(oracle.decode(got, dtype), 0.5 * oracle.decode(c, dtype))


COL_CASES = [
    # (label, N, M, m, n, k, op_b, force_tile): sparse 2:4 full tiles (copy-ring kernel, both B layouts,
    # 128 and 256 tiles), ragged 2:4, general N:M gather, small n, and N = 0 for the dense comparator
    ("24-ring-NT", 2, 4, 256, 256, 256, "T", None),
    ("24-ring-NN", 2, 4, 256, 384, 192, "N", None),
    ("24-ring-256", 2, 4, 512, 512, 128, "T", "256"),
    ("24-ragged", 2, 4, 200, 144, 336, "N", None),
    ("gather-4of32", 4, 32, 150, 80, 544, "T", None),
    ("skinny-24", 2, 4, 100, 8, 1088, "N", None),
    ("skinny-4of32", 4, 32, 100, 3, 1088, "T", None),
    ("dense-ring", 0, 0, 256, 256, 320, "T", None),
    ("dense-ragged", 0, 0, 272, 144, 208, "N", None),
    ("dense-skinny", 0, 0, 200, 8, 1040, "N", None),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("case", COL_CASES, ids=[c[0] for c in COL_CASES])
@pytest.mark.parametrize("beta", [0.0, 1.0])
def test_col_major_cd(dtype, case, beta):
    """Column-major C and D (the blog's column-major output): D element (i, j) at
    j * ldd + i, with ldd > m so that the rows past m of every column (the caller's
    bytes) must stay untouched; C read column-major the same way."""
    label, N, M, m, n, k, op_b, tile = case
    es_cd = 4 if dtype == "i8" else 2
    ld = -(-m // (16 // es_cd)) * (16 // es_cd) + 16 // es_cd      # 16-byte columns, padded past m
    seed = 7000 + m + n + k
    alpha = 1.0 if dtype == "i8" else 0.75
    a = rand(dtype, (m, k), seed)
    b_log = rand(dtype, (k, n), seed + 1)
    b_st = b_log if op_b == "N" else np.ascontiguousarray(b_log.T)
    c = None
    if beta != 0:
        c = (inputs.uniform_int((m, n), seed + 2, -2**20, 2**20, np.int32) if dtype == "i8"
             else rand(dtype, (m, n), seed + 2))
    plan = plan_for(dtype, m, n, k, N or 2, M or 4, op_b=op_b, ldc=ld, ldd=ld, order_cd="col", tile=tile)
    raw = np.int32 if dtype == "i8" else np.uint16
    sentinel = np.full((n, ld), 0x3C3C if es_cd == 2 else 0x3C3C3C3C, dtype=raw)
    d = Guarded((n, ld), torch.int32 if dtype == "i8" else torch.int16, fill=dev(sentinel))
    dc = None
    if c is not None:
        c_col = np.zeros((n, ld), dtype=raw)
        c_col[:, :m] = c.T
        dc = dev(c_col)
    if N:
        ahat, _ = oracle.prune_1d(a, dtype, N, M)
        vref, mref = oracle.compress(a, dtype, N, M)
        nm.nm_spmm(plan, alpha, dev(vref), dev(mref), dev(b_st), beta, dc, d.t)
    else:
        ahat = a
        nm.nm_dense_gemm(plan, alpha, dev(a), dev(b_st), beta, dc, d.t)
    sync()
    d.check()
    got = host(d.t, raw)
    assert np.array_equal(got[:, m:], sentinel[:, m:]), label
    ref, tol = ref_product(dtype, ahat, b_log, alpha, beta, c)
    assert_close(dtype, np.ascontiguousarray(got[:, :m].T), ref, tol)


I8OUT_CASES = [
    # (label, N, M, m, n, k, op_b, order_cd): copy-ring kernel (both B layouts, both C/D orders),
    # ragged, general N:M gather, small n, and N = 0 for the dense comparator
    ("24-ring-NT", 2, 4, 256, 256, 256, "T", "row"),
    ("24-ring-NN-col", 2, 4, 256, 256, 256, "N", "col"),
    ("24-ragged", 2, 4, 200, 144, 336, "N", "row"),
    ("24-ragged-col", 2, 4, 200, 144, 336, "T", "col"),
    ("gather-4of32", 4, 32, 150, 80, 544, "T", "row"),
    ("skinny-24", 2, 4, 100, 8, 1088, "N", "row"),
    ("skinny-8of32-col", 8, 32, 100, 3, 1088, "N", "col"),
    ("dense-ring", 0, 0, 256, 256, 320, "T", "row"),
    ("dense-ragged-col", 0, 0, 272, 144, 208, "N", "col"),
]


@pytest.mark.parametrize("case", I8OUT_CASES, ids=[c[0] for c in I8OUT_CASES])
@pytest.mark.parametrize("ab", [(1.0, 0.0), (2.0, -1.0)])
def test_int8_output(case, ab):
    """int8 C and D: the exact integer alpha acc + beta C saturated to int8, bit
    for bit. Inputs in [-3, 3] put outputs both inside and beyond the int8 range."""
    label, N, M, m, n, k, op_b, order = case
    alpha, beta = ab
    seed = 8100 + m + n + k
    a = inputs.uniform_int((m, k), seed, -3, 3)
    b_log = inputs.uniform_int((k, n), seed + 1, -3, 3)
    b_st = b_log if op_b == "N" else np.ascontiguousarray(b_log.T)
    c = inputs.uniform_int((m, n), seed + 2, -128, 127) if beta != 0 else None
    lines, length = (n, m) if order == "col" else (m, n)
    ld = -(-length // 16) * 16                                  # 16-byte rows (columns) of int8
    plan = plan_for("i8", m, n, k, N or 2, M or 4, op_b=op_b, order_cd=order, out_dtype="i8", ldc=ld, ldd=ld)
    d = Guarded((lines, ld), torch.int8)
    dc = None
    if c is not None:
        c_st = np.zeros((lines, ld), np.int8)
        c_st[:, :length] = c.T if order == "col" else c
        dc = dev(c_st)
    if N:
        ahat, _ = oracle.prune_1d(a, "i8", N, M)
        vref, mref = oracle.compress(a, "i8", N, M)
        nm.nm_spmm(plan, alpha, dev(vref), dev(mref), dev(b_st), beta, dc, d.t)
    else:
        ahat = a
        nm.nm_dense_gemm(plan, alpha, dev(a), dev(b_st), beta, dc, d.t)
    sync()
    d.check()
    got = host(d.t, np.int8)[:, :length]
    if order == "col":
        got = got.T
    ref = oracle.gemm_i8_saturated(ahat, b_log, int(alpha), int(beta), c)
    assert np.array_equal(got, ref), (label, np.argwhere(got != ref)[:5])
    exact = oracle.gemm_i64(ahat, b_log, int(alpha), int(beta), c.astype(np.int32) if c is not None else None)
    assert (np.abs(exact) > 127).any() and (np.abs(exact) <= 127).any()   # both regimes are exercised


@pytest.mark.parametrize("dtype", ["f16", "i8"])
def test_algorithm_ids_pin_the_tile_and_autotune(dtype):
    """Each algorithm id launches its tile's kernel and gives the oracle's result;
    autotuning times them all and leaves the fastest pinned on the plan."""
    from structured_sparse_gemm_nm_amd.tuning import autotune_spmm
    m, n, k = 512, 512, 256
    a = rand(dtype, (m, k), 31)
    b = rand(dtype, (n, k), 32)
    ahat, _ = oracle.prune_1d(a, dtype, 2, 4)
    v, meta = oracle.compress(a, dtype, 2, 4)
    plan = plan_for(dtype, m, n, k, 2, 4, op_b="T")
    odt, raw = (torch.int32, np.int32) if dtype == "i8" else (torch.int16, np.uint16)
    dv, dm, db = dev(v), dev(meta), dev(b)
    ref, tol = ref_product(dtype, ahat, np.ascontiguousarray(b.T), 1.0, 0.0, None)
    tiles = {nm.NM_ALG_TILE128: "128, 128,", nm.NM_ALG_TILE256X128: "256, 128,", nm.NM_ALG_TILE256: "256, 256,"}
    for alg in range(nm.NM_ALG_COUNT):
        nm.nm_plan_set_algorithm(plan, alg)
        kern = plan.spmm_kernel
        if alg in tiles:
            assert tiles[alg] in kern, (alg, kern)
        d = Guarded((m, n), odt)
        nm.nm_spmm(plan, 1.0, dv, dm, db, 0.0, None, d.t)
        sync()
        d.check()
        assert_close(dtype, host(d.t, raw), ref, tol)
    d = Guarded((m, n), odt)
    times = autotune_spmm(plan, 1.0, dv, dm, db, 0.0, None, d.t, reps=3, split_ks=(1, 2))
    best = (nm.nm_plan_get_algorithm(plan), nm.nm_plan_get_split_k(plan)[0])
    assert set(times) == {(a, s) for a in range(nm.NM_ALG_COUNT) for s in (1, 2)}
    assert times[best][0] == min(t for t, _ in times.values())
    sync()
    assert_close(dtype, host(d.t, raw), ref, tol)
    # the pinned setting runs with the workspace it asks for
    d2 = Guarded((m, n), odt)
    nm.nm_spmm(plan, 1.0, dv, dm, db, 0.0, None, d2.t, workspace=plan.empty_workspace())
    sync()
    assert_close(dtype, host(d2.t, raw), ref, tol)


@pytest.mark.parametrize("dtype", ["f16", "i8"])
def test_c_may_alias_d_full_tiles(dtype):
    """C == D on the copy-ring kernel with beta != 0 (the staged epilogue reads
    each C quad and writes the same D quad from one thread)."""
    m, n, k = 256, 256, 128
    a = rand(dtype, (m, k), 81)
    v, meta = oracle.compress(a, dtype, 2, 4)
    ahat, _ = oracle.prune_1d(a, dtype, 2, 4)
    b = rand(dtype, (n, k), 82)
    if dtype == "i8":
        c = inputs.uniform_int((m, n), 83, -2**20, 2**20, np.int32)
        alpha, beta, raw = 2.0, -1.0, np.int32
    else:
        c = rand(dtype, (m, n), 83)
        alpha, beta, raw = 0.5, 1.5, np.uint16
    plan = plan_for(dtype, m, n, k, 2, 4, op_b="T")
    dc = dev(c)
    nm.nm_spmm(plan, alpha, dev(v), dev(meta), dev(b), beta, dc, dc)
    sync()
    ref, tol = ref_product(dtype, ahat, np.ascontiguousarray(b.T), alpha, beta, c)
    assert_close(dtype, host(dc, raw), ref, tol)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("op_b", ["N", "T"])
@pytest.mark.parametrize("order", ["row", "col"])
def test_beta_epilogue_on_256_tiles(dtype, op_b, order):
    """beta != 0 on 256 x 256 tiles, whose raw 4-byte tile does not fit LDS at
    once: row-major D drains in rounds of one fragment column of every wave
    (C loads issued several thread steps ahead), column-major D in rounds of
    one wave column group; then again with C aliasing D."""
    m, n, k = 512, 768, 384
    a = rand(dtype, (m, k), 91)
    v, meta = oracle.compress(a, dtype, 2, 4)
    ahat, _ = oracle.prune_1d(a, dtype, 2, 4)
    b_log = rand(dtype, (k, n), 92)
    b_st = b_log if op_b == "N" else np.ascontiguousarray(b_log.T)
    if dtype == "i8":
        c = inputs.uniform_int((m, n), 93, -2**20, 2**20, np.int32)
        alpha, beta, raw, odt = 3.0, 2.0, np.int32, torch.int32
    else:
        c = rand(dtype, (m, n), 93)
        alpha, beta, raw, odt = 0.75, -1.25, np.uint16, torch.int16
    plan = plan_for(dtype, m, n, k, 2, 4, op_b=op_b, tile="256", order_cd=order)
    assert "256, 256," in plan.spmm_kernel, plan.spmm_kernel
    c_st = c if order == "row" else np.ascontiguousarray(c.T)
    ref, tol = ref_product(dtype, ahat, b_log, alpha, beta, c)
    logical = (lambda x: x) if order == "row" else (lambda x: np.ascontiguousarray(x.T))
    d = Guarded(c_st.shape, odt)
    nm.nm_spmm(plan, alpha, dev(v), dev(meta), dev(b_st), beta, dev(c_st), d.t)
    sync()
    d.check()
    assert_close(dtype, logical(host(d.t, raw)), ref, tol)
    dc = dev(c_st)
    nm.nm_spmm(plan, alpha, dev(v), dev(meta), dev(b_st), beta, dc, dc)
    sync()
    assert_close(dtype, logical(host(dc, raw)), ref, tol)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("tile", ["128", "256"])
@pytest.mark.parametrize("op_b", ["N", "T"])
def test_batched_metadata_step_counts(dtype, tile, op_b):
    """16-bit 2:4 kernels with the metadata staged four k-steps at a time, on
    k-step counts that exercise the first step, the steady steps four at a
    time, the remaining refill steps and the last steps (1, 2, 5, 6, 9 and 14
    steps of 64), with beta != 0 and column-major D on some of them."""
    m, n = (256, 384) if tile == "128" else (512, 512)
    for i, steps in enumerate([1, 2, 5, 6, 9, 14]):
        k = 64 * steps
        a = rand(dtype, (m, k), 300 + steps)
        v, meta = oracle.compress(a, dtype, 2, 4)
        ahat, _ = oracle.prune_1d(a, dtype, 2, 4)
        b_log = rand(dtype, (k, n), 400 + steps)
        b_st = b_log if op_b == "N" else np.ascontiguousarray(b_log.T)
        order = "col" if i % 2 else "row"
        beta = -0.5 if i % 3 == 1 else 0.0
        c = rand(dtype, (m, n), 500 + steps)
        plan = plan_for(dtype, m, n, k, 2, 4, op_b=op_b, tile=tile, order_cd=order)
        assert "%s, %s," % (tile, tile) in plan.spmm_kernel and plan.spmm_kernel.endswith(
            ", %d>(nm::GemmArgs)" % (5 if op_b == "T" else 4)), plan.spmm_kernel
        c_st = c if order == "row" else np.ascontiguousarray(c.T)
        ref, tol = ref_product(dtype, ahat, b_log, 1.25, beta, c if beta else None)
        d = Guarded(c_st.shape, torch.int16)
        nm.nm_spmm(plan, 1.25, dev(v), dev(meta), dev(b_st), beta, dev(c_st) if beta else None, d.t)
        sync()
        d.check()
        got = host(d.t, np.uint16)
        assert_close(dtype, got if order == "row" else np.ascontiguousarray(got.T), ref, tol)


def test_col_major_k_zero_and_alias():
    m, n = 40, 24
    c = rand("f16", (m, n), 11)
    plan = plan_for("f16", m, n, 0, 2, 4, order_cd="col")
    d = torch.empty((n, m), dtype=torch.int16, device="cuda")
    nm.nm_spmm(plan, 1.0, None, None, None, 0.5, dev(np.ascontiguousarray(c.T)), d)
    sync()
    assert np.array_equal(oracle.decode(host(d, np.uint16).T, "f16"), 0.5 * oracle.decode(c, "f16"))
    # C == D, column-major, on the copy-ring kernel
    m, n, k = 256, 256, 128
    a = rand("f16", (m, k), 12)
    v, meta = oracle.compress(a, "f16", 2, 4)
    ahat, _ = oracle.prune_1d(a, "f16", 2, 4)
    b = rand("f16", (n, k), 13)
    c = rand("f16", (m, n), 14)
    plan = plan_for("f16", m, n, k, 2, 4, op_b="T", order_cd="col")
    dc = dev(np.ascontiguousarray(c.T))
    nm.nm_spmm(plan, 1.0, dev(v), dev(meta), dev(b), -1.0, dc, dc)
    sync()
    ref, tol = ref_product("f16", ahat, np.ascontiguousarray(b.T), 1.0, -1.0, c)
    assert_close("f16", np.ascontiguousarray(host(dc, np.uint16).T), ref, tol)


def test_c_may_alias_d():
    m, n, k = 64, 64, 128
    a = rand("f16", (m, k), 8)
    v, meta = oracle.compress(a, "f16", 2, 4)
    ahat, _ = oracle.prune_1d(a, "f16", 2, 4)
    b = rand("f16", (k, n), 9)
    c = rand("f16", (m, n), 10)
    plan = plan_for("f16", m, n, k, 2, 4)
    dc = dev(c)
    nm.nm_spmm(plan, 1.0, dev(v), dev(meta), dev(b), 1.0, dc, dc)
    sync()
    ref, tol = ref_product("f16", ahat, b, 1.0, 1.0, c)
    assert_close("f16", host(dc, np.uint16), ref, tol)


# ------------------------------------------------------------------ split-k with a workspace

SPLIT_CASES = [
    # (label, m, n, k, op_b, tile, splits, beta, order_cd): even and uneven k ranges, the
    # clamp to the number of k-steps, both B layouts, all three block tiles, beta and
    # column-major C/D, and the eight-wave 128 x 128 kernel (B stored k x n, few tiles)
    ("128-NT-2", 256, 256, 1024, "T", "128", 2, 0.0, "row"),
    ("128-NN-4-beta", 256, 256, 1024, "N", "128", 4, 1.0, "row"),
    ("256-NT-3-col", 512, 512, 640, "T", "256", 3, 1.0, "col"),
    ("128-NN-clamped-col", 256, 384, 384, "N", "128", 16, 0.0, "col"),
    ("256x128-NT-5", 1024, 256, 2048, "T", "256x128", 5, -0.5, "row"),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_split_k(dtype, case):
    """Split-k on the whole-tile 2:4 kernel: each k range writes its partial sums
    to its own workspace plane and the reduction adds them in order. int8 is
    bit-exact (and equal to the unsplit product); fp16/bf16 within tolerance.
    The workspace is guarded on both sides and its size is the documented one."""
    label, m, n, k, op_b, tile, splits, beta, order = case
    seed = 9100 + m + n + k
    a = rand(dtype, (m, k), seed)
    ahat, _ = oracle.prune_1d(a, dtype, 2, 4)
    vref, mref = oracle.compress(a, dtype, 2, 4)
    b_log = rand(dtype, (k, n), seed + 1)
    b_st = b_log if op_b == "N" else np.ascontiguousarray(b_log.T)
    c = None
    if beta != 0:
        c = (inputs.uniform_int((m, n), seed + 2, -2**20, 2**20, np.int32) if dtype == "i8"
             else rand(dtype, (m, n), seed + 2))
    alpha = 1.0 if dtype == "i8" else 0.75
    if dtype == "i8" and beta != 0:
        beta = 1.0
    plan = plan_for(dtype, m, n, k, 2, 4, op_b=op_b, tile=tile, order_cd=order)
    nm.nm_plan_set_split_k(plan, splits)
    kl = 128 if dtype == "i8" else 64
    eff = min(splits, k // kl)
    assert nm.nm_plan_get_split_k(plan) == (splits, eff)
    assert nm.nm_spmm_workspace_size(plan) == (eff * m * n * 4 if eff > 1 else 0)
    raw = np.int32 if dtype == "i8" else np.uint16
    odt = torch.int32 if dtype == "i8" else torch.int16
    dshape = (n, m) if order == "col" else (m, n)
    dc = None
    if c is not None:
        dc = dev(np.ascontiguousarray(c.T) if order == "col" else c)
    ws = Guarded((max(1, nm.nm_spmm_workspace_size(plan)),), torch.uint8)
    d = Guarded(dshape, odt)
    nm.nm_spmm(plan, alpha, dev(vref), dev(mref), dev(b_st), beta, dc, d.t, workspace=ws.t)
    sync()
    d.check(); ws.check()
    got = host(d.t, raw)
    got = np.ascontiguousarray(got.T) if order == "col" else got
    ref, tol = ref_product(dtype, ahat, b_log, alpha, beta, c)
    assert_close(dtype, got, ref, tol)
    # a second call on the same workspace (its old contents must not leak in)
    d2 = Guarded(dshape, odt)
    nm.nm_spmm(plan, alpha, dev(vref), dev(mref), dev(b_st), beta, dc, d2.t, workspace=ws.t)
    sync()
    assert np.array_equal(host(d2.t, raw), host(d.t, raw))
    if dtype == "i8":
        unsplit = plan_for(dtype, m, n, k, 2, 4, op_b=op_b, tile=tile, order_cd=order)
        d3 = Guarded(dshape, odt)
        nm.nm_spmm(unsplit, alpha, dev(vref), dev(mref), dev(b_st), beta, dc, d3.t)
        sync()
        assert np.array_equal(host(d3.t, raw), host(d.t, raw))


@pytest.mark.parametrize("dtype", ["f16", "i8"])
def test_split_k_c_aliases_d_and_kernel_name(dtype):
    """C == D through the reduction (each quad is read and written by one thread),
    and the plan still names the product kernel, not the reduction."""
    m, n, k = 256, 256, 512
    a = rand(dtype, (m, k), 71)
    ahat, _ = oracle.prune_1d(a, dtype, 2, 4)
    v, meta = oracle.compress(a, dtype, 2, 4)
    b = rand(dtype, (n, k), 72)
    if dtype == "i8":
        c = inputs.uniform_int((m, n), 73, -2**20, 2**20, np.int32)
        alpha, beta, raw = 2.0, -1.0, np.int32
    else:
        c = rand(dtype, (m, n), 73)
        alpha, beta, raw = 0.5, 1.5, np.uint16
    plan = plan_for(dtype, m, n, k, 2, 4, op_b="T", tile="128")
    nm.nm_plan_set_split_k(plan, 3)
    assert "gemm_dma_kernel" in plan.spmm_kernel
    ws = plan.empty_workspace()
    dc = dev(c)
    nm.nm_spmm(plan, alpha, dev(v), dev(meta), dev(b), beta, dc, dc, workspace=ws)
    sync()
    ref, tol = ref_product(dtype, ahat, np.ascontiguousarray(b.T), alpha, beta, c)
    assert_close(dtype, host(dc, raw), ref, tol)


def test_split_k_not_applicable_runs_unsplit():
    """Ragged shapes, general N:M and small n ignore the split and need no workspace."""
    for (N, M, m, n, k) in [(2, 4, 200, 144, 336), (4, 32, 150, 80, 544), (2, 4, 100, 8, 1088)]:
        a = rand("f16", (m, k), 5 + m)
        ahat, _ = oracle.prune_1d(a, "f16", N, M)
        v, meta = oracle.compress(a, "f16", N, M)
        b = rand("f16", (k, n), 6 + m)
        plan = plan_for("f16", m, n, k, N, M)
        nm.nm_plan_set_split_k(plan, 4)
        assert nm.nm_spmm_workspace_size(plan) == 0
        d = Guarded((m, n), torch.int16)
        nm.nm_spmm(plan, 1.0, dev(v), dev(meta), dev(b), 0.0, None, d.t)
        sync()
        d.check()
        ref, tol = ref_product("f16", ahat, b, 1.0, 0.0, None)
        assert_close("f16", host(d.t, np.uint16), ref, tol)


# ------------------------------------------------------------------ several streams

STREAM_CASES = [
    # (label, N, M, V, m, n, k, op_b, splits, order): whole tiles on both B layouts, a ragged last
    # row block, vector-wise rows, a split-k plan sharing its workspace, column-major D
    ("24-NT", 2, 4, 0, 1024, 256, 512, "T", 1, "row"),
    ("24-NN-ragged", 2, 4, 0, 600, 144, 336, "N", 1, "row"),
    ("vw16-4of32", 4, 32, 16, 768, 256, 512, "N", 1, "row"),
    ("24-split", 2, 4, 0, 768, 256, 1024, "T", 2, "col"),
]


@pytest.mark.parametrize("dtype", ["f16", "i8"])
@pytest.mark.parametrize("case", STREAM_CASES, ids=[c[0] for c in STREAM_CASES])
def test_spmm_streams(dtype, case):
    """nm_spmm_streams splits D's rows over three streams; the result matches the
    oracle (int8 bit-exact) and, for int8, nm_spmm's single-stream result."""
    label, N, M, V, m, n, k, op_b, splits, order = case
    seed = 9900 + m + n
    a = rand(dtype, (m, k), seed)
    if V:
        ahat, _ = oracle.prune_vw(a, dtype, V, N, M)
        v, meta = oracle.compress_vw(a, dtype, V, N, M)
    else:
        ahat, _ = oracle.prune_1d(a, dtype, N, M)
        v, meta = oracle.compress(a, dtype, N, M)
    b_log = rand(dtype, (k, n), seed + 1)
    b_st = b_log if op_b == "N" else np.ascontiguousarray(b_log.T)
    plan = plan_for(dtype, m, n, k, N, M, op_b=op_b, order_cd=order, vector_rows=V)
    nm.nm_plan_set_split_k(plan, splits)
    ws = plan.empty_workspace()
    raw, odt = (np.int32, torch.int32) if dtype == "i8" else (np.uint16, torch.int16)
    dshape = (n, m) if order == "col" else (m, n)
    streams = [torch.cuda.Stream() for _ in range(3)]
    dv, dm, db = dev(v), dev(meta), dev(b_st)
    sync()
    d = Guarded(dshape, odt)
    nm.nm_spmm_streams(plan, 1.0, dv, dm, db, 0.0, None, d.t, streams, workspace=ws)
    for s_ in streams:
        s_.synchronize()
    d.check()
    got = host(d.t, raw)
    got = np.ascontiguousarray(got.T) if order == "col" else got
    ref, tol = ref_product(dtype, ahat, b_log, 1.0, 0.0, None)
    assert_close(dtype, got, ref, tol)
    if dtype == "i8":
        d1 = Guarded(dshape, odt)
        nm.nm_spmm(plan, 1.0, dv, dm, db, 0.0, None, d1.t, workspace=ws)
        sync()
        assert np.array_equal(host(d1.t, raw), host(d.t, raw))
