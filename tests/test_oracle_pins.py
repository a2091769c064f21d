"""Pins for the CPU oracle: checks against facts that do not come from the oracle.

Each test fixes the oracle to something else the pages or the mathematics
determine: IEEE decoding of every bit pattern, brute force over all C(M, N)
subsets, the closed-form count of 4x4 0/1 matrices with all line sums 2, an
independent dynamic programme for the tile optimum, round trips, the sparse
loop against the dense loop, and library/closed-form special cases of the
product. The pages print no worked numeric example, so none is stored here.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
from structured_sparse_gemm_nm_amd import inputs


# ------------------------------------------------------------------ decoding

def test_f16_decode_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)          # library routine
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)   # bf16 = top half of binary32
    got = oracle.decode(bits.astype(np.uint16), "bf16")
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ------------------------------------------------------------------ 1-D N:M prune

def _exact_abs(raw, dtype):
    vals = oracle.decode(raw, dtype)
    return [Fraction(abs(float(v))) for v in vals]


def _brute_force_keep(raw_group, dtype, N):
    """argmax over all N-subsets of the exact kept sum of |w|; among equal sums the
    lexicographically smallest sorted index tuple (this equals 'ties to the lower index')."""
    mags = _exact_abs(raw_group, dtype)
    best, best_set = None, None
    for sub in itertools.combinations(range(len(mags)), N):   # lexicographic order
        s = sum((mags[i] for i in sub), Fraction(0))
        if best is None or s > best:
            best, best_set = s, sub
    keep = np.zeros(len(mags), np.uint8)
    keep[list(best_set)] = 1
    return keep


def _groups(dtype, M, count, seed, ties=False):
    rng = np.random.default_rng(seed)
    if dtype == "i8":
        return rng.integers(-127 if not ties else -3, (127 if not ties else 3) + 1, size=(count, M)).astype(np.int8)
    if ties:
        x = rng.choice(np.array([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -0.0]), size=(count, M)).astype(np.float32)
    else:
        x = rng.standard_normal((count, M)).astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    return inputs._fp32_to_bf16_bits(x).reshape(count, M)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("M,Ns,count", [(4, (1, 2, 3), 300), (8, (1, 2, 3, 4, 5, 6, 7), 80),
                                        (16, (1, 2, 3), 20), (32, (1, 2, 4), 3)])
@pytest.mark.parametrize("ties", [False, True])
def test_prune_1d_equals_brute_force(dtype, M, Ns, count, ties):
    g = _groups(dtype, M, count, seed=M * 7 + (1 if ties else 0), ties=ties)
    for N in Ns:
        _, keep = oracle.prune_1d(g, dtype, N, M)
        for r in range(count):
            assert np.array_equal(keep[r], _brute_force_keep(g[r], dtype, N)), (dtype, M, N, r, g[r])


@pytest.mark.parametrize("N", [1, 2, 3])
def test_prune_1d_exhaustive_int8_small_values(N):
    """Every group over {-2..2}^4: heavy ties, including all-equal magnitudes."""
    g = np.array(list(itertools.product(range(-2, 3), repeat=4)), np.int8)
    _, keep = oracle.prune_1d(g, "i8", N, 4)
    for r in range(g.shape[0]):
        assert np.array_equal(keep[r], _brute_force_keep(g[r], "i8", N))


def test_prune_1d_hand_case():
    # one row, two groups of 4 (fp16): [0.5, -3, 0, 2 | 1, 1, -1, 4]
    # group 0 keeps |-3| and |2| (offsets 1, 3); group 1 keeps |4| (offset 3) and,
    # among the three equal magnitudes 1, the lowest offset 0.
    a = np.array([[0.5, -3, 0, 2, 1, 1, -1, 4]], np.float16).view(np.uint16)
    p, keep = oracle.prune_1d(a, "f16", 2, 4)
    assert keep.tolist() == [[0, 1, 0, 1, 1, 0, 0, 1]]
    assert p.view(np.float16).tolist() == [[0, -3, 0, 2, 1, 0, 0, 4]]


@pytest.mark.parametrize("dtype,N,M", [("f16", 2, 4), ("bf16", 2, 4), ("i8", 2, 4), ("f16", 4, 32), ("f16", 8, 32),
                                       ("f16", 3, 8), ("bf16", 5, 16)])
@pytest.mark.parametrize("op", ["N", "T"])
def test_prune_1d_invariants(dtype, N, M, op):
    rows, k = 24, 4 * M
    shape = (rows, k) if op == "N" else (k, rows)
    a = _groups(dtype, shape[0] * shape[1] // M, M, seed=5, ties=False).reshape(shape) if dtype != "i8" \
        else inputs.uniform_int(shape, 9, -127, 127)
    p, keep = oracle.prune_1d(a, dtype, N, M, op)
    logical_keep = keep if op == "N" else keep.T
    assert (logical_keep.reshape(-1, M).sum(1) == N).all()
    # kept elements copied verbatim, others exactly +0 (bits 0)
    assert np.array_equal(p[keep == 1], a[keep == 1])
    assert (p[keep == 0].view(np.uint8 if dtype == "i8" else np.uint16) == 0).all()
    # the result conforms, and pruning is idempotent
    assert oracle.check_1d(p, dtype, N, M, op) == 0
    p2, keep2 = oracle.prune_1d(p, dtype, N, M, op)
    assert np.array_equal(p2, p)
    # every kept magnitude >= every dropped magnitude in the same group
    mag = np.abs(oracle.decode(a, dtype))
    lm = (mag if op == "N" else mag.T).reshape(-1, M)
    lk = logical_keep.reshape(-1, M).astype(bool)
    for r in range(lm.shape[0]):
        if (~lk[r]).any():
            assert lm[r][lk[r]].min() >= lm[r][~lk[r]].max()


# ------------------------------------------------------------------ transposable 4x4 tiles

PAIRS = [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]


def _valid_tile_masks():
    """All 4x4 0/1 matrices with every row and column sum 2, from the full 2^16 enumeration."""
    out = []
    for v in range(1 << 16):
        t = np.array([(v >> i) & 1 for i in range(16)], np.uint8).reshape(4, 4)
        if (t.sum(0) == 2).all() and (t.sum(1) == 2).all():
            out.append(t)
    return out


def test_exactly_90_transposable_patterns():
    masks = _valid_tile_masks()
    assert len(masks) == 90                      # closed-form count for 4x4, line sums 2
    # the oracle's candidates are the same set, ordered lexicographically by row pair index
    as_pairs = sorted(tuple(PAIRS.index(tuple(np.flatnonzero(t[r]))) for r in range(4)) for t in masks)
    assert [tuple(p) for p in oracle.tile_patterns().tolist()] == as_pairs


def _tile_bruteforce(w_abs):
    """First (in row-pair lexicographic order) maximiser of the exact kept sum."""
    best, best_p = None, None
    for p in itertools.product(range(6), repeat=4):
        cols = [0] * 4
        for r in range(4):
            for c in PAIRS[p[r]]:
                cols[c] += 1
        if cols != [2, 2, 2, 2]:
            continue
        s = sum(w_abs[r][c] for r in range(4) for c in PAIRS[p[r]])
        if best is None or s > best:
            best, best_p = s, p
    keep = np.zeros((4, 4), np.uint8)
    for r in range(4):
        keep[r, list(PAIRS[best_p[r]])] = 1
    return keep, best


def _tile_dp(w_abs):
    """Independent optimum: DP over rows with state = column counts so far."""
    states = {(0, 0, 0, 0): Fraction(0)}
    for r in range(4):
        nxt = {}
        for st, val in states.items():
            for a, b in PAIRS:
                ns = list(st); ns[a] += 1; ns[b] += 1
                if max(ns) > 2:
                    continue
                v = val + w_abs[r][a] + w_abs[r][b]
                ns = tuple(ns)
                if ns not in nxt or v > nxt[ns]:
                    nxt[ns] = v
        states = nxt
    return states[(2, 2, 2, 2)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("ties", [False, True])
def test_prune_tile_equals_brute_force_and_dp(dtype, ties):
    ntiles = 60
    g = _groups(dtype, 4, 4 * ntiles, seed=31 + ties, ties=ties)      # (4*ntiles) x 4
    _, keep = oracle.prune_tile(g, dtype)
    for t in range(ntiles):
        blk = g[4 * t:4 * t + 4]
        w_abs = [_exact_abs(blk[r], dtype) for r in range(4)]
        ref_keep, ref_best = _tile_bruteforce(w_abs)
        assert np.array_equal(keep[4 * t:4 * t + 4], ref_keep), (t, blk)
        assert _tile_dp(w_abs) == ref_best


def test_prune_tile_all_equal_magnitudes_picks_first_pattern():
    # every candidate scores the same, so the first one in the order wins:
    # rows keep (0,1), (0,1), (2,3), (2,3)
    a = np.ones((4, 4), np.float16).view(np.uint16)
    _, keep = oracle.prune_tile(a, "f16")
    assert keep.tolist() == [[1, 1, 0, 0], [1, 1, 0, 0], [0, 0, 1, 1], [0, 0, 1, 1]]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prune_tile_invariants(dtype):
    a = inputs.normal((64, 96), 77, 0.02, dtype)
    p, keep = oracle.prune_tile(a, dtype)
    t = keep.reshape(16, 4, 24, 4).transpose(0, 2, 1, 3)
    assert (t.sum(3) == 2).all() and (t.sum(2) == 2).all()
    assert oracle.check_tile(p, dtype) == 0
    # both directions are 2:4 along their k
    assert oracle.check_1d(p, dtype, 2, 4, "N") == 0
    assert oracle.check_1d(p, dtype, 2, 4, "T") == 0
    # kept sum never beats the row-wise or the column-wise 1-D optimum
    mag = np.abs(oracle.decode(a, dtype))
    _, krow = oracle.prune_1d(a, dtype, 2, 4, "N")
    _, kcol = oracle.prune_1d(a, dtype, 2, 4, "T")
    def tile_sums(kp):
        return (mag * kp).reshape(16, 4, 24, 4).sum(axis=(1, 3))
    st, sr, sc = tile_sums(keep), tile_sums(krow), tile_sums(kcol)
    assert (st <= sr + 1e-12).all() and (st <= sc + 1e-12).all()
    # where the row-wise 1-D mask is itself transposable, the tile optimum equals it
    kr = krow.reshape(16, 4, 24, 4).transpose(0, 2, 1, 3)
    transposable = (kr.sum(2) == 2).all(axis=2)
    assert np.allclose(st[transposable], sr[transposable], rtol=0, atol=1e-12)


def _tile_first_max_float(w):
    """First maximiser over the 90 patterns when magnitudes may be NaN or Inf: a
    candidate keeping a NaN has a NaN score, which never compares greater, so it
    can never replace the current winner; when no candidate has an ordered score
    the first pattern (rows (0,1), (0,1), (2,3), (2,3)) stays."""
    best, best_p = None, (0, 0, 5, 5)
    for p in itertools.product(range(6), repeat=4):
        cols = [0] * 4
        for r in range(4):
            for c in PAIRS[p[r]]:
                cols[c] += 1
        if cols != [2, 2, 2, 2]:
            continue
        kept = [w[r][c] for r in range(4) for c in PAIRS[p[r]]]
        if any(np.isnan(x) for x in kept):
            continue
        if any(np.isinf(x) for x in kept):
            s = float("inf")
        else:
            s = sum((Fraction(float(x)) for x in kept), Fraction(0))
        if best is None or s > best:
            best, best_p = s, p
    keep = np.zeros((4, 4), np.uint8)
    for r in range(4):
        keep[r, list(PAIRS[best_p[r]])] = 1
    return keep


def nan_inf_tiles(dtype):
    """4x4 tiles (stacked vertically) holding NaN and Inf: one NaN element, a NaN
    row, a NaN column, NaN everywhere, one +Inf, two -Inf in different rows."""
    nan_bits = 0x7E00 if dtype == "f16" else 0x7FC0
    inf_bits = 0x7C00 if dtype == "f16" else 0x7F80
    base = _groups(dtype, 4, 24, seed=404, ties=False)
    t = base.copy()
    t[0, 0] = nan_bits
    t[4 + 2, :] = nan_bits
    t[8:12, 1] = nan_bits
    t[12:16, :] = nan_bits | 0x8000
    t[16 + 1, 2] = inf_bits
    t[20 + 0, 3] = inf_bits | 0x8000
    t[20 + 3, 0] = inf_bits | 0x8000
    return t


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prune_tile_nan_and_inf(dtype):
    t = nan_inf_tiles(dtype)
    _, keep = oracle.prune_tile(t, dtype)
    mags = np.abs(oracle.decode(t, dtype))
    for i in range(t.shape[0] // 4):
        ref = _tile_first_max_float(mags[4 * i:4 * i + 4])
        assert np.array_equal(keep[4 * i:4 * i + 4], ref), i
    # a NaN row, a NaN column and an all-NaN tile leave no ordered candidate: first pattern
    first = [[1, 1, 0, 0], [1, 1, 0, 0], [0, 0, 1, 1], [0, 0, 1, 1]]
    for i in (1, 2, 3):
        assert keep[4 * i:4 * i + 4].tolist() == first, i
    # every tile still keeps two per row and per column
    kt = keep.reshape(-1, 4, 4)
    assert (kt.sum(1) == 2).all() and (kt.sum(2) == 2).all()


# ------------------------------------------------------------------ keep-mask packing

def test_mask_bits_hand_cases():
    """Keep masks pack into uint32 words least significant bit first, each row
    starting a new word (ceil(cols / 32) words per row)."""
    k = np.array([[1, 0, 1, 1]], np.uint8)                       # bits 0, 2, 3
    assert oracle.mask_bits(k).tolist() == [[0b1101]]
    k = np.zeros((2, 33), np.uint8)
    k[0, 0] = k[0, 5] = k[0, 32] = 1                              # word 0 = 1 + 32, word 1 = 1 (column 32)
    k[1, 31] = 1                                                  # a new row starts a new word
    assert oracle.mask_bits(k).tolist() == [[33, 1], [0x80000000, 0]]
    k = np.zeros((1, 64), np.uint8)
    k[0, 31] = k[0, 63] = k[0, 40] = 1
    assert oracle.mask_bits(k).tolist() == [[0x80000000, 0x80000100]]
    k = np.zeros((3, 4), np.uint8)
    k[2, 1] = 1
    assert oracle.mask_bits(k).tolist() == [[0], [0], [2]]
    k = np.ones((1, 70), np.uint8)                                # ragged last word: 6 low bits
    assert oracle.mask_bits(k).tolist() == [[0xFFFFFFFF, 0xFFFFFFFF, 0x3F]]


# ------------------------------------------------------------------ prune check

def test_check_counts_injected_violations():
    a = inputs.normal((8, 32), 3, 1.0, "f16")
    p, keep = oracle.prune_1d(a, "f16", 2, 4)
    assert oracle.check_1d(p, "f16", 2, 4) == 0
    q = p.copy()
    r, c = 3, 9
    zero_pos = np.flatnonzero(keep[r, 8:12] == 0)[0] + 8
    q[r, zero_pos] = np.float16(1.5).view(np.uint16)
    assert oracle.check_1d(q, "f16", 2, 4) == 1
    q[5, 20:24] = np.float16(1.0).view(np.uint16)          # a full group: one more violation
    assert oracle.check_1d(q, "f16", 2, 4) == 2
    # -0.0 is zero
    z = p.copy(); z[keep == 0] = np.float16(-0.0).view(np.uint16)
    assert oracle.check_1d(z, "f16", 2, 4) == 0


def test_check_tile_counts_rows_and_columns():
    a = inputs.normal((8, 8), 4, 1.0, "bf16")
    p, keep = oracle.prune_tile(a, "bf16")
    assert oracle.check_tile(p, "bf16") == 0
    q = p.copy()
    r, c = np.argwhere(keep[:4, :4] == 0)[0]
    q[r, c] = 0x3F80                                         # bf16 1.0 at a dropped slot
    assert oracle.check_tile(q, "bf16") == 2                 # its tile row and its tile column


# ------------------------------------------------------------------ compress / decompress

def test_compress_hand_case_2of4():
    a = np.array([[0.5, -3, 0, 2, 1, 1, -1, 4]], np.float16).view(np.uint16)
    v, m = oracle.compress(a, "f16", 2, 4)
    # values: kept entries in increasing offset: -3, 2 | 1, 4; padded to 16 bytes
    assert v.shape == (1, 8) and v.view(np.float16)[0, :4].tolist() == [-3, 2, 1, 4]
    assert (v[0, 4:] == 0).all()
    # metadata: group 0 offsets (1, 3) -> 1 | 3<<2 = 0xD; group 1 offsets (0, 3) -> 0 | 3<<2 = 0xC
    # little-endian bit stream: byte 0 = 0xD | 0xC << 4 = 0xCD; row padded to 16 bytes
    assert m.shape == (1, 16) and m[0, 0] == 0xCD and (m[0, 1:] == 0).all()


def test_compress_hand_case_4of32():
    # one group of 32 with the four largest magnitudes at offsets 3, 7, 20, 31
    x = np.full(32, 0.25, np.float16)
    x[[3, 7, 20, 31]] = [8, -7, 6, -5]
    v, m = oracle.compress(x[None, :].view(np.uint16), "f16", 4, 32)
    assert v.view(np.float16)[0, :4].tolist() == [8, -7, 6, -5]
    # 5-bit fields: 3 | 7<<5 | 20<<10 | 31<<15 = 3 + 224 + 20480 + 1015808 = 1036515 = 0x0FD0E3
    assert oracle.meta_bits(32) == 5
    assert m[0, :3].tolist() == [0xE3, 0xD0, 0x0F] and (m[0, 3:] == 0).all()


@pytest.mark.parametrize("dtype,N,M", [("f16", 2, 4), ("bf16", 2, 4), ("i8", 2, 4), ("f16", 4, 32),
                                       ("f16", 8, 32), ("bf16", 1, 8), ("i8", 3, 16), ("f16", 7, 8)])
@pytest.mark.parametrize("op", ["N", "T"])
def test_round_trips(dtype, N, M, op):
    rows, k = 20, 3 * M * (2 if M < 32 else 1)
    shape = (rows, k) if op == "N" else (k, rows)
    a = inputs.normal(shape, 11, 1.0, dtype) if dtype != "i8" else inputs.uniform_int(shape, 11, -127, 127)
    p, keep = oracle.prune_1d(a, dtype, N, M, op)
    v, m = oracle.compress(a, dtype, N, M, op)
    # compress(A) == compress(prune(A))
    v2, m2 = oracle.compress(p, dtype, N, M, op)
    assert np.array_equal(v, v2) and np.array_equal(m, m2)
    # decompress(compress(A)) == prune(A) bitwise
    d = oracle.decompress(v, m, dtype, rows, k, N, M, op)
    assert np.array_equal(d, p)
    # compress(decompress(V, meta)) == (V, meta)
    v3, m3 = oracle.compress(d, dtype, N, M, op)
    assert np.array_equal(v3, v) and np.array_equal(m3, m)
    # sizes and zero padding
    b = oracle.meta_bits(M)
    used_bits = (k // M) * N * b
    assert m.shape[1] % 16 == 0 and m.shape[1] * 8 >= used_bits
    bits = np.unpackbits(m, axis=1, bitorder="little")
    assert (bits[:, used_bits:] == 0).all()
    assert (v[:, k * N // M:].view(np.uint8) == 0).all()
    # offsets inside each group are strictly increasing
    fields = bits[:, :used_bits].reshape(rows, -1, b)
    offs = (fields * (1 << np.arange(b))).sum(2).reshape(rows, k // M, N)
    assert (np.diff(offs, axis=2) > 0).all()


# ------------------------------------------------------------------ the product

def _pruned_case(dtype, m, k, n, N, M, seed):
    a = inputs.normal((m, k), seed, 1.0, dtype) if dtype != "i8" else inputs.uniform_int((m, k), seed, -127, 127)
    p, _ = oracle.prune_1d(a, dtype, N, M)
    v, meta = oracle.compress(a, dtype, N, M)
    b = inputs.normal((k, n), seed + 1, 1.0, dtype) if dtype != "i8" else inputs.uniform_int((k, n), seed + 1, -127, 127)
    return p, v, meta, b


@pytest.mark.parametrize("dtype,N,M", [("f16", 2, 4), ("bf16", 2, 4), ("f16", 4, 32), ("bf16", 3, 8)])
def test_sparse_loop_equals_dense_loop_exactly(dtype, N, M):
    m, k, n = 33, 128, 17
    p, v, meta, b = _pruned_case(dtype, m, k, n, N, M, 100)
    A = oracle.decode(p, dtype); B = oracle.decode(b, dtype)
    C = oracle.decode(inputs.normal((m, n), 7, 1.0, dtype), dtype)
    dense = oracle.gemm_f64(A, B, 0.75, -0.5, C)
    sparse = oracle.spmm_compressed_f64(v, meta, dtype, m, k, N, M, B, 0.75, -0.5, C)
    assert np.array_equal(dense, sparse)


def test_gemm_matches_library_matmul():
    rng = np.random.default_rng(0)
    A = rng.standard_normal((37, 53)); B = rng.standard_normal((53, 29)); C = rng.standard_normal((37, 29))
    got = oracle.gemm_f64(A, B, 1.5, 0.25, C)
    ref = 1.5 * (A @ B) + 0.25 * C
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    pi = np.array([0, 36, 5, 17]); pj = np.array([0, 28, 13, 2])
    pts = oracle.gemm_f64_points(A, np.ascontiguousarray(B.T), pi, pj, 1.5, 0.25, C[pi, pj])
    assert np.array_equal(pts, got[pi, pj]) or np.allclose(pts, got[pi, pj], rtol=1e-14, atol=0)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gemm_special_cases(dtype):
    m, k = 24, 64
    p, v, meta, _ = _pruned_case(dtype, m, k, 8, 2, 4, 300)
    A = oracle.decode(p, dtype)
    I = np.eye(k)
    assert np.array_equal(oracle.gemm_f64(A, I), A)                              # B = I -> D = A
    perm = np.random.default_rng(1).permutation(k)
    P = I[:, perm]
    assert np.array_equal(oracle.gemm_f64(A, P), A[:, perm])                     # permutation -> permuted columns
    C = np.random.default_rng(2).standard_normal((m, k))
    assert np.array_equal(oracle.gemm_f64(A, I, 0.0, 1.0, C), C)                 # alpha = 0, beta = 1 -> C
    assert not oracle.gemm_f64(A, I, 0.0, 0.0, C).any()                          # alpha = beta = 0 -> 0
    # the sparse loop agrees on the identity too (the metadata points at the right rows of B)
    assert np.array_equal(oracle.spmm_compressed_f64(v, meta, dtype, m, k, 2, 4, I), A)


def test_int_gemm_exact():
    m, k, n = 40, 64, 24
    p, v, meta, b = _pruned_case("i8", m, k, n, 2, 4, 500)
    C = inputs.uniform_int((m, n), 9, -2**20, 2**20, np.int32)
    got = oracle.gemm_i64(p, b, 1, 1, C)
    ref = p.astype(np.int64) @ b.astype(np.int64) + C                              # exact integer library product
    assert np.array_equal(got, ref)
    got2 = oracle.gemm_i64(p, b, -3, 2, C)
    assert np.array_equal(got2, -3 * (p.astype(np.int64) @ b.astype(np.int64)) + 2 * C.astype(np.int64))


def test_tolerance_formula():
    absA = np.array([[1.0, 2.0]]); absB = np.array([[3.0], [4.0]])
    # 1e-2 * (1*3 + 2*4) + 1e-3 = 0.111
    assert np.allclose(oracle.tolerance(absA, absB), [[0.111]], rtol=0, atol=1e-15)
    C = np.array([[10.0]])
    assert np.allclose(oracle.tolerance(absA, absB, 2.0, -1.0, C), [[1e-2 * (22 + 10) + 1e-3]], rtol=0, atol=1e-15)


def test_int8_output_saturates_the_exact_integer():
    """Closed forms: a row of 127s against a column of 127s sums to 127^2 k
    (saturates high), its negation saturates low, alternating signs cancel to
    0, and small sums pass through unchanged; beta * C with int8 C adds in."""
    k = 8
    a = np.full((1, k), 127, np.int8)
    b = np.full((k, 1), 127, np.int8)
    assert oracle.gemm_i8_saturated(a, b)[0, 0] == 127
    assert oracle.gemm_i8_saturated(a, -b)[0, 0] == -128
    alt = np.array([[1, -1] * (k // 2)], np.int8)
    assert oracle.gemm_i8_saturated(alt, b)[0, 0] == 0
    small = np.array([[1, 2, 3, 0, 0, 0, 0, -1]], np.int8)
    ones = np.ones((k, 1), np.int8)
    assert oracle.gemm_i8_saturated(small, ones)[0, 0] == 5
    c = np.array([[-100]], np.int8)
    assert oracle.gemm_i8_saturated(small, ones, 2, 1, c)[0, 0] == -90
    assert oracle.gemm_i8_saturated(small, ones, 1, 3, c)[0, 0] == -128


# ------------------------------------------------------------------ vector-wise N:M

def _vw_scores_exact(block, dtype):
    """Exact |sum over the block's rows| per column (Fractions)."""
    vals = oracle.decode(block, dtype)
    return [abs(sum((Fraction(float(vals[r, j])) for r in range(vals.shape[0])), Fraction(0)))
            for j in range(vals.shape[1])]


def _vw_brute_force(block, dtype, N):
    """argmax over all N-subsets of the exact summed vector scores; among equal
    sums the lexicographically smallest index tuple (ties to the lower offset)."""
    sc = _vw_scores_exact(block, dtype)
    best, best_set = None, None
    for sub in itertools.combinations(range(len(sc)), N):
        s = sum((sc[i] for i in sub), Fraction(0))
        if best is None or s > best:
            best, best_set = s, sub
    keep = np.zeros(len(sc), np.uint8)
    keep[list(best_set)] = 1
    return keep


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("V,M,Ns,blocks", [(2, 4, (1, 2, 3), 60), (4, 8, (1, 3, 5), 20), (16, 32, (1, 2, 4), 2),
                                           (16, 4, (2,), 20)])
@pytest.mark.parametrize("ties", [False, True])
def test_prune_vw_equals_brute_force(dtype, V, M, Ns, blocks, ties):
    g = _groups(dtype, M, V * blocks, seed=V * 13 + M + ties, ties=ties)       # (V*blocks) x M
    for N in Ns:
        _, keep = oracle.prune_vw(g, dtype, V, N, M)
        for b in range(blocks):
            blk = g[b * V:(b + 1) * V]
            ref = _vw_brute_force(blk, dtype, N)
            for r in range(V):
                assert np.array_equal(keep[b * V + r], ref), (dtype, V, M, N, b, blk)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("N,M", [(2, 4), (4, 32), (3, 8)])
def test_prune_vw_with_one_row_is_the_1d_rule(dtype, N, M):
    """A vector of one element scores |w|: V = 1 is the element-wise rule."""
    a = _groups(dtype, M, 40, seed=N + M, ties=True).reshape(10, 4 * M)
    p1, k1 = oracle.prune_1d(a, dtype, N, M)
    pv, kv = oracle.prune_vw(a, dtype, 1, N, M)
    assert np.array_equal(k1, kv) and np.array_equal(p1, pv)


def test_prune_vw_scores_the_signed_sum():
    """The page's vector score is |sum|, not sum of |.|: a vector whose values
    cancel scores zero. Rows (1, 3, -2, 0.5) and (-1, 0, 2, 0.5): scores 0, 3,
    0, 1 keep offsets 1 and 3 (the sum of magnitudes 2, 3, 4, 1 would keep 1, 2)."""
    a = np.array([[1, 3, -2, 0.5], [-1, 0, 2, 0.5]], np.float16).view(np.uint16)
    p, keep = oracle.prune_vw(a, "f16", 2, 2, 4)
    assert keep.tolist() == [[0, 1, 0, 1], [0, 1, 0, 1]]
    assert p.view(np.float16).tolist() == [[0, 3, 0, 0.5], [0, 0, 0, 0.5]]


@pytest.mark.parametrize("dtype,V,N,M", [("f16", 16, 4, 32), ("bf16", 16, 8, 32), ("i8", 32, 2, 4), ("f16", 64, 2, 8)])
def test_prune_vw_invariants(dtype, V, N, M):
    rows, k = 2 * V, 4 * M
    a = (_groups(dtype, k, rows, seed=77, ties=False) if dtype != "i8"
         else inputs.uniform_int((rows, k), 9, -127, 127))
    p, keep = oracle.prune_vw(a, dtype, V, N, M)
    kb = keep.reshape(rows // V, V, k)
    assert (kb == kb[:, :1, :]).all()                               # a block's rows share the offsets
    assert (keep.reshape(-1, M).sum(1) == N).all()
    assert np.array_equal(p[keep == 1], a[keep == 1])
    assert (p[keep == 0].view(np.uint8 if dtype == "i8" else np.uint16) == 0).all()
    assert oracle.check_vw(p, dtype, V, N, M) == 0
    p2, _ = oracle.prune_vw(p, dtype, V, N, M)
    assert np.array_equal(p2, p)


def test_check_vw_counts_blocks_using_too_many_offsets():
    a = inputs.normal((32, 64), 5, 1.0, "f16")
    p, keep = oracle.prune_vw(a, "f16", 16, 4, 32)
    assert oracle.check_vw(p, "f16", 16, 4, 32) == 0
    q = p.copy()
    j = int(np.flatnonzero(keep[3, :32] == 0)[0])
    q[3, j] = np.float16(0.25).view(np.uint16)                     # one row uses a fifth offset
    assert oracle.check_vw(q, "f16", 16, 4, 32) == 1
    q[20, 32 + int(np.flatnonzero(keep[20, 32:] == 0)[0])] = np.float16(1).view(np.uint16)
    assert oracle.check_vw(q, "f16", 16, 4, 32) == 2
    z = p.copy(); z[keep == 0] = np.float16(-0.0).view(np.uint16)   # -0 is zero
    assert oracle.check_vw(z, "f16", 16, 4, 32) == 0


def test_compress_vw_hand_case():
    # V = 2, 2:4, k = 8, fp16. Block rows (1, 3, -2, 0.5 | 0, 0, 4, -4) and
    # (-1, 0, 2, 0.5 | 0, 0, 4, 4): group 0 scores 0, 3, 0, 1 -> offsets 1, 3;
    # group 1 scores 0, 0, 8, 0 -> offsets 2 and, among the tied zeros, 0.
    a = np.array([[1, 3, -2, 0.5, 0, 0, 4, -4], [-1, 0, 2, 0.5, 0, 0, 4, 4]], np.float16).view(np.uint16)
    v, meta = oracle.compress_vw(a, "f16", 2, 2, 4)
    assert v.shape == (2, 8) and meta.shape == (1, 16)
    assert v.view(np.float16)[:, :4].tolist() == [[3, 0.5, 0, 4], [0, 0.5, 0, 4]]
    assert (v[:, 4:] == 0).all()
    # one metadata row for the block: nibbles 1 | 3 << 2 = 0xD, then 0 | 2 << 2 = 0x8
    assert meta[0, 0] == 0x8D and (meta[0, 1:] == 0).all()


@pytest.mark.parametrize("dtype,V,N,M", [("f16", 16, 4, 32), ("bf16", 16, 2, 4), ("i8", 32, 8, 32), ("f16", 16, 3, 8)])
def test_vw_round_trips(dtype, V, N, M):
    rows, k = 2 * V, 3 * M * 2
    a = (_groups(dtype, k, rows, seed=3, ties=True) if dtype != "i8"
         else inputs.uniform_int((rows, k), 4, -3, 3))
    p, _ = oracle.prune_vw(a, dtype, V, N, M)
    v, meta = oracle.compress_vw(a, dtype, V, N, M)
    assert np.array_equal(oracle.decompress_vw(v, meta, dtype, rows, k, V, N, M), p)
    v2, m2 = oracle.compress_vw(oracle.decompress_vw(v, meta, dtype, rows, k, V, N, M), dtype, V, N, M)
    assert np.array_equal(v2, v) and np.array_equal(m2, meta)
    # compress(A) == compress(prune(A))
    v3, m3 = oracle.compress_vw(p, dtype, V, N, M)
    assert np.array_equal(v3, v) and np.array_equal(m3, meta)


@pytest.mark.parametrize("dtype,V,N,M", [("f16", 16, 4, 32), ("bf16", 16, 8, 32), ("f16", 32, 2, 4)])
def test_vw_sparse_loop_equals_dense_loop(dtype, V, N, M):
    m, k, n = 2 * V, 4 * M, 24
    a = inputs.normal((m, k), 8, 1.0, dtype)
    b = inputs.normal((k, n), 9, 1.0, dtype)
    p, _ = oracle.prune_vw(a, dtype, V, N, M)
    v, meta = oracle.compress_vw(a, dtype, V, N, M)
    B = oracle.decode(b, dtype)
    dense = oracle.gemm_f64(oracle.decode(p, dtype), B)
    sparse = oracle.spmm_compressed_vw_f64(v, meta, dtype, m, k, V, N, M, B)
    assert np.array_equal(dense, sparse)
