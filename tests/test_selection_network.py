"""CPU model of the per-group top-N selection network that the register path
uses for M = 32 (N = 4 or 8), and of its search-free 2 of 4, checked against
brute force on tie-heavy groups.

The model performs the same compare-exchange sequence as the device code: runs
of four sorted, (N = 8) pairs of runs merged into sorted runs of eight through
a bitonic sort, then repeated element-wise maxima of one run against the other
reversed (the top N of the pair, as a bitonic sequence), sorted again between
levels. Keys are (|x| << 6) | ((31 - j) << 1) | sign, unique per group. The
selection must equal the N largest magnitudes with ties to the lower offset j,
and the key must give back the element's offset, sign and magnitude. The GPU
parity tests run the network itself on the same kind of tie-heavy groups."""
import random


def _cx(k, a, b):
    k[a], k[b] = max(k[a], k[b]), min(k[a], k[b])


def _bitonic_desc(k, o, n):
    st = n // 2
    while st >= 1:
        for i in range(n):
            if (i & st) == 0:
                _cx(k, o + i, o + i + st)
        st //= 2


def _network_top_n32(keys, N):
    k = list(keys)
    for g in range(8):
        for a, b in [(0, 1), (2, 3), (0, 2), (1, 3), (1, 2)]:
            _cx(k, 4 * g + a, 4 * g + b)
    runs = [k[4 * g:4 * g + 4] for g in range(8)]
    if N == 8:
        merged = []
        for i in range(0, 8, 2):
            c = runs[i] + runs[i + 1][::-1]
            _bitonic_desc(c, 0, 8)
            merged.append(c)
        runs = merged
    while len(runs) > 1:
        nxt = []
        for i in range(0, len(runs), 2):
            c = [max(runs[i][t], runs[i + 1][N - 1 - t]) for t in range(N)]
            if len(runs) > 2:
                _bitonic_desc(c, 0, N)
            nxt.append(c)
        runs = nxt
    return runs[0]


def test_selection_network_matches_brute_force():
    rng = random.Random(1)
    for trial in range(20000):
        N = rng.choice([4, 8])
        mags = [rng.choice([0, 1, 2, 3, rng.randint(0, 0x7FFF)]) for _ in range(32)]
        signs = [rng.randint(0, 1) for _ in range(32)]
        keys = [(mags[j] << 6) | ((31 - j) << 1) | signs[j] for j in range(32)]
        sel = _network_top_n32(keys, N)
        got = sorted(31 - ((x >> 1) & 31) for x in sel)
        ref = sorted(sorted(range(32), key=lambda j: (-mags[j], j))[:N])
        assert got == ref, (trial, N, mags)
        # offset order of the winners, and their bits recovered from the keys
        rk = sorted([(((x >> 1) & 31) << 16) | ((x & 1) << 15) | (x >> 6) for x in sel], reverse=True)
        assert [31 - (r >> 16) for r in rk] == ref
        assert all((r & 0xFFFF) == ((signs[31 - (r >> 16)] << 15) | mags[31 - (r >> 16)]) for r in rk)


def test_selection_network_all_equal_and_zero_groups():
    for N in (4, 8):
        for mag in (0, 1, 0x7C00):
            for signs in ([0] * 32, [1] * 32, [j % 2 for j in range(32)]):
                keys = [(mag << 6) | ((31 - j) << 1) | signs[j] for j in range(32)]
                got = sorted(31 - ((x >> 1) & 31) for x in _network_top_n32(keys, N))
                assert got == list(range(N))


# ---- 2 of 4 without a search (the register path's 2:4 prune and compress)
#
# Keys (mag << 2) | (3 - j) are unique per group; with a, b the smaller and
# larger key of elements 0 and 1 and c, d those of elements 2 and 3, the kernel
# takes the largest key as max(b, d) and the second largest as
# max(min(b, d), a, c), and reads the two kept offsets from their low bits.

def _top2of4_model(mag):
    k = [(mag[j] << 2) | (3 - j) for j in range(4)]
    a, b, c, d = min(k[0], k[1]), max(k[0], k[1]), min(k[2], k[3]), max(k[2], k[3])
    t1, t2 = max(b, d) & 3, max(min(b, d), a, c) & 3
    return 3 - max(t1, t2), 3 - min(t1, t2)


def _top2of4_brute(mag):
    order = sorted(range(4), key=lambda j: (-mag[j], j))   # larger magnitude first, then lower offset
    return tuple(sorted(order[:2]))


def test_two_of_four_network_every_tie_pattern():
    """Every group over a five-value magnitude alphabet (all tie patterns), and
    the extremes of the 15-bit magnitude key."""
    vals = [0, 1, 2, 3, 0x7FFF]
    for m0 in vals:
        for m1 in vals:
            for m2 in vals:
                for m3 in vals:
                    mag = [m0, m1, m2, m3]
                    assert _top2of4_model(mag) == _top2of4_brute(mag), mag


def test_two_of_four_network_random():
    rng = random.Random(2024)
    for _ in range(20000):
        mag = [rng.choice([rng.randrange(0x8000), rng.randrange(4)]) for _ in range(4)]
        assert _top2of4_model(mag) == _top2of4_brute(mag), mag
