"""The pins are strong enough: each plants one plausible mistake in a copy of the
oracle's C source (on the CPU, in a temporary directory), rebuilds it, and checks
that a pin from test_oracle_pins fails. The real oracle is restored afterwards."""
import os
import shutil
import subprocess

import pytest

import oracle
import oracle.oracle as orc
from tests import test_oracle_pins as pins

MUTATIONS = [
    ("ties go to the higher index",
     "while (b >= 0 && key[order[b]] < key[o])", "while (b >= 0 && key[order[b]] <= key[o])",
     lambda: pins.test_prune_1d_exhaustive_int8_small_values(2)),
    ("keeps the smallest magnitudes",
     "order[b + 1] = o;\n  }\n  memset(keep, 0, (size_t)M);\n  for (int s = 0; s < N; s++) keep[order[s]] = 1;",
     "order[b + 1] = o;\n  }\n  memset(keep, 0, (size_t)M);\n  for (int s = 0; s < N; s++) keep[order[M - 1 - s]] = 1;",
     lambda: pins.test_prune_1d_equals_brute_force("f16", 4, (2,), 50, False)),
    ("tile score drops its last row",
     "double score = ((s[0] + s[1]) + s[2]) + s[3];", "double score = ((s[0] + s[1]) + s[2]);",
     lambda: pins.test_prune_tile_equals_brute_force_and_dp("f16", False)),
    ("tile enumeration skips candidates",
     "if (col[0] == 2 && col[1] == 2 && col[2] == 2 && col[3] == 2) {",
     "if (col[0] == 2 && col[1] == 2 && col[2] == 2 && col[3] == 2 && p0 <= p3) {",
     pins.test_exactly_90_transposable_patterns),
    ("metadata fields written most-significant bit first",
     "row, (size_t)(g * M + j), dt);\n        int64_t t0 = (g * N + s) * (int64_t)b;\n        for (int q = 0; q < b; q++) put_bit(mrow, t0 + q, (j >> q) & 1);",
     "row, (size_t)(g * M + j), dt);\n        int64_t t0 = (g * N + s) * (int64_t)b;\n        for (int q = 0; q < b; q++) put_bit(mrow, t0 + (b - 1 - q), (j >> q) & 1);",
     lambda: pins.test_round_trips("f16", 2, 4, "N")),
    ("fp16 exponent bias off by one",
     "else v = ldexp((double)(f + 1024), e - 25);", "else v = ldexp((double)(f + 1024), e - 24);",
     pins.test_f16_decode_all_bit_patterns),
    ("product reads B transposed",
     "for (int64_t j = 0; j < n; j++) acc[j] += a * brow[j];", "for (int64_t j = 0; j < n; j++) acc[j] += a * B[j * k + kk];",
     pins.test_gemm_matches_library_matmul),
    ("negative zero counted as a non-zero",
     "return (((const uint16_t*)p)[i] & 0x7FFFu) != 0;", "return ((const uint16_t*)p)[i] != 0;",
     pins.test_check_counts_injected_violations),
    ("decompress drops the last kept value of each group",
     "meta + r * meta_ld;\n    for (int64_t g = 0; g < cols / M; g++)\n      for (int s = 0; s < N; s++) {",
     "meta + r * meta_ld;\n    for (int64_t g = 0; g < cols / M; g++)\n      for (int s = 0; s < N - 1; s++) {",
     lambda: pins.test_round_trips("bf16", 2, 4, "T")),
    ("vector score sums magnitudes",
     "for (int v = 0; v < V; v++) s += elem_f64(a, dt, (size_t)((r0 + v) * cols + c));",
     "for (int v = 0; v < V; v++) s += fabs(elem_f64(a, dt, (size_t)((r0 + v) * cols + c)));",
     pins.test_prune_vw_scores_the_signed_sum),
    ("vector score skips the block's last row",
     "for (int v = 0; v < V; v++) s += elem_f64(a, dt, (size_t)((r0 + v) * cols + c));",
     "for (int v = 0; v < V - 1; v++) s += elem_f64(a, dt, (size_t)((r0 + v) * cols + c));",
     lambda: pins.test_prune_vw_equals_brute_force("f16", 2, 4, (1, 2, 3), 60, False)),
    ("vector ties go to the higher offset",
     "while (y >= 0 && key[order[y]] < key[o])", "while (y >= 0 && key[order[y]] <= key[o])",
     lambda: pins.test_prune_vw_equals_brute_force("i8", 2, 4, (1, 2, 3), 60, True)),
    ("vector-wise compress writes the block's offsets into the wrong metadata field",
     "        int64_t t0 = (g * N + s) * (int64_t)b;\n        for (int q = 0; q < b; q++) put_bit(mrow, t0 + q, (j >> q) & 1);\n        s++;\n      }\n    }\n  }\n}\n\nvoid or_decompress_vw",
     "        int64_t t0 = (g * N + (N - 1 - s)) * (int64_t)b;\n        for (int q = 0; q < b; q++) put_bit(mrow, t0 + q, (j >> q) & 1);\n        s++;\n      }\n    }\n  }\n}\n\nvoid or_decompress_vw",
     pins.test_compress_vw_hand_case),
]


@pytest.mark.parametrize("name,old,new,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, pin, tmp_path, monkeypatch):
    src = open(orc._SRC).read()
    assert src.count(old) == 1, name
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                           "-o", str(so), str(mutated), "-lm"])
    monkeypatch.setattr(orc, "_SRC", str(mutated))
    monkeypatch.setattr(orc, "_SO", str(so))
    monkeypatch.setattr(orc, "_lib", None)
    with pytest.raises(AssertionError):
        pin()
    monkeypatch.setattr(orc, "_lib", None)


# Mistakes planted in the Python side of the oracle (the keep-mask packing):
# the mutated function replaces oracle.mask_bits for the duration of the pin.
PY_MUTATIONS = [
    ("mask bits packed most-significant bit first", 'bitorder="little"', 'bitorder="big"'),
    ("mask rows padded to 64-bit words", "words = (cols + 31) // 32", "words = (cols + 63) // 64 * 2"),
    ("mask rows run on without a fresh word", "padded[:, :cols] = keep",
     "padded = np.zeros((rows, words * 32), np.uint8); padded.reshape(-1)[:rows * cols] = keep.reshape(-1)"),
]


@pytest.mark.parametrize("name,old,new", PY_MUTATIONS, ids=[m[0] for m in PY_MUTATIONS])
def test_planted_mask_mistake_is_caught(name, old, new, monkeypatch):
    import inspect
    import numpy as np
    src = inspect.getsource(orc.mask_bits)
    assert src.count(old) == 1, name
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    monkeypatch.setattr(orc, "mask_bits", ns["mask_bits"])
    monkeypatch.setattr(oracle, "mask_bits", ns["mask_bits"])
    with pytest.raises(AssertionError):
        pins.test_mask_bits_hand_cases()
