"""AddressSanitizer / UndefinedBehaviorSanitizer builds on the CPU: the C ABI's
host code (plan validation, size queries, settings, argument checks; no device
call) and the oracle, each driven by a small C/C++ program under tests/sanitize.
The library's host TU is rebuilt with the sanitizers on its host side only and
linked with the normally built kernel objects; the oracle is plain C."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "structured_sparse_gemm_nm_amd", "csrc")
OBJS = os.path.join(ROOT, "structured_sparse_gemm_nm_amd", "_build")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
# sanitizers on the host compilation only (the device code is built as usual)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-ffp-contract=off",
         "-o", exe, os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm"])
    r = run([exe], env=ENV)
    assert "oracle driver: 0 failures" in r.stdout


def test_host_api_under_address_and_undefined_sanitizers(tmp_path):
    kernels = ["nm_prune", "nm_rows", "nm_vw", "nm_gemm", "nm_gemm_f16", "nm_gemm_bf16", "nm_gemm_i8",
               "nm_skinny_f16", "nm_skinny_bf16", "nm_skinny_i8"]
    objs = [os.path.join(OBJS, k + ".o") for k in kernels]
    if not all(os.path.exists(o) for o in objs) or not os.path.exists(HIPCC):
        pytest.skip("the library's kernel objects are not built (run the build first)")
    api = str(tmp_path / "nm_api_san.o")
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC"] + HOST_SAN +
        ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-c", os.path.join(CSRC, "nm_api.hip"), "-o", api])
    exe = str(tmp_path / "api_san")
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17"] + HOST_SAN +
        ["-I" + os.path.join(ROOT, "include"), "-x", "hip", os.path.join(SAN, "api_driver.cpp"),
         "-x", "none", api] + objs + ["-o", exe])
    r = run([exe], env=ENV, timeout=300)
    assert "api driver: 0 failures" in r.stdout
