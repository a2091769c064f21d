"""Build libnmsparse.so (HIP kernels + C ABI) for gfx950, in-tree.

The library is linked against the HIP runtime that PyTorch ships (torch/lib),
so that a process using torch for device memory and streams has exactly one
HIP runtime: the stream handles and device pointers torch hands over are then
valid inside the library.
"""
import importlib.util
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnmsparse.so")
CAL_LIB = os.path.join(HERE, "libnmcal.so")       # calibration loops for the benchmark (not the ABI)
SOURCES = ["nm_api.hip", "nm_prune.hip", "nm_rows.hip", "nm_vw.hip", "nm_gemm.hip", "nm_gemm_f16.hip", "nm_gemm_bf16.hip",
           "nm_gemm_i8.hip",
           "nm_skinny_f16.hip", "nm_skinny_bf16.hip", "nm_skinny_i8.hip"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
ARCH = "gfx950"
CFLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          # keep the compiler from forming packed fp32 instructions
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def torch_lib_dir():
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        raise RuntimeError("torch is not importable: cannot locate its HIP runtime")
    return os.path.join(list(spec.submodule_search_locations)[0], "lib")


# The GEMM kernels' global-to-LDS copies write M0 (the LDS address of each
# copy) from inline asm without saving it. That is sound only while the
# compiler leaves M0 unused in those kernels, so the build also compiles the
# 16-bit GEMM unit to device assembly and fails if an instruction outside an
# inline-asm block names M0 or is one of those that read it implicitly.
M0_SOURCE = "nm_gemm_f16.hip"
M0_IMPLICIT = ("global_load_lds", "s_movrel", "v_movrel", "s_sendmsg", "ds_append", "ds_consume", "ds_gws", "ds_ordered")


def check_m0_unused(asm_path):
    """Instructions outside inline asm that name or implicitly use M0 (empty list: sound)."""
    import re
    bad, inside = [], False
    for line in open(asm_path):
        t = line.split(";;")[0].strip() if not line.strip().startswith(";;#ASM") else line.strip()
        if t.startswith(";;#ASMSTART"):
            inside = True
            continue
        if t.startswith(";;#ASMEND"):
            inside = False
            continue
        t = t.split(";")[0].strip()
        if inside or not t or t.startswith(".") or t.endswith(":"):
            continue
        op = t.split()[0]
        if (re.search(r"\bm0\b", t) or op.startswith(M0_IMPLICIT)
                or (op.startswith("buffer_load") and re.search(r"\blds\b", t))):
            bad.append(t)
    return bad


def _m0_check():
    out = os.path.join(BUILD, "m0_check.s")
    cmd = [HIPCC] + CFLAGS + ["--cuda-device-only", "-S", os.path.join(CSRC, M0_SOURCE), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    bad = check_m0_unused(out)
    if bad:
        raise RuntimeError("the compiler uses M0 in the GEMM kernels, which the copy asm overwrites: " +
                           "; ".join(bad[:5]))
    return out


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), msgs))
    if msgs.strip():
        sys.stderr.write(msgs + "\n")
    return obj


def _link(objs, out, soname):
    tl = torch_lib_dir()
    hip_rt = os.path.join(tl, "libamdhip64.so")
    if not os.path.exists(hip_rt):
        raise RuntimeError("torch's HIP runtime not found at " + hip_rt)
    tmp = out + ".tmp"
    cmd = [CLANG, "-shared", "-fPIC", "-o", tmp] + objs + [
        "-L" + tl, "-l:libamdhip64.so", "-Wl,-rpath," + tl, "-Wl,--no-undefined", "-Wl,-soname," + soname]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, out)


def build(verbose=True):
    """Compile every HIP source for gfx950 and link libnmsparse.so and libnmcal.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES) + 2) as ex:
        m0 = ex.submit(_m0_check)
        objs = list(ex.map(_compile, SOURCES + ["nm_calib.hip"]))
        m0.result()
    _link(objs[-1:], CAL_LIB, "libnmcal.so")
    objs = objs[:-1]
    tl = torch_lib_dir()
    hip_rt = os.path.join(tl, "libamdhip64.so")
    if not os.path.exists(hip_rt):
        raise RuntimeError("torch's HIP runtime not found at " + hip_rt)
    tmp = LIB + ".tmp"
    cmd = [CLANG, "-shared", "-fPIC", "-o", tmp] + objs + [
        "-L" + tl, "-l:libamdhip64.so", "-Wl,-rpath," + tl, "-Wl,--no-undefined", "-Wl,-soname,libnmsparse.so"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
