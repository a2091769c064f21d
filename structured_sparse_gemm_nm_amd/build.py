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
    with ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        objs = list(ex.map(_compile, SOURCES + ["nm_calib.hip"]))
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
