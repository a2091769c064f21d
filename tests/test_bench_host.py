"""Host-side checks of bench.py (no GPU): the one-GPU refusal and which GEMMs
of a workload share a pruned and a compressed weight within one step."""
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from structured_sparse_gemm_nm_amd import inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _gemm(wname):
    """The fields bench.py's step construction reads for one GEMM (shapes only)."""
    w = inputs.WORKLOADS[wname]
    return dict(w=w, host=dict(a=types.SimpleNamespace(shape=inputs.stored_shape_a(w))), dtype=w["dtype"],
                mode="tile" if w.get("tile") else "1d", vrows=max(1, w.get("vector_rows", 0)), N=w["N"], M=w["M"],
                op_a=w.get("op_a", "N"), m=w["m"], k=w["k"])


def _groups(workload):
    gs = [_gemm(wname) for _, wname in bench.WORKLOAD_SETS[workload]]
    pruned = [bench.weight_key(g) for g in gs]
    packed = [bench.weight_key(g) + (g["op_a"], g["m"], g["k"]) for g in gs]
    return len(set(pruned)), len(set(packed))


@pytest.mark.parametrize("workload,pruned,packed", [
    ("x1", 1, 2),          # one W, read forward (op_a = N) and backward (op_a = T): pruned once, compressed twice
    ("c3", 1, 2),
    ("x2", 1, 1),          # the GEMV and the n = 8 product read the same 4:32 weight in the same orientation
    ("c5_4of32", 1, 1),
    ("vw_8of32", 1, 1),
    ("bert", 3, 3),        # three different weights
    ("x3", 4, 4),
    ("c4", 1, 1),
])
def test_shared_weights(workload, pruned, packed):
    assert _groups(workload) == (pruned, packed)


def test_one_d_pruning_keys_on_orientation():
    """A 1-D N:M mask depends on the direction of k, a 4x4 tile mask does not."""
    g = _gemm("c5_4of32_n1")
    t = dict(g, op_a="T")
    assert bench.weight_key(g) != bench.weight_key(t)
    x = _gemm("x1_fwd")
    assert bench.weight_key(x) == bench.weight_key(dict(x, op_a="T"))
