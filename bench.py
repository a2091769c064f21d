"""Benchmark: N:M structured-sparse GEMM hot path on one MI355X.

A step is one pass of the whole hot path over one workload's weights and
activations: for each weight, prune (1-D top-N, or the transposable 4x4-tile
2:4 mask) and conformance check once; then, for each orientation the step's
GEMMs read it in, compress, the SpMM (in every B layout the workload names)
and decompress. Weights are re-sparsified every step, as in
runtime-sparsified training where the weights change between steps (the
cuSPARSELt blog: compress again whenever A changes).

Default workload (x1): the training pair at its largest shapes in fp16, W
11008 x 4096 pruned to transposable 2:4, X 8192 x 4096 and dY 8192 x 11008:
the forward Y^T = W X^T (11008 x 8192 x 4096) and the input gradient
dX^T = W^T dY^T (4096 x 8192 x 11008). Other workloads: --workload NAME.

value  = dense-equivalent TFLOP/s of the step's SpMMs (2*m*n*k each) over the
         whole step time (prune/check/compress/decompress included).
Also reported: the SpMM kernels alone, the same-shape dense MFMA GEMM written
in this library (with its fraction of the dense peak), the speed-up, the
roofline of the dominant kernel (measured with HIP events on the launch
stream over the timed region), and the CPU oracle timed on a bounded sample
of the same workload.

Order: W warm-up steps, a per-launch pass (K steps, every SpMM bracketed by
events), then untimed settling steps (at least W, and enough for 60 ms of
continuous work: after an idle gap the GPU's power management runs the next
tens of milliseconds of work slower than steady state), then the K timed steps.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "i8": 5033.0}   # dense matrix peaks (TFLOP/s, TOP/s)

# workload name -> list of (label, inputs.WORKLOADS key) GEMMs making one step
WORKLOAD_SETS = {
    "bert": [("fc1", "c2_fc1"), ("fc2", "c2_fc2"), ("proj", "c2_proj")],
    "c1": [("c1", "c1_fp16_256")],
    "c3": [("fwd", "c3_fwd"), ("bwd", "c3_bwd")],
    "linear": [("fwd", "c3_fwd"), ("dx", "c3_bwd")],
    "c4": [("int8", "c4_int8")],
    "x1": [("fwd", "x1_fwd"), ("bwd", "x1_bwd")],
    "x3": [("qkv", "x3_qkv"), ("proj", "x3_proj"), ("fc1", "x3_fc1"), ("fc2", "x3_fc2")],
    "x2": [("n1", "x2_4of32_n1"), ("n8", "x2_4of32_n8")],
    "c5_4of32": [("n1", "c5_4of32_n1"), ("n8", "c5_4of32_n8"), ("n4096", "c5_4of32_n4096")],
    "c5_8of32": [("n1", "c5_8of32_n1"), ("n8", "c5_8of32_n8"), ("n4096", "c5_8of32_n4096")],
    "vw_4of32": [("n1", "c5vw_4of32_n1"), ("n8", "c5vw_4of32_n8"), ("n4096", "c5vw_4of32_n4096")],
    "vw_8of32": [("n1", "c5vw_8of32_n1"), ("n8", "c5vw_8of32_n8"), ("n4096", "c5vw_8of32_n4096")],
}
WORKLOAD_DESC = {
    "bert": "BERT-Large GEMMs (FC1 4096x1024, FC2 1024x4096, PROJ 1024x1024 weights, 4096 tokens), fp16 2:4, NT+NN",
    "c1": "fp16 2:4, A 256x256, B 256x64, NN",
    "c3": "bf16 transposable 2:4 training pair, W 11008x4096, X 8192x4096, dY 8192x11008, NT",
    "c4": "int8 2:4, 4096^3, int32 C/D, beta=1, NN+NT",
    "linear": "training step of the runtime-sparsified linear layer at the bf16 pair's shapes (W 11008x4096, "
              "8192 tokens): tile prune, check, compress along k and along m, Y = X W^T and dX = dY W on 2:4 "
              "with column-major D, dense dW = dY^T X",
    "x1": "fp16 transposable 2:4 pair at the training shapes: W 11008x4096, X 8192x4096, dY 8192x11008, NT",
    "x2": "fp16 4:32 GEMV and n = 8 beyond the Infinity Cache: A 32768x32768 (compressed 268 MB + 84 MB metadata), NN",
    "x3": "the cuSPARSELt blog's Table 1 shapes: QKV 3072x1024, PROJ 1024x1024, FC1 4096x1024, FC2 1024x4096 "
          "weights, 16384 tokens, fp16 2:4, NT, D column-major as in the blog",
    "c5_4of32": "fp16 4:32, A 4096x4096, B 4096 x {1, 8, 4096}, NN",
    "c5_8of32": "fp16 8:32, A 4096x4096, B 4096 x {1, 8, 4096}, NN",
    "vw_4of32": "fp16 vector-wise 4:32 (16 rows share each group's offsets), A 4096x4096, B 4096 x {1, 8, 4096}, NN",
    "vw_8of32": "fp16 vector-wise 8:32 (16 rows share each group's offsets), A 4096x4096, B 4096 x {1, 8, 4096}, NN",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="x1", choices=sorted(WORKLOAD_SETS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-autotune", action="store_true",
                    help="keep every SpMM plan on its default block tile and no split-k (no timing-based choice)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain %d MiB elementwise copy (y = -x) %d times (for counter calibration)" % (CAL_MIB, CAL_REPS))
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into profiles/traffic_<workload>.md")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR",
                    help="turn a rocprofv3 --pmc run of the matrix-core counters into profiles/mfma_<workload>.md")
    ap.add_argument("--summarize-units", nargs="+", metavar="PMC_DIR",
                    help="turn rocprofv3 --pmc runs of memory-unit counters (with GRBM_GUI_ACTIVE) into "
                         "profiles/units_<workload>.md: each counter per CU and clock, per kernel")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="turn a rocprofv3 --kernel-trace --stats run into a profiles/ summary")
    ap.add_argument("--command", default="", help="the command that produced the runs (recorded in summaries)")
    ap.add_argument("--bench-log", default=None, help="stdout of the traced bench run (its JSON line is compared)")
    return ap.parse_args()


CAL_MIB, CAL_REPS = 1024, 3
SETTLE_MS, SETTLE_MAX_STEPS = 60.0, 2000   # continuous untimed work directly before the timed region
PROFILES = os.path.join(ROOT, "profiles")


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence:
    recording it writes a timestamp without the system-scope cache writeback
    and invalidation a default event performs at every record (which costs a
    few microseconds on the queue and leaves the next kernel with cold
    caches). It is read only after a device synchronisation, which orders it
    with the work it brackets."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            import torch
            hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            TimingEvent._hip = hip
        self._c = ctypes
        self.h = ctypes.c_void_p()
        st = self._hip.hipEventCreateWithFlags(ctypes.byref(self.h), self.DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError("hipEventCreateWithFlags failed (%d)" % st)

    def record(self, stream):
        st = self._hip.hipEventRecord(self.h, self._c.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % st)

    def elapsed_time(self, end):
        ms = self._c.c_float()
        st = self._hip.hipEventElapsedTime(self._c.byref(ms), self.h, end.h)
        if st != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % st)
        return ms.value


def source_fingerprint():
    """sha256 over the library's kernel and host sources: counters taken on other sources do not apply."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "structured_sparse_gemm_nm_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.summarize_trace:
        summarize_trace(args)
        return
    if args.summarize_mfma:
        summarize_mfma(args)
        return
    if args.summarize_units:
        summarize_units(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this library's hot path is single-GPU "
              "(sharding is described in DESIGN.md, not implemented); got --gpus %d" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import structured_sparse_gemm_nm_amd as nm
    from structured_sparse_gemm_nm_amd import inputs

    torch.cuda.set_device(0)
    dev = "cuda"
    stream = torch.cuda.current_stream()

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    # ---------------------------------------------------------------- set-up (not timed)
    gemms = []
    for label, wname in WORKLOAD_SETS[args.workload]:
        w = inputs.WORKLOADS[wname]
        dtype, N, M, m, n, k = w["dtype"], w["N"], w["M"], w["m"], w["n"], w["k"]
        op_a = w.get("op_a", "N")
        layouts = ["T", "N"] if args.workload in ("bert", "c4") else [w.get("op_b", "N")]
        a, b_first, c = inputs.workload_inputs(wname, layouts[0])
        bs = {layouts[0]: b_first}
        for ob in layouts[1:]:
            bs[ob] = inputs.workload_inputs(wname, ob)[1]
        mode = "tile" if w.get("tile") else "1d"
        g = dict(label=label, name=wname, w=w, dtype=dtype, m=m, n=n, k=k, N=N, M=M, mode=mode, op_a=op_a)
        order = "col" if args.workload == "linear" else w.get("order_cd", "row")
        vr = w.get("vector_rows", 0)
        g["vrows"] = max(1, vr)
        g["plan"] = nm.nm_plan_init(m, n, k, N, M, op_a=op_a, op_b=layouts[0], dtype=dtype, order_cd=order,
                                    vector_rows=vr)
        g["plans"] = {ob: nm.nm_plan_init(m, n, k, N, M, op_a=op_a, op_b=ob, dtype=dtype, order_cd=order,
                                          vector_rows=vr) for ob in layouts}
        g["A"] = to_dev(a)
        g["Ap"] = torch.empty_like(g["A"])
        g["Ad"] = torch.empty_like(g["A"])
        g["vals"] = g["plan"].empty_values()
        g["meta"] = g["plan"].empty_meta()
        g["cnt"] = torch.zeros(1, dtype=torch.int32, device=dev)
        g["B"] = {ob: to_dev(bs[ob]) for ob in layouts}
        g["C"] = to_dev(c) if c is not None else None
        odt = torch.int32 if dtype == "i8" else torch.float16 if dtype == "f16" else torch.bfloat16
        dshape = (n, m) if order == "col" else (m, n)
        g["D"] = {ob: torch.empty(dshape, dtype=odt, device=dev) for ob in layouts}
        g["layouts"] = layouts
        g["host"] = dict(a=a, b=bs, c=c)
        gemms.append(g)

    # Algorithm selection, once per plan and outside every timed region (the
    # blog's plan-time choice): each SpMM plan tries every block tile and split-k
    # in {1, 2, 4} on the workload's own operands and keeps the fastest; a
    # split-k choice gets its workspace here, allocated by the caller.
    tuned = {}
    if not args.no_autotune and args.workload != "linear":
        from structured_sparse_gemm_nm_amd.tuning import autotune_spmm
        for g in gemms:
            nm.nm_prune(g["plan"], g["A"], g["Ap"], g["mode"])
            nm.nm_compress(g["plan"], g["Ap"], g["vals"], g["meta"])
            for ob in g["layouts"]:
                pl = g["plans"][ob]
                if pl.kernel_name != "spmm_smfmac_2of4":
                    continue
                # every setting keeps its best of four interleaved passes (the
                # first brings the clocks up)
                autotune_spmm(pl, g["w"]["alpha"], g["vals"], g["meta"], g["B"][ob], g["w"]["beta"], g["C"],
                              g["D"][ob], reps=10, warmup=3, split_ks=(1, 2, 4), rounds=4)
                tuned[(g["label"], ob)] = (nm.nm_plan_get_algorithm(pl), nm.nm_plan_get_split_k(pl)[1])
        torch.cuda.synchronize()
    for g in gemms:
        g["WS"] = {ob: g["plans"][ob].empty_workspace() for ob in g["layouts"]}

    # The step calls the C ABI with arguments marshalled once, so that the host
    # enqueues well ahead of the GPU and the events around a SpMM launch
    # (recorded on the stream the kernels run on) time the kernel, not host gaps.
    import ctypes
    L = nm.lib()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    calls = []            # (callable, args, spmm key or None)
    # A weight that several GEMMs of the step read (the training pair's W, read
    # as op_a = N forward and op_a = T backward) is pruned and checked once and
    # compressed once per orientation it is read in, as a training step does.
    pruned, packed = {}, {}
    for g in gemms:
        h = g["plan"].handle
        mode = nm.MODES[g["mode"]]
        g["_ab"] = (ctypes.c_float(g["w"]["alpha"]), ctypes.c_float(g["w"]["beta"]))
        src = pruned.setdefault(weight_key(g), g)
        if src is g:
            calls.append((L.nm_prune, (h, P(g["A"]), P(g["Ap"]), mode, None, sp), None))
            calls.append((L.nm_prune_check, (h, P(g["Ap"]), mode, P(g["cnt"]), sp), None))
        else:
            g["Ap"] = src["Ap"]
        csrc = packed.setdefault(weight_key(g) + (g["op_a"], g["m"], g["k"]), g)
        if csrc is g:
            calls.append((L.nm_compress, (h, P(g["Ap"]), P(g["vals"]), P(g["meta"]), sp), None))
        else:
            g["vals"], g["meta"] = csrc["vals"], csrc["meta"]
        for ob in g["layouts"]:
            calls.append((L.nm_spmm, (g["plans"][ob].handle, ctypes.byref(g["_ab"][0]), P(g["vals"]), P(g["meta"]),
                                      P(g["B"][ob]), ctypes.byref(g["_ab"][1]), P(g["C"]), P(g["D"][ob]),
                                      P(g["WS"][ob]), sp),
                          (g["label"], ob)))
        if csrc is g:
            calls.append((L.nm_decompress, (h, P(g["vals"]), P(g["meta"]), P(g["Ad"]), sp), None))

    if args.workload == "linear":
        # the layer's step as the C-ABI calls SemiStructuredSparseLinear makes:
        # one weight, pruned and checked once, compressed along k (forward) and
        # along m (input gradient); the weight gradient on the dense product
        gf, gx = gemms
        gx["Ap"] = gf["Ap"]                                  # the same pruned weight, read as op_a = T
        tok, out_f, in_f = gf["n"], gf["m"], gf["k"]
        plan_dw = nm.nm_plan_init(out_f, in_f, tok, 2, 4, op_a="T", op_b="N", dtype=gf["dtype"])
        gf["dW"] = torch.empty((out_f, in_f), dtype=torch.bfloat16, device=dev)
        one, zero = ctypes.c_float(1.0), ctypes.c_float(0.0)
        tile = nm.MODES["tile"]
        calls = [
            (L.nm_prune, (gf["plan"].handle, P(gf["A"]), P(gf["Ap"]), tile, None, sp), None),
            (L.nm_prune_check, (gf["plan"].handle, P(gf["Ap"]), tile, P(gf["cnt"]), sp), None),
            (L.nm_compress, (gf["plan"].handle, P(gf["Ap"]), P(gf["vals"]), P(gf["meta"]), sp), None),
            (L.nm_compress, (gx["plan"].handle, P(gf["Ap"]), P(gx["vals"]), P(gx["meta"]), sp), None),
            (L.nm_spmm, (gf["plans"]["T"].handle, ctypes.byref(one), P(gf["vals"]), P(gf["meta"]), P(gf["B"]["T"]),
                         ctypes.byref(zero), None, P(gf["D"]["T"]), None, sp), ("fwd", "T")),
            (L.nm_spmm, (gx["plans"]["T"].handle, ctypes.byref(one), P(gx["vals"]), P(gx["meta"]), P(gx["B"]["T"]),
                         ctypes.byref(zero), None, P(gx["D"]["T"]), None, sp), ("dx", "T")),
            (L.nm_dense_gemm, (plan_dw.handle, ctypes.byref(one), P(gx["B"]["T"]), P(gf["B"]["T"]), ctypes.byref(zero),
                               None, P(gf["dW"]), sp), None),
        ]
        args.no_cpu_baseline = True                          # the oracle baseline is quoted on the default workload

    n_spmm = sum(1 for c in calls if c[2] is not None)
    spmm_kernel = {(g["label"], ob): g["plans"][ob].spmm_kernel for g in gemms for ob in g["layouts"]}
    # events (timing-only HIP events, see TimingEvent) are created before any timed pass
    pool = [(TimingEvent(), TimingEvent()) for _ in range(n_spmm * args.steps)]
    empty_pool = [(TimingEvent(), TimingEvent()) for _ in range(args.steps)]

    def step(ev=None, only=None, empty=None):
        """One pass of the hot path. With `ev`, the SpMM launches whose device
        kernel is in `only` (all when None) are bracketed by an event pair on the
        launch stream; with `empty`, an event pair around nothing is recorded first
        (the events' own cost on the queue)."""
        if empty is not None:
            e0, e1 = empty_pool[len(empty)]
            e0.record(stream)
            e1.record(stream)
            empty.append((e0, e1))
        for fn, a, key in calls:
            if ev is not None and key is not None and (only is None or spmm_kernel[key] in only):
                e0, e1 = pool[len(ev)]
                e0.record(stream)
                st = fn(*a)
                e1.record(stream)
                ev.append((key, e0, e1))
            else:
                st = fn(*a)
            if st != 0:
                raise nm.NmError(st, L.nm_last_error().decode())

    if args.copy_calibration:
        src = torch.ones(CAL_MIB << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(CAL_REPS):
            torch.neg(src, out=dst)           # reads and writes CAL_MIB MiB with 16-byte vector accesses
        torch.cuda.synchronize()
        del src, dst

    # W untimed warm-up steps precede the per-launch pass. After an idle gap
    # (host-side set-up, the per-launch pass's bookkeeping) the GPU's power
    # management runs the following tens of milliseconds of work up to 30%
    # slower than steady state, so the timed region is preceded by untimed
    # settling steps: at least W, and enough for SETTLE_MS of continuous work,
    # with no host work between them and the timed region.
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    viol = [int(g["cnt"].item()) for g in gemms]
    assert all(v == 0 for v in viol), "prune check failed: %s" % viol

    # Per-launch pass (not the timed region): every SpMM launch bracketed by
    # events, to time each GEMM and find the device kernel with the most time.
    all_ev, empty = [], []
    t_pl = time.perf_counter()
    for _ in range(args.steps):
        step(all_ev, None, empty)
    torch.cuda.synchronize()
    pass_ms_per_step = (time.perf_counter() - t_pl) * 1e3 / args.steps
    event_ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in empty]))
    per = {}
    for key, e0, e1 in all_ev:
        per.setdefault(key, []).append(e0.elapsed_time(e1))
    spmm_ms = {k: max(float(np.median(v)) - event_ms, 1e-6) for k, v in per.items()}   # events' cost removed
    kern_ms = {}
    for key, t in spmm_ms.items():
        kern_ms[spmm_kernel[key]] = kern_ms.get(spmm_kernel[key], 0.0) + t
    dom_key = max(kern_ms, key=kern_ms.get)

    # Timed region: K steps; only the dominant kernel's launches carry events
    # (each event pair adds its own few microseconds to the queue).
    events = []
    settle_steps = min(max(args.warmup, math.ceil(SETTLE_MS / max(pass_ms_per_step, 1e-3))), SETTLE_MAX_STEPS)
    for _ in range(settle_steps):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(events, {dom_key})
    t_enq = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    host_ms_per_step = (t_enq - t0) * 1e3 / args.steps
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    def flops_dense_eq(g):
        return 2.0 * g["m"] * g["n"] * g["k"]

    step_flops = sum(flops_dense_eq(g) * len(g["layouts"]) for g in gemms)
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    spmm_total_ms = sum(spmm_ms[(g["label"], ob)] for g in gemms for ob in g["layouts"])
    spmm_only_tflops = step_flops / (spmm_total_ms * 1e-3) / 1e12

    # Roofline of the dominant kernel (the device kernel, as the profiler names
    # it, with the most SpMM time). Its launches in the timed region may cover
    # several GEMM shapes (the same kernel serves several weights): each launch
    # is priced with the work of its own shape, and the kernel's figure is the
    # sum of that work over the sum of the launch times (a mean, so that it
    # compares with the profiler's average duration over the same launches).
    gemm_of = {g["label"]: g for g in gemms}
    by_label = {}
    for key, e0, e1 in events:
        by_label.setdefault(key, []).append(max(e0.elapsed_time(e1) - event_ms, 1e-6))
    dtype_dom = gemm_of[next(iter(by_label))[0]]["dtype"]
    kname = gemm_of[next(iter(by_label))[0]]["plans"][next(iter(by_label))[1]].kernel_name
    peak_f = PEAK_TFLOPS[dtype_dom]
    ridge = peak_f * 1e12 / (HBM_PEAK_GBS * 1e9)

    def kernel_work(g):
        """(flops per launch as this kernel executes them, algorithmic bytes per launch)."""
        keep = g["N"] / g["M"]
        if kname == "spmm_gather_mfma":
            # element-wise N:M: each k-step's kept values are expanded into a dense
            # tile and run on the dense matrix instructions, so the executed
            # matrix work is the dense product's
            return 2.0 * g["m"] * g["n"] * g["k"], spmm_bytes(g)
        return 2.0 * g["m"] * g["n"] * g["k"] * keep, spmm_bytes(g)    # multiply-adds of the kept values

    tot_ms = tot_flops = tot_bytes = 0.0
    n_launch = 0
    per_shape = []
    for key, ts in sorted(by_label.items()):
        g = gemm_of[key[0]]
        f, by = kernel_work(g)
        tot_ms += sum(ts); tot_flops += f * len(ts); tot_bytes += by * len(ts); n_launch += len(ts)
        mean = float(np.mean(ts))
        per_shape.append({"gemm": key[0], "layout": "N" + key[1], "m": g["m"], "n": g["n"], "k": g["k"],
                          "launches": len(ts), "mean_ms": round(mean, 5),
                          "tflops": round(f / (mean * 1e-3) / 1e12, 2), "gbs": round(by / (mean * 1e-3) / 1e9, 1)})
    avg_ms = tot_ms / n_launch
    avg_bytes = tot_bytes / n_launch
    ai = tot_flops / tot_bytes
    if kname == "spmm_skinny" or (kname == "spmm_smfmac_2of4" and ai < ridge):
        achieved = tot_bytes / (tot_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        achieved = tot_flops / (tot_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_f, "unit": "TFLOP/s",
                    "frac": round(achieved / peak_f, 4), "traffic": None}
    roofline["kernel"] = dom_key
    roofline["work_counted"] = ("dense multiply-adds of the expanded tile (2 m n k), executed on the dense matrix "
                                "instructions" if kname == "spmm_gather_mfma" else
                                "multiply-adds of the kept values (2 m n k N/M), executed on the dense matrix "
                                "instructions over the gathered rows of B, against the dense matrix peak"
                                if kname == "spmm_vw_mfma" else
                                "multiply-adds of the kept values (2 m n k N/M) against the dense matrix peak, the same "
                                "ratio as dense-equivalent flops against the 2:4 peak" if roofline["bound"] == "mfma"
                                else "compressed A + metadata + B + D (+ C) bytes per launch")
    roofline["per_shape"] = per_shape
    # operands of one launch against the 256 MB Infinity Cache: below it, repeated
    # steps can find them there (cache-warm); above it, every launch streams from HBM
    roofline["working_set_mb"] = round(avg_bytes / 1e6, 1)
    roofline["cache"] = "warm (below the 256 MB Infinity Cache)" if avg_bytes < 256e6 else "cold (beyond the 256 MB Infinity Cache)"
    roofline["launch_ms"] = round(avg_ms, 5)
    roofline["launch_ms_method"] = ("mean over the timed steps of the HIP-event interval around each launch of this "
                                    "kernel (the only events in the timed region; timing-only events without the "
                                    "system-scope fence), less the median interval of an empty "
                                    "event pair (%.5f ms); achieved = the launches' summed work / their summed time"
                                    % event_ms)
    roofline["launches_per_step"] = n_launch // args.steps
    traffic = load_traffic(args.workload, dom_key)
    if traffic is not None:
        roofline["traffic"] = traffic["bytes_per_launch"]
        roofline["traffic_over_algorithmic"] = round(traffic["bytes_per_launch"] / avg_bytes, 3)
        roofline["traffic_note"] = traffic["note"]

    # dense comparator, same shapes, same B layouts. Dense A is always given row
    # by row of op(A) (op_a = N): for a backward operand (op_a = T) that means
    # the pruned weight transposed once outside the timing, the faster layout
    # for the dense kernels (their op_a = T path stages A through registers), so
    # the comparison is against the better dense formulation of the product.
    def best_pass_ms(f, passes=3):
        """ms per call of f: the best of `passes` timed passes (each after its own
        warm-up calls), so that the clock drop after an idle gap does not decide."""
        best = None
        for _ in range(passes):
            for _ in range(max(2, args.warmup)):
                f()
            e0 = torch.cuda.Event(enable_timing=True); e1 = torch.cuda.Event(enable_timing=True)
            reps = max(5, args.steps)
            e0.record(stream)
            for _ in range(reps):
                f()
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / reps
            best = t if best is None else min(best, t)
        return best

    dense = {}
    if not args.no_dense:
        for g in gemms:
            a_dense = g["Ap"]
            if g["op_a"] == "T":
                a_dense = g["Ap"].t().contiguous()
            for ob in g["layouts"]:
                # its own plan, every block tile timed, the fastest kept (the
                # comparator gets the same plan-time choice as the SpMM)
                pl = nm.nm_plan_init(g["m"], g["n"], g["k"], g["N"], g["M"], op_a="N", op_b=ob, dtype=g["dtype"],
                                     order_cd=g["w"].get("order_cd", "row"))
                f = lambda: nm.nm_dense_gemm(pl, g["w"]["alpha"], a_dense, g["B"][ob], g["w"]["beta"], g["C"], g["D"][ob])
                best = None
                for alg in range(nm.NM_ALG_COUNT if not args.no_autotune else 1):
                    nm.nm_plan_set_algorithm(pl, alg)
                    t = best_pass_ms(f)
                    best = t if best is None else min(best, t)
                dense[(g["label"], ob)] = best
    # vendor dense GEMM (torch.matmul, hipBLASLt on this platform) on the same
    # pruned A and B, as a reference for the in-library dense comparator: the
    # plain product op(A) op(B) in the operand type (no alpha, beta or C), int8
    # through torch._int_mm where the build supports it
    vendor = {}
    if not args.no_dense:
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16}
        for g in gemms:
            a_dense = g["Ap"] if g["op_a"] == "N" else g["Ap"].t().contiguous()
            for ob in g["layouts"]:
                bt = g["B"][ob]
                try:
                    if g["dtype"] == "i8":
                        a8 = a_dense.view(torch.int8)
                        b8 = (bt.view(torch.int8).t() if ob == "T" else bt.view(torch.int8))
                        f = lambda: torch._int_mm(a8, b8)
                    else:
                        av = a_dense.view(tdt[g["dtype"]])
                        bv = bt.view(tdt[g["dtype"]])
                        f = (lambda: torch.matmul(av, bv.t())) if ob == "T" else (lambda: torch.matmul(av, bv))
                    vendor[(g["label"], ob)] = best_pass_ms(f)
                except (RuntimeError, NotImplementedError):
                    pass
    per_gemm = []
    for g in gemms:
        for ob in g["layouts"]:
            key = (g["label"], ob)
            t_s = spmm_ms[key]
            row = {"gemm": g["label"], "layout": "N" + ob, "m": g["m"], "n": g["n"], "k": g["k"],
                   "kernel": g["plans"][ob].kernel_name, "algorithm": nm.nm_plan_get_algorithm(g["plans"][ob]),
                   "split_k": nm.nm_plan_get_split_k(g["plans"][ob])[1], "spmm_ms": round(t_s, 5),
                   "spmm_tflops": round(flops_dense_eq(g) / (t_s * 1e-3) / 1e12, 2)}
            row["spmm_frac_of_sparse_peak"] = round(row["spmm_tflops"] / (2 * PEAK_TFLOPS[g["dtype"]]), 4)
            if key in dense:
                row["dense_ms"] = round(dense[key], 5)
                row["dense_tflops"] = round(flops_dense_eq(g) / (dense[key] * 1e-3) / 1e12, 2)
                row["dense_frac_of_dense_peak"] = round(row["dense_tflops"] / PEAK_TFLOPS[g["dtype"]], 4)
                row["speedup"] = round(dense[key] / t_s, 3)
            if key in vendor:
                row["vendor_dense_ms"] = round(vendor[key], 5)
                row["vendor_dense_tflops"] = round(flops_dense_eq(g) / (vendor[key] * 1e-3) / 1e12, 2)
                row["speedup_vs_vendor_dense"] = round(vendor[key] / t_s, 3)
            per_gemm.append(row)
    speedup = None
    if dense:
        speedup = round(sum(dense.values()) / spmm_total_ms, 3)
    speedup_vendor = None
    if vendor and len(vendor) == len(spmm_ms):
        speedup_vendor = round(sum(vendor.values()) / spmm_total_ms, 3)

    # measured achievable peaks (calibration loops, outside the timed region)
    cal = calibrate(torch, stream, dtype_dom)
    if cal is not None:
        roofline["achievable"] = cal
        if roofline["bound"] == "mfma" and cal["sparse_matrix"] > 0:
            # the kept multiply-adds of the sparse instruction run at half its dense-equivalent rate
            roofline["frac_of_achievable"] = round(roofline["achieved"] / (cal["sparse_matrix"] / 2), 4)
        elif roofline["bound"] == "hbm" and cal["copy_gbs"] > 0:
            roofline["frac_of_achievable"] = round(roofline["achieved"] / cal["copy_gbs"], 4)

    # CPU oracle on one step of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(gemms)

    dtype = gemms[0]["dtype"]
    out = {
        "metric": "dense-equivalent TFLOP/s of 2:4 SpMM (fp16, bf16, int8) + speedup vs dense GEMM",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_per_step, 4),
        "host_enqueue_ms_per_step": round(host_ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f16": "f16", "bf16": "bf16", "i8": "i8"}[dtype],
        "data": "synthetic",
        "config": {"workload": WORKLOAD_DESC[args.workload], "pattern": "%d:%d" % (gemms[0]["N"], gemms[0]["M"]),
                   "step": "prune+check per weight; compress+spmm(per layout)+decompress per orientation it is read in"},
        "spmm_only_tflops": round(spmm_only_tflops, 2),
        "speedup_vs_dense": speedup,
        "speedup_vs_vendor_dense": speedup_vendor,
        "per_gemm": per_gemm,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def calibrate(torch, stream, dtype):
    """Achievable peaks on this GPU: the 2:4 and dense matrix instructions with no
    memory traffic, and a streaming copy (libnmcal.so, built with the library)."""
    import ctypes
    path = os.path.join(ROOT, "structured_sparse_gemm_nm_amd", "libnmcal.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.nmcal_matrix_tflops.restype = ctypes.c_double
    L.nmcal_matrix_tflops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p]
    L.nmcal_copy_gbs.restype = ctypes.c_double
    L.nmcal_copy_gbs.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    sp = ctypes.c_void_p(stream.cuda_stream)
    blocks, iters = 1024, 2000
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    i8 = 1 if dtype == "i8" else 0
    sparse = L.nmcal_matrix_tflops(1, i8, ctypes.c_void_p(out.data_ptr()), blocks, iters, sp)
    dense = L.nmcal_matrix_tflops(0, i8, ctypes.c_void_p(out.data_ptr()), blocks, iters, sp)
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    copy = L.nmcal_copy_gbs(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes, sp)
    del src, dst, out
    return {"sparse_matrix": round(sparse, 1), "dense_matrix": round(dense, 1),
            "unit": "TFLOP/s" if not i8 else "TOP/s", "copy_gbs": round(copy, 1),
            "method": "%s matrix instructions in a loop with no memory traffic (%d blocks x 4 waves, %d x 8 "
                      "instructions; sparse figure dense-equivalent), and a 1 GiB streaming copy (read + write "
                      "bytes)" % ("int8" if i8 else "fp16", blocks, iters)}


def load_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, if taken on these sources."""
    path = os.path.join(PROFILES, "traffic_%s.md" % workload)
    if not os.path.exists(path):
        return None
    rec = None
    for line in open(path):
        if line.startswith("record: "):
            rec = json.loads(line[len("record: "):])
    if rec is None or rec.get("sources") != source_fingerprint() or kernel not in rec["kernels"]:
        return None
    k = rec["kernels"][kernel]
    b = k["fetch_kib"] * 1024 * rec["fetch_scale"] + k["write_kib"] * 1024 * rec["write_scale"]
    return {"bytes_per_launch": round(b), "note": "FETCH_SIZE + WRITE_SIZE per dispatch (%d dispatches), scaled by "
            "a %d MiB elementwise copy's readings (x%.3f, x%.3f); %s" % (k["dispatches"], CAL_MIB, rec["fetch_scale"],
                                                             rec["write_scale"], os.path.relpath(path, ROOT))}


def _read_counter_csv(d, counter):
    """{kernel name: [value per dispatch]} from a rocprofv3 --pmc csv output directory."""
    import csv
    import glob
    out = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") != counter:
                continue
            did = int(r.get("Dispatch_Id", 0))
            out.setdefault(r["Kernel_Name"], {}).setdefault(did, 0.0)
            out[r["Kernel_Name"]][did] += float(r["Counter_Value"])
    return {k: [v[d] for d in sorted(v)] for k, v in out.items()}     # in dispatch order


def _dominant_from_log(bench_log):
    """(dominant kernel name, its launches in the timed region) from a bench run's stdout, or (None, 0)."""
    if not bench_log:
        return None, 0
    bl = json.loads([l for l in open(bench_log) if l.startswith("{")][-1])
    return bl["roofline"]["kernel"], bl["roofline"]["launches_per_step"] * bl["steps"]


def summarize_counters(args):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of every kernel, with the copy calibration."""
    fetch = _read_counter_csv(args.summarize_counters[0], "FETCH_SIZE")
    write = _read_counter_csv(args.summarize_counters[1], "WRITE_SIZE")
    cal_bytes = CAL_MIB * 1048576.0

    def copy_kernel(tab):
        cands = [k for k, v in tab.items() if "neg" in k.lower() and len(v) >= CAL_REPS]
        if not cands:
            raise SystemExit("no calibration copy with %d dispatches in the counter runs (run with --copy-calibration)" % CAL_REPS)
        return max(cands, key=lambda k: np.median(tab[k]))
    ck = copy_kernel(fetch)
    f_scale = cal_bytes / (np.median(fetch[ck]) * 1024)
    w_scale = cal_bytes / (np.median(write[copy_kernel(write)]) * 1024)
    # the bench line of the fetch run names the dominant kernel; its timed launches are
    # its last ones in the run (autotuning before them also runs split-k variants of
    # the same kernel, whose partial-sum planes would inflate an average over all)
    dom, n_timed = _dominant_from_log(args.bench_log)
    kernels = {}
    for k in fetch:
        if k in write and "nm::" in k:
            fv, wv = fetch[k], write[k]
            if k == dom and len(fv) >= n_timed and len(wv) >= n_timed:
                fv, wv = fv[-n_timed:], wv[-n_timed:]
            kernels[k] = {"fetch_kib": round(float(np.mean(fv)), 1), "write_kib": round(float(np.mean(wv)), 1),
                          "dispatches": len(fv), "timed_only": k == dom}
    rec = {"workload": args.workload, "sources": source_fingerprint(), "fetch_scale": round(float(f_scale), 4),
           "write_scale": round(float(w_scale), 4), "copy_kernel": ck[:100], "kernels": kernels}
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, "traffic_%s.md" % args.workload)
    with open(path, "w") as fh:
        fh.write("# HBM traffic per dispatch: %s\n\n" % WORKLOAD_DESC[args.workload])
        fh.write("Commands (each a separate rocprofv3 run of the same bench command):\n\n")
        for line in args.command.split(" ;; "):
            fh.write("    %s\n" % line)
        fh.write("\nCalibration: a plain %d MiB elementwise copy y = -x (`%s`) read FETCH_SIZE %.0f KiB and WRITE_SIZE %.0f KiB "
                 "per dispatch (median of %d); scale factors %.4f (fetch) and %.4f (write).\n\n"
                 % (CAL_MIB, ck[:80], np.median(fetch[ck]), np.median(write[copy_kernel(write)]), CAL_REPS, f_scale, w_scale))
        fh.write("| kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | scaled MB/dispatch |\n|---|---|---|---|---|\n")
        for k, v in sorted(kernels.items(), key=lambda kv: -kv[1]["fetch_kib"]):
            mb = (v["fetch_kib"] * f_scale + v["write_kib"] * w_scale) * 1024 / 1e6
            fh.write("| `%s` | %d | %.1f | %.1f | %.2f |\n" % (k, v["dispatches"], v["fetch_kib"], v["write_kib"], mb))
        if dom:
            fh.write("\nThe dominant kernel of the bench line (`%s`) is averaged over its %d timed launches only (its "
                     "last dispatches of the run); every other kernel over all its dispatches.\n" % (dom, n_timed))
        fh.write("\nSource fingerprint %s: bench.py reports these figures only while the library sources match.\n\n"
                 % rec["sources"])
        fh.write("record: %s\n" % json.dumps(rec))
    print("wrote", path)


# Matrix-core rate per clock of the whole GPU at the datasheet peaks (2516.6 dense
# fp16/bf16 TFLOP/s at 2.4 GHz): MOPS counters count 512 flops each (dense
# equivalent for the 2:4 instructions), so 2048 MOPS/clock dense, 4096 sparse.
NOMINAL_MOPS_PER_CLK = {"dense": 2048.0, "sparse": 4096.0}
SPARSE_PEAK_F16 = 2 * PEAK_TFLOPS["f16"]          # 2:4 dense-equivalent datasheet figure
N_XCD, N_SIMD = 8, 1024


def summarize_mfma(args):
    """Matrix-core use per kernel from one rocprofv3 --pmc run of SQ_INSTS_VALU_MFMA_MOPS_<type>,
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE (the bench's calibration loops run in the same process)."""
    import csv
    import glob
    vals, dur = {}, {}
    for f in glob.glob(os.path.join(args.summarize_mfma, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            k = r["Kernel_Name"]
            key = (r["Dispatch_Id"], r["Counter_Name"])
            vals.setdefault(k, {}).setdefault(key, 0.0)
            vals[k][key] += float(r["Counter_Value"])
            dur.setdefault(k, {})[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    if not vals:
        raise SystemExit("no counter_collection.csv under %s" % args.summarize_mfma)
    dom, n_timed = _dominant_from_log(args.bench_log)
    rows = []
    for k, d in vals.items():
        keep = None
        if k == dom:                      # its timed launches: its last dispatches of the run
            ids = sorted({int(disp) for disp, _ in d}, key=int)
            keep = set(str(i) for i in ids[-n_timed:]) if len(ids) >= n_timed else None
            if keep is not None:
                dur[k] = {i: t for i, t in dur[k].items() if i in keep}
        per = {}
        for (disp, cname), v in d.items():
            if keep is not None and disp not in keep:
                continue
            per.setdefault(cname, []).append(v)
        mops_name = sorted((c for c in per if c.startswith("SQ_INSTS_VALU_MFMA_MOPS_")),
                           key=lambda c: -float(np.mean(per[c])))          # the type this kernel runs
        if not mops_name or "GRBM_GUI_ACTIVE" not in per:
            continue
        mops = float(np.mean(per[mops_name[0]]))
        if mops <= 0:
            continue
        cyc = float(np.mean(per["GRBM_GUI_ACTIVE"])) / N_XCD          # GRBM counts once per XCD
        busy = float(np.mean(per.get("SQ_VALU_MFMA_BUSY_CYCLES", [0.0])))
        sec = float(np.mean(list(dur[k].values())))
        scale = 2.0 if mops_name[0].endswith("_I8") else 1.0     # int8 matrix rate per clock is twice fp16's
        rows.append(dict(kernel=k, dispatches=len(per["GRBM_GUI_ACTIVE"]), us=sec * 1e6, mops=mops, cycles=cyc,
                         ghz=cyc / sec / 1e9, tflops=mops * 512 / sec / 1e12, mops_clk=mops / cyc / scale,
                         busy=busy / (cyc * N_SIMD), counter=mops_name[0], scale=scale))
    rows.sort(key=lambda r: -r["us"] * r["dispatches"])
    loops = {("sparse" if "<true" in r["kernel"] else "dense"): r for r in rows if "matrix_loop" in r["kernel"]}
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, "mfma_%s.md" % args.workload)
    with open(path, "w") as fh:
        fh.write("# Matrix-core use: %s\n\nCommand:\n\n    %s\n\n" % (WORKLOAD_DESC[args.workload], args.command))
        fh.write("Counters: %s. " % ", ".join(sorted(set(r["counter"] for r in rows))))
        fh.write("Columns: dense-equivalent TFLOP/s (TOP/s for int8) = MOPS x 512 / dispatch time; clock = GRBM_GUI_ACTIVE / %d XCDs "
                 "/ dispatch time; MOPS/clk (halved for int8, whose datasheet rate is twice fp16's) against the datasheet "
                 "rate per clock (%d dense, %d sparse for the whole GPU); busy = SQ_VALU_MFMA_BUSY_CYCLES / (%d SIMDs x clocks). The `matrix_loop` rows are the "
                 "bench's calibration loops (matrix instructions only, no memory traffic): the achievable rate.\n\n"
                 % (N_XCD, NOMINAL_MOPS_PER_CLK["dense"], NOMINAL_MOPS_PER_CLK["sparse"], N_SIMD))
        fh.write("For dispatches of a few tens of microseconds GRBM_GUI_ACTIVE also counts the dispatch's own "
                 "overhead (the clock column then reads above the real clock), so the per-clock columns understate "
                 "those kernels; `of sparse peak` (dense-equivalent TFLOP/s / %.1f) uses time only.\n\n" % SPARSE_PEAK_F16)
        fh.write("| kernel | dispatches | us | dense-eq TFLOP/s | of sparse peak | clock GHz | MOPS/clk | of dense rate "
                 "| of sparse rate | of sparse loop | MFMA busy |\n|---|---|---|---|---|---|---|---|---|---|---|\n")
        if dom:
            fh.write("The dominant kernel of the bench line (`%s`) is averaged over its %d timed launches only (its last "
                     "dispatches of the run; autotuning runs other splits of it first); every other kernel over all "
                     "its dispatches.\n\n" % (dom, n_timed))
        for r in rows:
            sl = loops.get("sparse")
            fh.write("| `%s` | %d | %.1f | %.1f | %.3f | %.2f | %.0f | %.3f | %.3f | %s | %.3f |\n" % (
                r["kernel"][:90], r["dispatches"], r["us"], r["tflops"], r["tflops"] / (SPARSE_PEAK_F16 * r["scale"]), r["ghz"], r["mops_clk"],
                r["mops_clk"] / NOMINAL_MOPS_PER_CLK["dense"], r["mops_clk"] / NOMINAL_MOPS_PER_CLK["sparse"],
                "%.3f" % (r["mops_clk"] / sl["mops_clk"]) if sl else "n/a", r["busy"]))
    print("wrote", path)


def summarize_units(args):
    """Memory-unit counters per kernel as a fraction of CU clocks (counter / (clocks x 256 CUs), clocks =
    GRBM_GUI_ACTIVE / 8 XCDs of the same pass), one column per counter, from one or more --pmc passes."""
    import csv
    import glob
    cols, table = [], {}
    for d in args.summarize_units:
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                key = (r["Kernel_Name"], r["Dispatch_Id"])
                vals.setdefault(key, {}).setdefault(r["Counter_Name"], 0.0)
                vals[key][r["Counter_Name"]] += float(r["Counter_Value"])
        per = {}
        for (k, _), cv in vals.items():
            if "GRBM_GUI_ACTIVE" not in cv or "nm::" not in k:
                continue
            cyc = cv["GRBM_GUI_ACTIVE"] / N_XCD
            for c, v in cv.items():
                if c != "GRBM_GUI_ACTIVE" and cyc > 0:
                    per.setdefault(k, {}).setdefault(c, []).append(v / (cyc * 256))
        for k, cv in per.items():
            for c, v in cv.items():
                if c not in cols:
                    cols.append(c)
                table.setdefault(k, {})[c] = float(np.mean(v))
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, "units_%s.md" % args.workload)
    with open(path, "w") as fh:
        fh.write("# Memory-unit counters: %s\n\nCommands (one rocprofv3 --pmc pass each):\n\n" % WORKLOAD_DESC[args.workload])
        for line in args.command.split(" ;; "):
            fh.write("    %s\n" % line)
        fh.write("\nEach entry: the counter summed over the GPU per dispatch, divided by the dispatch's clocks "
                 "(GRBM_GUI_ACTIVE / %d XCDs) times 256 CUs, i.e. the fraction of CU clocks the event held "
                 "(short dispatches also count their dispatch overhead in the clocks, so their fractions read low).\n\n" % N_XCD)
        fh.write("| kernel | " + " | ".join(cols) + " |\n|---|" + "---|" * len(cols) + "\n")
        for k in sorted(table):
            fh.write("| `%s` | " % k[:80] + " | ".join("%.3f" % table[k][c] if c in table[k] else "" for c in cols) + " |\n")
    print("wrote", path)


def summarize_trace(args):
    """Kernel-trace statistics (rocprofv3 --stats) as a short text summary."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(args.summarize_trace, "**", "*kernel_stats.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    if not rows:
        raise SystemExit("no kernel_stats.csv under %s" % args.summarize_trace)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, "kernel_trace_%s.md" % args.workload)
    with open(path, "w") as fh:
        fh.write("# Kernel trace: %s\n\nCommand:\n\n    %s\n\n" % (WORKLOAD_DESC[args.workload], args.command))
        fh.write("| kernel | calls | total ms | average us | share % |\n|---|---|---|---|---|\n")
        for r in rows[:25]:
            fh.write("| `%s` | %s | %.3f | %.2f | %.1f |\n" % (r["Name"][:120], r["Calls"], float(r["TotalDurationNs"]) / 1e6,
                                                          float(r["AverageNs"]) / 1e3, float(r["Percentage"])))
        if args.bench_log:
            line = [l for l in open(args.bench_log) if l.startswith("{")][-1]
            bl = json.loads(line)
            roof = bl["roofline"]
            prof = {r["Name"]: float(r["AverageNs"]) / 1e3 for r in rows}
            avg = prof.get(roof["kernel"])
            # the timed region's launches of that kernel are its last ones in the run (the
            # dense comparator, the vendor GEMM and the calibration loops use other kernels)
            n_timed = roof["launches_per_step"] * bl["steps"]
            durs = []
            for f in glob.glob(os.path.join(args.summarize_trace, "**", "*kernel_trace.csv"), recursive=True):
                for r in csv.DictReader(open(f)):
                    if r["Kernel_Name"] == roof["kernel"]:
                        durs.append((int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
            durs.sort()
            timed = [d for _, d in durs[-n_timed:]] if len(durs) >= n_timed else []
            t_avg = sum(timed) / len(timed) if timed else None
            fh.write("\nThe bench line of this same run names `%s` as its dominant kernel: HIP-event mean %.2f us per "
                     "launch over the %d timed launches; rocprofv3 mean over those same launches (the kernel's last %d "
                     "dispatches) %s us%s; over all %d of its dispatches (autotuning and warm-up included) %s us.\n"
                     % (roof["kernel"], roof["launch_ms"] * 1e3, n_timed, n_timed,
                        "%.2f" % t_avg if t_avg else "n/a",
                        " (ratio %.3f)" % (roof["launch_ms"] * 1e3 / t_avg) if t_avg else "",
                        len(durs), "%.2f" % avg if avg else "n/a"))
            fh.write("\nBench line: `%s`\n" % line.strip()[:600])
    print("wrote", path)


def spmm_bytes(g):
    """Algorithmic HBM bytes of one SpMM launch: compressed values + metadata + B + D (+ C when beta != 0)."""
    es = 1 if g["dtype"] == "i8" else 2
    cd = 4 if g["dtype"] == "i8" else 2
    keep = g["N"] / g["M"]
    bits = int(np.ceil(np.log2(g["M"])))
    total = g["m"] * g["k"] * keep * es + g["m"] * (g["k"] // g["M"]) * g["N"] * bits / 8.0
    total += g["k"] * g["n"] * es + g["m"] * g["n"] * cd
    if g["w"]["beta"] != 0:
        total += g["m"] * g["n"] * cd
    return total


CPU_SAMPLE_FLOPS = 2.0e11   # bound on the oracle's product work (about 10-20 s on 8-16 cores)


CPU_MIN_SECONDS = 10.0                              # whole steps are repeated until at least this much CPU work


def weight_key(g):
    """What fixes a GEMM's pruned weight: the dense draw, its stored shape, the
    element type and the pruning (mode, vector rows, N:M)."""
    along = None if g["mode"] == "tile" else g["op_a"]      # a 4x4 tile pattern serves both orientations
    return (g["w"]["a"], g["host"]["a"].shape, g["dtype"], g["mode"], g["vrows"], g["N"], g["M"], along)


def cpu_baseline(gemms):
    """The oracle (test infrastructure, untuned) doing whole steps of the same work on the host cores,
    repeated until at least CPU_MIN_SECONDS have passed."""
    import oracle
    total = sum(2.0 * g["m"] * g["n"] * g["k"] * len(g["layouts"]) for g in gemms)
    frac = min(1.0, CPU_SAMPLE_FLOPS / total)

    def one_step():
        flops = 0.0
        pruned, packed = {}, {}          # each weight pruned once, compressed once per orientation
        for g in gemms:
            dtype, N, M = g["dtype"], g["N"], g["M"]
            a = g["host"]["a"]
            V = g["vrows"]
            wk = weight_key(g)
            if wk not in pruned:
                if g["mode"] == "tile":
                    p, _ = oracle.prune_tile(a, dtype)
                    oracle.check_tile(p, dtype)
                elif V > 1:
                    p, _ = oracle.prune_vw(a, dtype, V, N, M)
                    oracle.check_vw(p, dtype, V, N, M)
                else:
                    p, _ = oracle.prune_1d(a, dtype, N, M, g["op_a"])
                    oracle.check_1d(p, dtype, N, M, g["op_a"])
                pruned[wk] = p
            p = pruned[wk]
            ck = wk + (g["op_a"], g["m"], g["k"])
            if ck not in packed:
                if V > 1:
                    v, meta = oracle.compress_vw(p, dtype, V, N, M)
                    packed[ck] = oracle.decompress_vw(v, meta, dtype, g["m"], g["k"], V, N, M)
                else:
                    v, meta = oracle.compress(p, dtype, N, M, g["op_a"])
                    packed[ck] = oracle.decompress(v, meta, dtype, g["m"], g["k"], N, M, g["op_a"])
            ahat = packed[ck]
            ahat_log = ahat if g["op_a"] == "N" else np.ascontiguousarray(ahat.T)
            rows = max(1, int(round(g["m"] * frac)))      # the product on the first rows only
            for ob in g["layouts"]:
                b = g["host"]["b"][ob]
                b_log = b if ob == "N" else np.ascontiguousarray(b.T)
                if dtype == "i8":
                    c = g["host"]["c"][:rows] if g["host"]["c"] is not None else None
                    oracle.gemm_i64(ahat_log[:rows], b_log, int(g["w"]["alpha"]), int(g["w"]["beta"]), c)
                else:
                    oracle.gemm_f64(oracle.decode(ahat_log[:rows], dtype), oracle.decode(b_log, dtype), g["w"]["alpha"], 0.0)
                flops += 2.0 * rows * g["n"] * g["k"]
        return flops

    flops, steps = 0.0, 0
    t0 = time.perf_counter()
    while steps == 0 or time.perf_counter() - t0 < CPU_MIN_SECONDS:
        flops += one_step()
        steps += 1
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": "%d step(s) of the workload, each: prune and check of every weight, compress and decompress of it "
                      "in every orientation a GEMM reads it, all in full, and "
                      "the fp64 dense-loop product for every GEMM and layout on the first %.1f%% of the rows "
                      "(value = product flops done / total time), %.1f s" % (steps, 100 * frac, dt)}


if __name__ == "__main__":
    main()
