"""Pick a plan's algorithm id by timing (the blog's algorithm selection, done
by measurement instead of a fixed table).

`autotune_spmm` runs nm_spmm with every algorithm id on the caller's buffers,
times each with HIP events on the launch stream, pins the fastest on the plan
and returns the measured times. It only drives the C ABI; it writes D (and
reads C) exactly as nm_spmm does.
"""
import torch

from . import (NM_ALG_COUNT, nm_plan_get_algorithm, nm_plan_set_algorithm, nm_plan_spmm_kernel, nm_spmm)


def autotune_spmm(plan, alpha, d_values, d_meta, dB, beta, dC, dD, reps=10, warmup=2, stream=None):
    """Returns {algorithm id: (ms per launch, device kernel)} and leaves the fastest id set on the plan."""
    s = stream if stream is not None else torch.cuda.current_stream()
    times, seen = {}, {}
    for alg in range(NM_ALG_COUNT):
        nm_plan_set_algorithm(plan, alg)
        kern = nm_plan_spmm_kernel(plan)
        if kern in seen:                      # same device kernel as an id already timed
            times[alg] = (times[seen[kern]][0], kern)
            continue
        for _ in range(warmup):
            nm_spmm(plan, alpha, d_values, d_meta, dB, beta, dC, dD, stream=s)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            nm_spmm(plan, alpha, d_values, d_meta, dB, beta, dC, dD, stream=s)
        e1.record(s)
        e1.synchronize()
        times[alg] = (e0.elapsed_time(e1) / reps, kern)
        seen[kern] = alg
    best = min(times, key=lambda a: (times[a][0], a))
    nm_plan_set_algorithm(plan, best)
    assert nm_plan_get_algorithm(plan) == best
    return times
