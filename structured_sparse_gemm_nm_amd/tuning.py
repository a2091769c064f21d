"""Pick a plan's algorithm id and split-k by timing (the blog's algorithm
selection, done by measurement instead of a fixed table).

`autotune_spmm` runs nm_spmm with every algorithm id (and every split-k value
asked for) on the caller's buffers, times each with HIP events on the launch
stream, pins the fastest setting on the plan and returns the measured times.
It only drives the C ABI; it writes D (and reads C) exactly as nm_spmm does.
A split-k setting that needs a workspace gets one from torch for its timing;
the caller then allocates the pinned setting's workspace
(nm_spmm_workspace_size) for its own calls.
"""
import torch

from . import (NM_ALG_COUNT, nm_plan_get_algorithm, nm_plan_get_split_k, nm_plan_set_algorithm, nm_plan_set_split_k,
               nm_plan_spmm_kernel, nm_spmm, nm_spmm_workspace_size)


def autotune_spmm(plan, alpha, d_values, d_meta, dB, beta, dC, dD, reps=10, warmup=2, stream=None, split_ks=(1,),
                  rounds=3):
    """Returns {(algorithm id, split-k): (ms per launch, device kernel)} and leaves the
    fastest setting on the plan. Settings that launch the same kernel with the same
    effective split are timed once. Every setting is timed in each of `rounds`
    passes over all of them and keeps its best pass, so that a pass slowed by
    the clock (which drops after idle gaps and recovers over some milliseconds
    of work) does not decide the choice."""
    s = stream if stream is not None else torch.cuda.current_stream()
    cands, alias = [], {}                  # (alg, sk, kernel, workspace); settings sharing a timed one
    seen = {}
    for alg in range(NM_ALG_COUNT):
        for sk in split_ks:
            nm_plan_set_algorithm(plan, alg)
            nm_plan_set_split_k(plan, sk)
            kern = nm_plan_spmm_kernel(plan)
            key = (kern, nm_plan_get_split_k(plan)[1])
            if key in seen:
                alias[(alg, sk)] = seen[key]
                continue
            nbytes = nm_spmm_workspace_size(plan)
            ws = torch.empty((nbytes,), dtype=torch.uint8, device=dD.device) if nbytes else None
            seen[key] = (alg, sk)
            cands.append((alg, sk, kern, ws))
    best_ms = {}
    for _ in range(rounds):
        for alg, sk, kern, ws in cands:
            nm_plan_set_algorithm(plan, alg)
            nm_plan_set_split_k(plan, sk)
            for _ in range(warmup):
                nm_spmm(plan, alpha, d_values, d_meta, dB, beta, dC, dD, stream=s, workspace=ws)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(reps):
                nm_spmm(plan, alpha, d_values, d_meta, dB, beta, dC, dD, stream=s, workspace=ws)
            e1.record(s)
            e1.synchronize()
            ms = e0.elapsed_time(e1) / reps
            best_ms[(alg, sk)] = min(ms, best_ms.get((alg, sk), ms))
    times = {(alg, sk): (best_ms[(alg, sk)], kern) for alg, sk, kern, _ in cands}
    for a, src in alias.items():
        times[a] = times[src]
    del cands
    best = min(times, key=lambda a: (times[a][0], a))
    nm_plan_set_algorithm(plan, best[0])
    nm_plan_set_split_k(plan, best[1])
    assert nm_plan_get_algorithm(plan) == best[0]
    return times
