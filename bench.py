#!/usr/bin/env python3
"""Optimizer-step benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one library call over the whole tensor list of the workload (default:
Adafactor with beta1 = 0.9 over a Llama-7B-shaped list, 291 tensors, 6.74e9 fp32
parameters, bf16 gradients), with parameters, states, gradients and workspace
resident in HBM before timing. W untimed steps, then exactly K steps between two
hipEvents on the stream (synchronised on both sides). One JSON line on stdout:

* ``value``: optimizer-step throughput in parameters per second (whole job).
* ``hbm``: the step's compulsory bytes (read G once, read and write the parameter
  and every full-size state once) over the step time, against 8 TB/s; beside it
  (``measured_*``) the bytes the step's kernels move by the committed rocprofv3
  counter record of the whole step (Adafactor workloads), over the same time.
* ``roofline``: the dominant pass (the apply pass for Adafactor), its algorithmic
  bytes per launch over its average duration, timed with hipEvents that the
  library records between its passes on the same stream during the timed steps.
* ``cpu_baseline``: the fp64 oracle stepping the whole list once on the host's
  cores (one worker process per CPU, at most 16), in parameters per second, with
  the CPU model, and a bounded single-thread sample beside it.

Adafactor with scale_parameter steps through meo_adafactor_step_carry by default
(``--param-sumsq carry``): each step's apply pass sums the squares of the
parameter it stores, and the next step takes RMS(X) from that sum instead of
reading the parameter again. Nothing else writes the parameters between the
steps here, which is what the carry requires. The same number of steps of the
plain call (RMS(X) read from the parameter every step) is timed afterwards on the
same buffers and reported under ``read_param_sumsq``; ``--param-sumsq read``
times only the plain call.

With more than one GPU requested it exits: the step has no cross-GPU work to
measure here (see the design notes on sharding).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0


def _moment_bytes(wl, spec) -> float:
    """Bytes per element of the tensor's first moment: 4, 2, or 1 + 4 / 128 for
    int8 codes with one float32 scale per 128 values (where the 8-bit rule applies)."""
    import torch
    from memory_efficient_optimizers_amd.optim import moment_dtype
    dt = moment_dtype(wl.optimizer, spec.shape, wl.state_dtype, wl.param_dtype)
    return {torch.float32: 4.0, torch.bfloat16: 2.0, torch.int8: 1.0 + 4.0 / 128}[dt]


def _bytes_per_param(wl, spec, numel) -> dict:
    """Algorithmic bytes of one tensor: whole step, and per pass. gb, xb, mb: bytes
    per element of the gradient, the parameter and the first moment."""
    gb = 2 if str(wl.grad_dtype).endswith("bfloat16") else 4
    xb = 2 if str(wl.param_dtype).endswith("bfloat16") else 4
    mb = _moment_bytes(wl, spec)
    fac = len(spec.shape) >= 2 and wl.optimizer != "lamb"
    n = numel
    if fac:
        lead = math.prod(spec.shape[:-2]) if len(spec.shape) > 2 else 1
        rc = lead * (spec.shape[-2] + spec.shape[-1])
    else:
        rc = 0
    if wl.optimizer == "adafactor":
        mom = wl.hparams.get("beta1") is not None
        step = n * (gb + 2 * xb + (2 * mb if mom else 0) + (0 if fac else 8)) + 8 * rc
        apply = n * (gb + 2 * xb + (2 * mb if mom else 0) + (0 if fac else 4)) + 4 * rc
        return {"step": step, "adafactor_apply": apply}
    if wl.optimizer == "came":
        step = n * (gb + 2 * xb + 2 * mb + (0 if fac else 8)) + 16 * rc
        mom = n * (gb + 2 * mb + (0 if fac else 4 + 2 * xb)) + 4 * rc   # G, M rw (1-D: also V read, X rw)
        app = (n * (mb + 2 * xb) + 4 * rc) if fac else 0                 # M read, X rw
        return {"step": step, "came_mom": mom, "came_apply": app}
    step = n * (gb + 2 * xb + 2 * mb + 8)
    return {"step": step, "lamb_moments": n * (gb + xb + 2 * mb + 8), "lamb_apply": n * (2 * xb + mb + 4)}


def algorithmic_bytes(wl) -> dict:
    tot: dict = {}
    for s in wl.specs:
        for k, v in _bytes_per_param(wl, s, s.numel).items():
            tot[k] = tot.get(k, 0) + v
    return tot


def _oracle_inputs(wl, k):
    """Tensor k's parameter, gradient (step 0), state and storage flags, drawn on
    the CPU (the same generators the tests use; not part of any timing)."""
    import torch
    import oracle
    import workloads
    from memory_efficient_optimizers_amd.optim import moment_dtype
    spec = wl.specs[k]
    x = workloads.init_params(wl, "cpu", [k])[0].to(torch.float64).numpy()
    sc = workloads.grad_scales(wl, "cpu", [k])
    g = workloads.grads(wl, 0, sc, "cpu", [k])[0].to(torch.float64).numpy()
    mdt = moment_dtype(wl.optimizer, spec.shape, wl.state_dtype, wl.param_dtype)
    storage = dict(param_bf16=wl.param_dtype == torch.bfloat16, exp_avg_bf16=mdt == torch.bfloat16,
                   exp_avg_i8=mdt == torch.int8)
    st = oracle.INIT_STATE[wl.optimizer](x.shape, dict(wl.hparams), exp_avg_i8=storage["exp_avg_i8"])
    return x, g, st, storage


def _oracle_tensor_job(job):
    """One worker task: draw tensor k's inputs, then time one fp64 oracle step of
    it. Returns (worker pid, k, elements, oracle seconds)."""
    import oracle
    import workloads
    name, k = job
    wl = workloads.WORKLOADS[name]
    x, g, st, storage = _oracle_inputs(wl, k)
    t0 = time.perf_counter()
    oracle.STEP_TENSOR[wl.optimizer](x, g, st, dict(wl.hparams), 1, **storage)
    return os.getpid(), k, x.size, time.perf_counter() - t0


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, single_budget_s: float = 15.0) -> dict:
    """The fp64 oracle (plain NumPy, as it stands) stepping the workload on the host.

    All cores: every tensor of the list, streamed tensor by tensor (largest first)
    over one worker process per CPU this process may run on (at most 16, the
    host share of one GPU); each worker draws a tensor's inputs on the CPU, then
    times one oracle step of it. ``value`` is the list's parameters over the
    longest per-worker sum of oracle seconds (the workers run side by side, so
    the oracle work of the whole list takes that long); ``wall_s`` is the pool's
    wall time including the draws. Single thread: the first tensors of the list in
    order, in this process, until about ``single_budget_s`` seconds of oracle
    time. Run before anything touches the GPU (the workers are fresh processes)."""
    import multiprocessing
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    jobs = sorted(range(len(wl.specs)), key=lambda k: -wl.specs[k].numel)
    t0 = time.perf_counter()
    with multiprocessing.get_context("spawn").Pool(workers) as pool:
        res = pool.map(_oracle_tensor_job, [(wl.name, k) for k in jobs], chunksize=1)
    wall = time.perf_counter() - t0
    per_worker: dict = {}
    for pid, _, _, dt in res:
        per_worker[pid] = per_worker.get(pid, 0.0) + dt
    total = sum(n for _, _, n, _ in res)
    makespan = max(per_worker.values())

    import oracle
    done, spent, count = 0, 0.0, 0
    for k in range(len(wl.specs)):
        x, g, st, storage = _oracle_inputs(wl, k)
        t1 = time.perf_counter()
        oracle.STEP_TENSOR[wl.optimizer](x, g, st, dict(wl.hparams), 1, **storage)
        spent += time.perf_counter() - t1
        done += x.size
        count += 1
        del x, g, st
        if spent > single_budget_s:
            break
    return {"value": total / makespan, "unit": "params/s", "cores": workers, "kind": "oracle",
            "cpu": _cpu_model(), "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"one fp64 oracle step of every tensor of the workload ({len(res)} tensors, {total} "
                      f"parameters), streamed tensor by tensor over {workers} worker processes; oracle seconds "
                      f"per worker measured (longest {makespan:.1f} s), inputs drawn on the CPU outside them",
            "wall_s": wall,
            "single_thread": {"value": done / spent, "unit": "params/s", "cores": 1,
                              "sample": f"the first {count} tensors of the list ({done} parameters, "
                                        f"{done / total:.1%} of it), {spent:.1f} s of oracle time"}}


def profile_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter record,
    or None if there is none or the kernel's sources changed since it was taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"{kernel}_{workload.split('_', 1)[1]}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel") != kernel or rec.get("workload") != workload:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(here, src), "rb") as f:
            h.update(f.read())
    return rec["bytes_per_launch"] if h.hexdigest() == rec["sources_sha256"] else None


def step_traffic(workload: str, passes: dict, steps: int, carry: bool):
    """HBM bytes per step from the committed whole-step counter record (per-launch
    bytes of every kernel of the step, rocprofv3 FETCH_SIZE / WRITE_SIZE), weighted
    by the launches the timed steps made; None without a record, or when the
    kernels' sources changed since it was taken, or when a timed pass has no entry."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"adafactor_step_{workload.split('_', 1)[1]}_traffic.json")
    if not workload.startswith("adafactor_") or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("workload") != workload:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(here, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    per = rec["bytes_per_launch"]
    total = 0.0
    for name, v in passes.items():
        key = "adafactor_apply_carry" if (name == "adafactor_apply" and carry) else name
        if key not in per:
            return None
        total += per[key] * v["launches"]
    return total / steps


def flat_views(torch, shapes, dtype, device):
    """Views of the given shapes into one buffer, each starting 256-byte aligned."""
    es = torch.empty((), dtype=dtype).element_size()
    align = 256 // es
    sizes = [math.prod(s) for s in shapes]
    offs, o = [], 0
    for n in sizes:
        offs.append(o)
        o += (n + align - 1) // align * align
    buf = torch.empty(max(o, 1), dtype=dtype, device=device)
    return [buf[a:a + n].view(s) for a, n, s in zip(offs, sizes, shapes)]


# Which buffers go to which third of HBM (memory_efficient_optimizers_amd/hbm.py):
# no pass may write two full-size streams into one third. Adafactor's apply writes
# the parameter and the first moment; CAME's passes write one each; LAMB's moment
# pass writes both moments. Index into the groups of chunks, largest first.
THIRDS = {"adafactor": {"param": 0, "exp_avg": 1, "grad": 2},
          "came": {"param": 0, "exp_avg": 1, "grad": 2},
          "lamb": {"exp_avg": 0, "exp_avg_sq": 1, "param": 2, "grad": 2}}


def thirds_buffers(torch, _lib, wl, mdts, beta1, dev, same_third_copy=False):
    """Parameters, gradients and states of the workload placed by HBM third: the
    device's free memory is taken as 2 GiB chunks, each chunk's third found by the
    timing probe, and each full-size kind packed into chunks of its own third (the
    small statistics are ordinary allocations). With ``same_third_copy`` a second
    first moment is packed into the parameter's third too, to time the layout the
    placement avoids. Returns (params, grads, states, placement record, extra first
    moment or None); unused chunks are freed."""
    from memory_efficient_optimizers_amd import hbm
    shapes = [s.shape for s in wl.specs]
    proto = [_lib.state_shapes(wl.optimizer, s, beta1=beta1, i8=m == torch.int8) for s, m in zip(shapes, mdts)]
    big = {"param": [(k, shapes[k], wl.param_dtype) for k in range(len(shapes))],
           "grad": [(k, shapes[k], wl.grad_dtype) for k in range(len(shapes))],
           "exp_avg": [(k, shapes[k], mdts[k]) for k in range(len(shapes)) if "exp_avg" in proto[k]]}
    if wl.optimizer == "lamb":
        big["exp_avg_sq"] = [(k, shapes[k], torch.float32) for k in range(len(shapes))]
    pool = hbm.ChunkPool(torch, dev)
    groups = pool.classify(_lib)
    need = {kind: hbm.chunks_needed([math.prod(s) * torch.empty((), dtype=d).element_size() for _, s, d in items])
            for kind, items in big.items()}
    plan = THIRDS[wl.optimizer]
    mode = "thirds"
    if groups is None or len(groups) < 2:
        groups, mode = [list(range(len(pool.chunks)))], "allocation order"
    taken = {g: 0 for g in range(len(groups))}
    chunk_ids = {}
    order = sorted(big, key=lambda kind: plan.get(kind, 0))
    if same_third_copy and "exp_avg" in big:
        order.append("exp_avg_same_third")
        need["exp_avg_same_third"] = need["exp_avg"]
    for kind in order:
        g = plan.get("exp_avg" if kind == "exp_avg_same_third" else kind, 0)
        if kind == "exp_avg_same_third":
            g = plan["param"]
        g = min(g, len(groups) - 1)
        if taken[g] + need[kind] > len(groups[g]):  # not enough room in that third: any other
            g = max(range(len(groups)), key=lambda i: len(groups[i]) - taken[i])
        chunk_ids[kind] = groups[g][taken[g]:taken[g] + need[kind]]
        taken[g] += need[kind]
        if len(chunk_ids[kind]) < need[kind]:
            raise RuntimeError(f"not enough device memory for the {kind} buffers")
    views = {kind: pool.views(chunk_ids[kind], [s for _, s, _ in big["exp_avg" if kind == "exp_avg_same_third"
                                                                    else kind]],
                              [d for _, _, d in big["exp_avg" if kind == "exp_avg_same_third" else kind]])
             for kind in chunk_ids}
    where = {c: k for k, grp in enumerate(groups) for c in grp}
    record = {"mode": mode, "chunk_gib": hbm.CHUNK // hbm.GiB, "chunks": len(pool.chunks),
              "groups": [len(g) for g in groups], "probe_apply_ms": pool.probe_ms,
              "third_of": {kind: sorted({where[c] for c in ids}) for kind, ids in chunk_ids.items()}}
    pool.release([c for ids in chunk_ids.values() for c in ids])
    params = [None] * len(shapes)
    grads = [None] * len(shapes)
    states = [dict() for _ in shapes]
    for kind, items in big.items():
        for (k, _, _), v in zip(items, views[kind]):
            if kind == "param":
                params[k] = v
            elif kind == "grad":
                grads[k] = v
            else:
                states[k][kind] = v
    for k, st in enumerate(proto):
        for key, shp in st.items():
            if key not in states[k]:
                states[k][key] = torch.zeros(shp, dtype=torch.float32, device=dev)
        for v in states[k].values():
            v.zero_()
    extra = None
    if "exp_avg_same_third" in views:
        extra = [None] * len(shapes)
        for (k, _, _), v in zip(big["exp_avg"], views["exp_avg_same_third"]):
            extra[k] = v.zero_()
    return params, grads, states, record, extra


def copy_calibration(torch, args) -> int:
    n = 1 << 29  # fp32 elements: 2 GiB read + 2 GiB written, one dispatch per copy
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    # torch.mul(..., out=) is one elementwise kernel that reads and writes n floats
    # (a same-dtype copy_ may go to a DMA engine that kernel counters do not see).
    for _ in range(max(args.warmup, 1)):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        torch.mul(src, 1.0, out=dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbps = 2 * 4 * n / (ms / 1e3) / 1e9
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "ms": ms, "GBps": gbps,
                      "frac_of_peak": gbps / HBM_PEAK_GBPS}), flush=True)
    return 0


def shard_bench(torch, _lib, workloads, wl, args) -> int:
    """One rank's share of a row-sharded step over N ranks, at the workload's real
    shapes: rank 0's rows of every factored tensor (all columns; the column
    statistic whole) and its element range of every 1-D tensor (LAMB: of every
    tensor); stats call, then apply call, per step (CAME: stats, moment, apply).
    The partial sums go from one call to the next unreduced: the all-reduce over
    ranks that sits between them is not part of the measured work, so the values
    reached are not a real step's. Adafactor with scale_parameter carries the
    shard's sum(X^2) as the whole-list bench does (``--param-sumsq``)."""
    from memory_efficient_optimizers_amd.optim import moment_dtype
    n, dev, opt = args.shard_ranks, "cuda", wl.optimizer
    hp = dict(wl.hparams)
    beta1 = hp.get("beta1") is not None or opt == "lamb"
    local, totals = [], []
    for s in wl.specs:
        if opt != "lamb" and len(s.shape) >= 2:
            local.append(tuple(s.shape[:-2]) + (s.shape[-2] // n,) + tuple(s.shape[-1:]))
            totals.append(s.shape[-2])
        else:
            local.append((math.prod(s.shape) // n,))
            totals.append(math.prod(s.shape))
    params = flat_views(torch, local, wl.param_dtype, dev)
    for p in params:
        p.normal_(0.0, 0.02)
    grads = flat_views(torch, local, wl.grad_dtype, dev)
    for g in grads:
        g.normal_(0.0, 1e-3)
    states = []
    for s, p in zip(wl.specs, params):
        st = _lib.init_state(opt, p, beta1=beta1, state_dtype=moment_dtype(opt, s.shape, wl.state_dtype, wl.param_dtype))
        if "exp_avg_sq_col" in st:
            st["exp_avg_sq_col"] = torch.zeros(tuple(s.shape[:-2]) + tuple(s.shape[-1:]), device=dev)
        states.append(st)
    carry = opt == "adafactor" and hp.get("scale_parameter", True) and args.param_sumsq == "carry"
    if carry:
        sums = torch.zeros(len(states), dtype=torch.float32, device=dev)
        for i, st in enumerate(states):
            st["param_sumsq"] = sums[i:i + 1]
    hps = {"adafactor": _lib.adafactor_hparams, "lamb": _lib.lamb_hparams, "came": _lib.came_hparams}[opt](**hp)
    ws = _lib.workspace(getattr(_lib, f"meo_{opt}_workspace_size")(params, grads), dev)
    part = torch.zeros(getattr(_lib, f"meo_{opt}_partials_size")(params, grads), device=dev)
    conf = torch.zeros(max(_lib.meo_came_confidence_size(params, grads), 1), device=dev) if opt == "came" else None
    call = _lib.PreparedShardStep(opt, hps, params, grads, totals, states, part, ws, conf, carry=carry)

    def step(t):
        call.stats(t, stream)
        if opt == "came":
            call.moment(t, stream)
        call.apply(t, stream)

    stream = torch.cuda.current_stream()
    t = 0
    for _ in range(args.warmup):
        t += 1
        step(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        t += 1
        step(t)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    numel = sum(math.prod(s) for s in local)
    whole = algorithmic_bytes(wl)["step"]
    step_bytes = whole * numel / wl.numel  # the same bytes per parameter on the rank's share
    out = {"metric": f"one rank's share of a row-sharded optimizer step over {n} ranks (all-reduce excluded)",
           "value": numel / (ms / 1e3), "unit": "params/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "data": "synthetic",
           "config": {"workload": wl.name, "ranks": n, "rank_params": numel, "partials_floats": part.numel(),
                      "param_sumsq": "carry" if carry else "read"},
           "hbm": {"step_bytes": step_bytes, "achieved": step_bytes / (ms / 1e3) / 1e9, "peak": HBM_PEAK_GBPS,
                   "unit": "GB/s", "frac": step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS}}
    print(json.dumps(out), flush=True)
    return 0


GALORE_WORKLOADS = {
    # name: (parameter dtype, rank, scale, update_proj_gap)
    "galore_llama7b": ("float32", 256, 0.25, 200),
    "galore_llama7b_bf16": ("bfloat16", 256, 0.25, 200),
}


def galore_bytes_flops(shapes, rank: int, xb: int) -> dict:
    """Algorithmic HBM bytes and matrix flops of one GaLore step (not a refresh
    step) per pass. Projected (2-D) tensor, d = min(m, n), D = max(m, n), r =
    min(rank, d): the projection reads G (bf16) and U^T once, reads and writes both
    moments ([D][r] fp32) and writes N's two bf16 planes; the back-projection reads
    N's planes and U once and reads and writes the parameter; 2 m n r flops for the
    projection, twice that for the back-projection (two planes). Other tensors:
    AdamW reads G and both moments and writes both moments, reads and writes X."""
    out = {"galore_project": 0, "galore_back": 0, "galore_adamw": 0,
           "flops_project": 0, "flops_back": 0}
    for shape in shapes:
        n_el = math.prod(shape)
        if len(shape) == 2 and n_el:
            m, n = shape
            d, D = min(m, n), max(m, n)
            r = min(rank, d)
            out["galore_project"] += m * n * 2 + D * r * (16 + 4) + d * r * 2
            out["galore_back"] += m * n * 2 * xb + D * r * 4 + d * r * 2
            out["flops_project"] += 2 * m * n * r
            out["flops_back"] += 4 * m * n * r
        else:
            out["galore_adamw"] += n_el * (2 + 2 * xb + 16)
    out["step"] = out["galore_project"] + out["galore_back"] + out["galore_adamw"]
    return out


def galore_cpu_baseline(shapes, rank: int, scale: float, param_bf16: bool, budget_s: float = 15.0) -> dict:
    """The fp64 oracle's GaLore step (a step that is not a refresh step, seeded
    projectors) on the workload's tensors in list order until about `budget_s`
    seconds, on one BLAS thread: parameters stepped per second."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import galore as ga
    rng = np.random.default_rng(0)
    hp = dict(rank=rank, scale=scale)
    done, spent, count = 0, 0.0, 0
    with threadpool_limits(limits=1):
        for shape in shapes:
            x = 0.02 * rng.standard_normal(shape)
            g = 1e-3 * rng.standard_normal(shape)
            st = ga.galore_init_state(shape, hp)
            if "projector" in st:
                st["projector"] = np.linalg.qr(rng.standard_normal(st["projector"].shape))[0]
            t0 = time.perf_counter()
            ga.galore_step_tensor(x, g, st, hp, 2, param_bf16=param_bf16)
            spent += time.perf_counter() - t0
            done += x.size
            count += 1
            if spent > budget_s:
                break
    return {"value": done / spent, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"one fp64 GaLore step (not a refresh step) of the first {count} tensors of the same "
                      f"list ({done} parameters), {spent:.1f} s of oracle time, NumPy on one BLAS thread"}


def galore_bench(torch, _lib, workloads, args) -> int:
    """The GaLore step over the Llama-7B-shaped list: every 2-D tensor projected at
    rank 256 (scale 0.25), norms by flat AdamW. Gradients of 2-D tensors are a
    rank-256 signal plus noise; the step's time does not depend on the values,
    the refresh's convergence does. The first warmup step is a refresh
    step (t = 1), which computes every projector; the timed steps are not (t - 1 is
    not a multiple of update_proj_gap). The refresh is timed on its own afterwards,
    started from the stored bases as every refresh after the first is
    (``refresh_ms``); ``first_step_ms`` is the t = 1 step, whose refresh starts from
    no basis."""
    pdt, rank, scale, gap = GALORE_WORKLOADS[args.workload]
    pdt = getattr(torch, pdt)
    specs = workloads.llama_specs()
    shapes = [s.shape for s in specs]
    dev = "cuda"
    gen = torch.Generator(device=dev).manual_seed(0)
    params = flat_views(torch, shapes, pdt, dev)
    grads = flat_views(torch, shapes, torch.bfloat16, dev)
    for p, g in zip(params, grads):
        p.copy_(0.02 * torch.randn(p.shape, generator=gen, device=dev))
        if p.dim() == 2:
            # rank-`rank` signal plus noise (entries ~1e-3): singular values decaying
            # by 0.99 per index, then a gap to a noise floor about a tenth of the
            # last one, the low-rank structure the projection relies on
            m, n = p.shape
            k = min(rank, m, n)
            a = torch.randn(m, k, generator=gen, device=dev)
            b = torch.randn(n, k, generator=gen, device=dev)
            sv = 0.99 ** torch.arange(k, device=dev, dtype=torch.float32)
            sig = (a * sv) @ b.T
            sig *= 1e-3 / sig.std()
            g.copy_(sig + 3e-5 * torch.randn(m, n, generator=gen, device=dev))
            del a, b, sig
        else:
            g.copy_(1e-3 * torch.randn(g.shape, generator=gen, device=dev))
    states = []
    for p in params:
        st = {}
        for k, shp in _lib.galore_state_shapes(p.shape, rank).items():
            st[k] = torch.zeros(shp, dtype=torch.bfloat16 if k.startswith("projector") else torch.float32,
                                device=dev)
        states.append(st)
    hp = _lib.galore_hparams(lr=1e-3, rank=rank, scale=scale, update_proj_gap=gap, weight_decay=0.0)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(hp, params, grads), dev)
    stream = torch.cuda.current_stream()
    numel = sum(p.numel() for p in params)

    t = 0
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(max(args.warmup, 1)):
        t += 1
        if i == 0:
            c0.record(stream)
        _lib.meo_galore_step(hp, t, params, grads, states, ws, stream)
        if i == 0:
            c1.record(stream)
    torch.cuda.synchronize()
    first_ms = c0.elapsed_time(c1)  # t = 1: the first refresh (no stored basis) and a step
    _lib.meo_profile_enable(True)
    _lib.meo_profile_collect()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        t += 1
        assert (t - 1) % gap != 0
        _lib.meo_galore_step(hp, t, params, grads, states, ws, stream)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    passes = _lib.meo_profile_collect()
    step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    ms_step = evs[0].elapsed_time(evs[-1]) / args.steps
    # the refresh alone
    nref = 2
    _lib.meo_profile_collect()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for _ in range(nref):
        _lib.meo_galore_refresh(hp, params, grads, states, ws, stream)
    r1.record(stream)
    torch.cuda.synchronize()
    _lib.meo_profile_enable(False)
    _lib.meo_profile_collect()
    refresh_ms = r0.elapsed_time(r1) / nref

    xb = 2 if pdt == torch.bfloat16 else 4
    ab = galore_bytes_flops(shapes, rank, xb)
    dominant = max((k for k in passes if k in ab), key=lambda k: passes[k]["ms"])
    avg_ms = passes[dominant]["ms"] / passes[dominant]["launches"]
    per_pass = {}
    for k in ("galore_project", "galore_back"):
        if k in passes:
            ms = passes[k]["ms"] / passes[k]["launches"]
            fl = ab["flops_project" if k == "galore_project" else "flops_back"]
            per_pass[k] = {"ms": ms, "GB/s": ab[k] / (ms / 1e3) / 1e9, "TFLOP/s": fl / (ms / 1e3) / 1e12}
    achieved = ab[dominant] / (avg_ms / 1e3) / 1e9
    value = numel / (ms_step / 1e3)
    out = {
        "metric": "optimizer-step params/s, 7B-shaped GaLore (rank 256) step",
        "value": value,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "step_ms": {"min": min(step_ms), "median": sorted(step_ms)[len(step_ms) // 2], "max": max(step_ms)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 mfma, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": args.workload, "optimizer": "galore", "tensors": len(shapes), "params": numel,
                   "grad_dtype": "bfloat16", "param_dtype": str(pdt).replace("torch.", ""), "rank": rank,
                   "scale": scale, "update_proj_gap": gap},
        "refresh_ms": refresh_ms,
        "first_step_ms": first_ms,
        "amortized_ms_per_step": ms_step + refresh_ms / gap,
        "hbm": {"step_bytes": ab["step"], "achieved": ab["step"] / (ms_step / 1e3) / 1e9, "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": ab["step"] / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBPS},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": profile_traffic(dominant, args.workload),
                     "bytes_per_launch": ab[dominant], "avg_ms": avg_ms},
        "mfma": {k: {"achieved": v["TFLOP/s"], "peak": 2500.0, "unit": "TFLOP/s", "frac": v["TFLOP/s"] / 2500.0}
                 for k, v in per_pass.items()},
        "passes_ms_per_step": {k: v["ms"] / args.steps for k, v in passes.items()},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = galore_cpu_baseline(shapes, rank, scale, pdt == torch.bfloat16)
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="adafactor_llama7b",
                    help="a workload of workloads.py, or galore_llama7b / galore_llama7b_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layout", choices=["thirds", "flat", "separate"], default="thirds",
                    help="thirds: each kind of full-size buffer in 2 GiB chunks of its own third of HBM, "
                         "found by a timing probe (default); flat: one buffer per kind of tensor, in "
                         "allocation order; separate: one allocation per tensor")
    ap.add_argument("--shard-ranks", type=int, default=0,
                    help="instead of the whole step: time one rank's share of a row-sharded step over N ranks "
                         "(the all-reduces of the partial sums between the calls are not part of it)")
    ap.add_argument("--param-sumsq", choices=["carry", "read"], default="carry",
                    help="Adafactor with scale_parameter: carry sum(X^2) from the previous step's apply pass "
                         "(default; the plain call is timed beside it), or read X for it every step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the step: time a plain device copy of 4 GiB (one elementwise kernel), "
                         "the reference for achievable bandwidth and for scaling rocprofv3 byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the optimizer step on one GPU; the step exchanges nothing between "
              "GPUs (each data-parallel rank runs the same step on its own copy), so there is no "
              "multi-GPU figure to take here. Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import workloads
    from memory_efficient_optimizers_amd import _lib
    from memory_efficient_optimizers_amd.optim import moment_dtype

    # The CPU leg first: its worker processes start before this process touches
    # the GPU.
    cpu = None
    if (not args.no_cpu_baseline and not args.copy_calibration and args.workload not in GALORE_WORKLOADS
            and args.shard_ranks <= 1):
        cpu = cpu_baseline(workloads.WORKLOADS[args.workload])

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    if args.copy_calibration:
        return copy_calibration(torch, args)
    _lib.load()
    if args.workload in GALORE_WORKLOADS:
        torch.cuda.set_device(0)
        return galore_bench(torch, _lib, workloads, args)
    wl = workloads.WORKLOADS[args.workload]
    dev = "cuda"
    torch.cuda.set_device(0)
    if args.shard_ranks > 1:
        return shard_bench(torch, _lib, workloads, wl, args)

    hp = dict(wl.hparams)
    beta1 = hp.get("beta1") is not None
    mdts = [moment_dtype(wl.optimizer, s.shape, wl.state_dtype, wl.param_dtype) for s in wl.specs]
    placement, m_same = None, None
    if args.layout == "thirds":
        params, grads, states, placement, m_same = thirds_buffers(
            torch, _lib, wl, mdts, beta1 or wl.optimizer != "adafactor", dev,
            same_third_copy=wl.optimizer == "adafactor" and beta1)
        workloads.init_params(wl, dev, out=params)
        workloads.grads(wl, 0, workloads.grad_scales(wl, dev), dev, out=grads)
    elif args.layout == "flat":
        # One flat buffer per kind (parameters, gradients, each state), tensors as
        # 256-byte aligned views, as flat-parameter training frameworks keep them.
        shapes = [s.shape for s in wl.specs]
        params = flat_views(torch, shapes, wl.param_dtype, dev)
        workloads.init_params(wl, dev, out=params)
        grads = flat_views(torch, shapes, wl.grad_dtype, dev)
        workloads.grads(wl, 0, workloads.grad_scales(wl, dev), dev, out=grads)
        proto = [_lib.state_shapes(wl.optimizer, s, beta1=beta1, i8=m == torch.int8) for s, m in zip(shapes, mdts)]
        states = [dict() for _ in shapes]
        for key, dt in sorted({(k, mdts[i] if k == "exp_avg" else torch.float32)
                               for i, st in enumerate(proto) for k in st}, key=str):
            idx = [i for i, st in enumerate(proto) if key in st and (key != "exp_avg" or mdts[i] == dt)]
            views = flat_views(torch, [proto[i][key] for i in idx], dt, dev)
            for i, v in zip(idx, views):
                v.zero_()
                states[i][key] = v
    else:
        params = workloads.init_params(wl, dev)
        grads = workloads.grads(wl, 0, workloads.grad_scales(wl, dev), dev)
        states = [_lib.init_state(wl.optimizer, p, beta1=beta1, state_dtype=m) for p, m in zip(params, mdts)]
    hps = {"adafactor": _lib.adafactor_hparams, "came": _lib.came_hparams,
           "lamb": _lib.lamb_hparams}[wl.optimizer](**hp)
    wsize = getattr(_lib, f"meo_{wl.optimizer}_workspace_size")(params, grads)
    ws = _lib.workspace(wsize, dev)
    carry = (wl.optimizer == "adafactor" and hp.get("scale_parameter", True) and args.param_sumsq == "carry")
    if carry:
        sums = torch.zeros(len(states), dtype=torch.float32, device=dev)
        for i, st in enumerate(states):
            st["param_sumsq"] = sums[i:i + 1]
    call = _lib.PreparedStep(wl.optimizer, hps, params, grads, states, ws, carry=carry)
    stream = torch.cuda.current_stream()
    numel = wl.numel

    def timed(call, t):
        """W untimed steps, then K timed ones; (step index, per-step ms, total ms, passes)."""
        for _ in range(args.warmup):
            t += 1
            call(t, stream)
        torch.cuda.synchronize()
        _lib.meo_profile_enable(True)
        _lib.meo_profile_collect()  # drop anything recorded before
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for i in range(args.steps):
            t += 1
            call(t, stream)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
        _lib.meo_profile_enable(False)
        return t, step_ms, evs[0].elapsed_time(evs[-1]), _lib.meo_profile_collect()

    t, step_ms, total_ms, passes = timed(call, 0)
    ms_step = total_ms / args.steps
    value = numel / (ms_step / 1e3)
    read = None
    if carry:  # the plain call on the same buffers, for comparison
        t, r_ms, r_total, r_passes = timed(_lib.PreparedStep(wl.optimizer, hps, params, grads, states, ws), t)
        read = {"ms_per_step": r_total / args.steps, "value": numel / (r_total / args.steps / 1e3),
                "step_ms": {"min": min(r_ms), "median": sorted(r_ms)[len(r_ms) // 2], "max": max(r_ms)},
                "passes_ms_per_step": {k: v["ms"] / args.steps for k, v in r_passes.items()}}
        r_meas = step_traffic(wl.name, r_passes, args.steps, False)
        read["measured_step_bytes"] = r_meas
        read["measured_frac"] = None if r_meas is None else r_meas / (read["ms_per_step"] / 1e3) / 1e9 / HBM_PEAK_GBPS

    if m_same is not None:
        # The plain step (RMS(X) read, as read_param_sumsq) with the first moment in
        # the parameter's third instead: the layout the placement avoids. Its apply
        # kernel is the plain one, so it stays apart from the carry apply's launches
        # in a kernel trace.
        sts2 = [dict(st, exp_avg=m) if m is not None else st for st, m in zip(states, m_same)]
        t, _, s_total, s_passes = timed(_lib.PreparedStep(wl.optimizer, hps, params, grads, sts2, ws), t)
        placement["plain_step_exp_avg_in_param_third"] = {
            "ms_per_step": s_total / args.steps,
            "apply_ms": s_passes["adafactor_apply"]["ms"] / s_passes["adafactor_apply"]["launches"]}
        if read is not None:
            placement["plain_step"] = {"ms_per_step": read["ms_per_step"],
                                       "apply_ms": read["passes_ms_per_step"]["adafactor_apply"]}

    ab = algorithmic_bytes(wl)
    step_gbps = ab["step"] / (ms_step / 1e3) / 1e9
    dominant = max((k for k in passes if k in ab), key=lambda k: passes[k]["ms"])  # the apply pass
    avg_ms = passes[dominant]["ms"] / passes[dominant]["launches"]
    achieved = ab[dominant] / (avg_ms / 1e3) / 1e9
    traffic = profile_traffic(dominant, wl.name)
    measured = step_traffic(wl.name, passes, args.steps, carry)

    metric = "optimizer-step params/s + achieved HBM GB/s (% peak), " + (
        "7B-shaped Adafactor" if wl.name == "adafactor_llama7b" else wl.name)
    out = {
        "metric": metric,
        "value": value,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "step_ms": {"min": min(step_ms), "median": sorted(step_ms)[len(step_ms) // 2], "max": max(step_ms)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "optimizer": wl.optimizer, "tensors": len(wl.specs), "layout": args.layout,
                   "params": numel, "grad_dtype": str(wl.grad_dtype).replace("torch.", ""),
                   "param_dtype": str(wl.param_dtype).replace("torch.", ""),
                   "exp_avg_dtype": str(wl.state_dtype).replace("torch.", ""),
                   "param_sumsq": "carry" if carry else "read",
                   "hparams": {k: (list(v) if isinstance(v, tuple) else v) for k, v in hp.items()}},
        "hbm": {"step_bytes": ab["step"], "achieved": step_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": step_gbps / HBM_PEAK_GBPS,
                "measured_step_bytes": measured,
                "measured_achieved": None if measured is None else measured / (ms_step / 1e3) / 1e9,
                "measured_frac": None if measured is None else measured / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBPS},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "bytes_per_launch": ab[dominant], "avg_ms": avg_ms},
        "passes_ms_per_step": {k: v["ms"] / args.steps for k, v in passes.items()},
    }
    if read is not None:
        out["read_param_sumsq"] = read
    if placement is not None:
        placement["apply_ms"] = avg_ms
        out["placement"] = placement
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
