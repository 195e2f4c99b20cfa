#!/usr/bin/env python3
"""Benchmark of the DP-SGD private-gradient step (ghost per-record norms -> clip -> clipped sum ->
Gaussian noise) on one MI355X, through the library's C ABI.

Default workload (the largest configuration that fits one GPU): the 7B-shaped rank-16 LoRA on
q, k, v, o of 32 blocks (256 linear layers, 16.8M trainables), 256 records x 512 tokens, bf16
activations and output gradients ~ N(0, 0.02) with Student-t(3) records 0, 100, 200, C = 0.5,
sigma = 0.8: 276 GB of inputs, all resident in HBM before timing.  --workload N (1-5) runs the
other configurations; --sum gemm replaces the default clipped-sum strategy (per-record gradient
blocks kept by the norm pass where that moves fewer bytes) by the GEMM A^T diag(c) G that
re-reads A and G.  Inputs are synthetic (the seeded generator, written straight into HBM).  A step
is one pass of the whole path over one logical batch (every physical batch, the noise once).

Prints one JSON line: records/s over --steps timed steps, the roofline of the dominant kernel
(its average duration from HIP events recorded around back-to-back launches of it on the stream
it runs on), every phase's rate, and the CPU oracle timed on the host's cores on a bounded sample
of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "records/sec per DP-SGD clip+noise step; % MFMA / HBM roofline"
HBM_PEAK_GBS = 8000.0
DESCENT_LR, DESCENT_L = 0.01, 1.0   # --descent: the sensitivity paper's release audit settings
MFMA_PEAK_TFLOPS = {0: 157.3, 1: 2500.0}   # dense fp32 / bf16 MFMA
DEFAULT_WORKLOAD = 3
N_SETS = 4   # distinct input batches a single-batch workload's timed steps cycle through
MAX_LAUNCH_LAYERS = 48   # layers per launch of the norm and tile-engine sum kernels (library)
MAX_DENSE_LAYERS = 32    # per launch of the dense clipped sum (its kernel-argument limit)
SUM_POLICIES = {"auto": 0, "gemm": 1, "stored": 2}
SUM_NAMES = {0: "auto", 1: "gemm", 2: "stored"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_work(w, plan, dp):
    """Algorithmic HBM bytes and flops of each phase for one physical batch of w: what the method
    must move or compute.  norms: one read of every A and G (the per-record gradients the ghost
    norms avoid are not counted); clipped_sum of the GEMM layers: one read of their A and G and the
    fp32 output; noise: read and write of every parameter (8 bytes).  The per-record gradient
    blocks that the STORED strategy writes during the norms and reads back in the sum are an
    implementation choice, reported apart ("stored_write" / "stored_read")."""
    e = 4 if w.dtype == 0 else 2
    B, T = w.B, w.T
    work = {"norms": [0, 0], "clipped_sum": [0, 0], "noise": [8 * w.n_params, 0],
            "stored_write": 0, "stored_read": 0}
    for l, (di, do) in enumerate(w.layers):
        path, sm = plan.layer_info(l)
        in_bytes = B * T * (di + do) * e
        work["norms"][0] += in_bytes
        work["norms"][1] += 2 * B * T * T * (di + do) if path == dp.PATH_GRAM else 2 * B * T * di * do
        if sm == dp.SUM_STORED:
            work["stored_write"] += B * di * do * 4
            work["stored_read"] += B * di * do * 4
        else:
            work["clipped_sum"][0] += in_bytes + di * do * 4
            work["clipped_sum"][1] += 2 * B * T * di * do
    return work


def norm_launches(w, plan, dp):
    """Launches of the norm kernels per physical batch: direct-path layers go out in groups of
    equal MFMA row blocks and strategy, Gram-path layers in their own, at most 48 layers a launch
    (the library's kernel-argument limit), split into near-equal launches."""
    groups = {}
    for l, (di, do) in enumerate(w.layers):
        path, sm = plan.layer_info(l)
        key = ("gram",) if path == dp.PATH_GRAM else ("direct", min(di, do) <= 16, sm)
        groups[key] = groups.get(key, 0) + 1
    return sum(-(-n // MAX_LAUNCH_LAYERS) for n in groups.values())


def sum_launches(w, plan, dp):
    """Launches of the GEMM clipped-sum kernels per physical batch: bf16 layers with both
    dimensions above 16 on the dense MFMA kernel, at most 32 layers a launch; the other GEMM layers
    on the tile engine in groups of equal MFMA row blocks, at most 48 layers a launch (each followed
    by its split reduce when the records are split)."""
    groups = {}
    for l, (di, do) in enumerate(w.layers):
        if plan.layer_info(l)[1] != dp.SUM_GEMM:
            continue
        key = "dense" if (w.dtype == dp.DTYPE_BF16 and min(di, do) > 16) else ("tile", min(di, do) <= 16)
        groups[key] = groups.get(key, 0) + 1
    return sum(-(-n // (MAX_DENSE_LAYERS if k == "dense" else MAX_LAUNCH_LAYERS))
               for k, n in groups.items())


def device_inputs(w, datagen, torch, dev, first, n):
    """Fill A and G of every layer for records [first, first+n) directly in HBM."""
    import numpy as np
    As, Gs = [], []
    tdt = torch.float32 if w.dtype == 0 else torch.int16
    for l, (di, do) in enumerate(w.layers):
        for tensor, d, lst in ((0, di, As), (1, do, Gs)):
            scale, heavy = datagen.record_params(w, l, tensor, first, n)
            ds = torch.from_numpy(scale).to(dev)
            dh = torch.from_numpy(heavy.astype(np.uint8)).to(dev)
            buf = torch.empty((n, w.T, d), dtype=tdt, device=dev)
            datagen.device_fill(w, l, tensor, buf.data_ptr(), first, n, ds.data_ptr(), dh.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
            lst.append(buf)
    torch.cuda.synchronize()
    return As, Gs


# sources the ghost-norm kernels and their launch configuration (layer grouping, store mode) come
# from: a stored HBM-traffic record applies only while these are unchanged
NORM_KERNEL_SOURCES = ("ghost_norm.hip", "tile_direct.h", "device_common.h", "internal.h", "dpsgd_api.cpp")
# the same for the clipped-sum kernels (tile engine, dense MFMA kernels, split reduce, split counts)
SUM_KERNEL_SOURCES = ("clipped_sum.hip", "clipped_sum_dense.hip", "tile_direct.h", "device_common.h",
                      "internal.h", "dpsgd_api.cpp")
# the same for the INT8 forward's kernels
I8_KERNEL_SOURCES = ("int8_forward.hip", "int8.h", "device_common.h", "internal.h")
PHASE_SOURCES = {"norms": NORM_KERNEL_SOURCES, "clipped_sum": SUM_KERNEL_SOURCES}


def kernel_src_hash(names=NORM_KERNEL_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "differentially_private_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_record_path(workload_name, phase, sum_name):
    return os.path.join(ROOT, "profiles", f"traffic_{phase}_{workload_name}_{sum_name}.json")


def stored_traffic(workload_name, phase, sum_name):
    """HBM-side bytes per launch of the dominant kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE
    (each scaled by what the same counter reads for a plain copy of known size); None when no
    record exists or the kernel sources differ from the ones it was measured on."""
    path = traffic_record_path(workload_name, phase, sum_name)
    if not os.path.exists(path):
        return None
    tr = json.load(open(path))
    if tr.get("src_hash") != kernel_src_hash(PHASE_SOURCES[phase]):
        return None
    return tr.get("bytes_per_launch")


def stored_i8_traffic():
    """HBM-side bytes per k_i8_gemm launch (mean over the OPT-125M layer shapes) from rocprofv3
    FETCH_SIZE / WRITE_SIZE, scaled by a plain copy of known size; None once the kernel sources
    differ from the ones it was measured on."""
    path = os.path.join(ROOT, "profiles", "int8_gemm_traffic.json")
    if not os.path.exists(path):
        return None
    tr = json.load(open(path))
    return tr.get("bytes_per_launch") if tr.get("src_hash") == kernel_src_hash(I8_KERNEL_SOURCES) else None


def cpu_baseline(w, seconds):
    """The oracle as it stands (plain C, fp64, OpenMP over gradient rows), timed on the host's
    threads on a bounded sample of the workload: whole steps when one takes well under `seconds`,
    else the first m records of the logical batch over every layer (m from a one-record probe, so
    that the timed run takes about `seconds`), the step's noise over every parameter included.
    Input generation is excluded.  A one-thread figure follows on a shorter sample."""
    import datagen
    import oracle
    cores = oracle.num_threads()

    def inputs(m, layers):
        return ([datagen.host_tensor(w, l, 0, 0, m) for l in layers],
                [datagen.host_tensor(w, l, 1, 0, m) for l in layers])

    def timed(As, Gs, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.step(As, Gs, w.C, w.sigma, w.noise_seed, 0)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return reps, el

    layers = range(w.n_layers)
    As, Gs = inputs(1, layers)
    t0 = time.perf_counter()
    oracle.step(As, Gs, w.C, w.sigma, w.noise_seed, 0)
    t1 = time.perf_counter() - t0
    n_all = min(w.B, w.logical_B)
    if t1 * n_all <= seconds / 4:
        m = n_all                    # whole (physical) batches, repeated
    else:
        m = max(1, min(n_all, int(seconds / t1)))
    if m > 1:
        As, Gs = inputs(m, layers)
    reps, el = timed(As, Gs, seconds if m == n_all else 0.0)
    value = m * reps / el
    sample = (f"{reps} x {m} records ({'the whole batch' if m == n_all else 'the first of the batch'}) "
              f"over all {w.n_layers} layers: norms, clip, clipped sum, noise over all {w.n_params} "
              f"parameters; input generation excluded; {el:.1f} s wall")
    # one thread: one record, over every k-th layer when a whole record would take long; the rate
    # is scaled by the share of the per-record work the sampled layers hold
    oracle.set_num_threads(1)
    try:
        per_layer = [2 * w.T * di * do for di, do in w.layers]
        est1 = t1 * cores
        k = max(1, int(math.ceil(est1 / (seconds / 3))))
        sub = list(range(0, w.n_layers, k))
        share = sum(per_layer[l] for l in sub) / sum(per_layer)
        As1, Gs1 = inputs(1, sub)
        reps1, el1 = timed(As1, Gs1, seconds / 3 if k == 1 else 0.0)
        single = {"value": share * reps1 / el1, "unit": "records/s", "cores": 1,
                  "sample": f"{reps1} x 1 record over {len(sub)} of {w.n_layers} layers "
                            f"({share:.3f} of a record's work; the rate is scaled by it), "
                            f"{el1:.1f} s wall"}
    finally:
        oracle.set_num_threads(cores)
    return {"value": value, "unit": "records/s", "cores": cores, "kind": "oracle", "sample": sample,
            "single_thread": single}


def phase_roofline(phase, nbytes, nflops, ms, dtype):
    """Rate of one phase against the roofline that binds it: MFMA (the dtype's dense peak) when its
    arithmetic intensity is above the ridge, else HBM."""
    if ms <= 0:
        return None
    s = ms * 1e-3
    mfma_peak = MFMA_PEAK_TFLOPS[dtype]
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    r = {"ms": ms, "algorithmic_bytes": nbytes, "flops": nflops,
         "GBps": nbytes / s / 1e9, "hbm_frac": nbytes / s / 1e9 / HBM_PEAK_GBS}
    if nflops:
        r["TFLOPs"] = nflops / s / 1e12
        r["mfma_frac"] = r["TFLOPs"] / mfma_peak
    r["bound"] = "mfma" if nflops and nflops / max(nbytes, 1) > ridge else "hbm"
    return r


KERNEL_NAMES = {
    "norms": {"direct": "k_norm_direct (ghost_norm, direct path)",
              "gram": "k_norm_gram_rec / k_norm_gram (ghost_norm, Gram path)"},
    "clipped_sum": {"dense": "k_sum_dense_dma (clipped_sum, dense MFMA GEMM A^T diag(c) G)",
                    "tile": "k_sum_direct (clipped_sum, GEMM A^T diag(c) G on the tile engine) + split reduce"},
}


def kernel_name(phase, w, plan, dp):
    paths = {plan.layer_info(l)[0] for l in range(w.n_layers)}
    if phase == "norms":
        return KERNEL_NAMES["norms"]["gram" if paths == {dp.PATH_GRAM} else "direct"]
    dense = w.dtype == 1 and all(min(di, do) > 16 for di, do in w.layers)
    return KERNEL_NAMES["clipped_sum"]["dense" if dense else "tile"]


def step_line(args, w, torch, dev, dp, datagen):
    """One JSON line for workload w: whole logical steps timed between HIP events (inputs resident
    in HBM; single-batch workloads that fit four times cycle through four distinct batches so that
    no step re-reads inputs the last-level cache kept), then every phase alone, K back-to-back
    launches between two HIP events on the stream they run on, with the C calls' arguments
    marshalled once so that the host does not pace the GPU."""
    import ctypes
    import numpy as np
    L = w.n_layers
    sum_policy = SUM_POLICIES[args.sum]
    plan = dp.Plan(w.layers, w.dtype, w.B, w.T, dp.PATH_AUTO, sum_policy)
    ws = plan.workspace(dev)
    out = [torch.empty(di * do, dtype=torch.float32, device=dev) for di, do in w.layers]
    theta = ([torch.zeros(di * do, dtype=torch.float32, device=dev) for di, do in w.layers]
             if args.descent else None)
    in_bytes = w.input_bytes_per_batch()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    log(f"{w.name}: filling {w.n_phys} physical batch(es) of {in_bytes / 1e9:.2f} GB in HBM")
    batches = [device_inputs(w, datagen, torch, dev, p * w.B, w.B) for p in range(w.n_phys)]
    cycle = [batches]
    free = torch.cuda.mem_get_info()[0]
    if w.n_phys == 1 and N_SETS * in_bytes < free // 2:
        cycle += [[device_inputs(w, datagen, torch, dev, k * w.B, w.B)] for k in range(1, N_SETS)]
    n_cycle = len(cycle)
    lib = dp.load()

    # whole logical steps: the physical batches with NO_NOISE (ACCUMULATE after the first), then
    # the noise once; a single physical batch is one dpsgd_step
    calls = []
    for bs in cycle:
        cs = []
        for p, (As, Gs) in enumerate(bs):
            flags = (dp.NO_NOISE if w.n_phys > 1 else 0) | (dp.ACCUMULATE if p else 0)
            last = w.n_phys == 1
            cs.append(dp.StepCall(plan, As, Gs, out, ws, w.C, w.sigma, w.noise_seed, 0, flags=flags,
                                  params=theta if last else None, lr=DESCENT_LR, normalizer=DESCENT_L))
        calls.append(cs)
    arr_o = dp._ptr_array(out)
    arr_t = dp._ptr_array(theta)
    wsp = ws.data_ptr()
    descent = args.descent

    def noise_call(st=None):
        st = sp if st is None else st
        if descent:
            rc = lib.dpsgd_noise_descent(plan.handle, arr_o, arr_t, w.C, w.sigma, w.noise_seed, 0,
                                         DESCENT_LR, DESCENT_L, wsp, st)
        else:
            rc = lib.dpsgd_noise(plan.handle, arr_o, w.C, w.sigma, w.noise_seed, 0, wsp, st)
        if rc:
            dp._check(rc)

    def step(i):
        for c in calls[i % len(calls)]:
            c()
        if w.n_phys > 1:
            noise_call()

    for i in range(max(args.warmup, len(calls))):
        step(i)
    torch.cuda.synchronize()
    assert dp.status(plan, ws) == dp.OK
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(fn, reps):
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1), (time.perf_counter() - t0) * 1e3

    gpu_ms, wall_ms = timed(step, args.steps)
    ms = max(gpu_ms, wall_ms) / args.steps
    assert dp.status(plan, ws) == dp.OK

    # each phase alone (norms and the GEMM clipped sum cycle through the same batches as the steps)
    flat_batches = [b for bs in cycle for b in bs]
    marsh = [(dp._ptr_array(A), dp._ptr_array(G)) for A, G in flat_batches]

    def checked(rc):
        if rc:
            dp._check(rc)

    def norms_fn(i):
        a, g = marsh[i % len(marsh)]
        checked(lib.dpsgd_norms(plan.handle, w.B, 0, L, a, g, wsp, sp))

    def clip_fn(i):
        checked(lib.dpsgd_clip(plan.handle, w.B, w.C, 0, wsp, None, None, sp))

    def sum_fn(i):
        a, g = marsh[i % len(marsh)]
        checked(lib.dpsgd_clipped_sum(plan.handle, w.B, 0, L, a, g, None, arr_o, 0, wsp, sp))

    reps = args.steps
    phase_ms = {}
    phase_ms["norms"] = timed(norms_fn, reps)[0] / reps
    phase_ms["clip"] = timed(clip_fn, reps)[0] / reps
    work = algorithmic_work(w, plan, dp)
    has_gemm = work["clipped_sum"][0] > 0
    has_stored = work["stored_write"] > 0
    if has_gemm:
        norms_fn(0)   # the stored blocks (if any) and factors of batch 0 for the sum phase
        clip_fn(0)
        phase_ms["clipped_sum"] = timed(sum_fn, reps)[0] / reps
    phase_ms["noise"] = graph_timed(torch, stream, lambda st: noise_call(st), reps)
    phase_ms["rest_of_step"] = max(ms - phase_ms["norms"] * w.n_phys, 0.0)
    torch.cuda.synchronize()
    assert dp.status(plan, ws) == dp.OK

    # per-phase rooflines; the dominant kernel: the GEMM clipped sum when the plan has one (the
    # MFMA GEMM A^T diag(c) G), else the norm kernel
    kernels = {}
    for ph in ("norms", "clipped_sum", "noise"):
        if ph in phase_ms:
            nb, nf = work[ph]
            kernels[ph] = phase_roofline(ph, nb, nf, phase_ms[ph], w.dtype)
    kernels["norms"]["kernel"] = kernel_name("norms", w, plan, dp)
    kernels["norms"]["launches"] = norm_launches(w, plan, dp)
    if has_stored:
        kernels["norms"]["stored_bytes_written"] = work["stored_write"]
        kernels["norms"]["GBps_incl_stored"] = (work["norms"][0] + work["stored_write"]) / (
            phase_ms["norms"] * 1e-3) / 1e9
    if "clipped_sum" in kernels:
        kernels["clipped_sum"]["kernel"] = kernel_name("clipped_sum", w, plan, dp)
        kernels["clipped_sum"]["launches"] = sum_launches(w, plan, dp)
    dom = "clipped_sum" if has_gemm else "norms"
    k = kernels[dom]
    if k["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": k["TFLOPs"], "peak": MFMA_PEAK_TFLOPS[w.dtype],
                "unit": "TFLOP/s", "frac": k["mfma_frac"]}
    else:
        roof = {"bound": "hbm", "achieved": k["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": k["hbm_frac"]}
    launches = k.get("launches", 1)
    roof["traffic"] = stored_traffic(w.name, dom, SUM_NAMES[sum_policy])
    roof["kernel"] = k["kernel"]
    roof["phase"] = dom
    roof["launches_per_phase"] = launches
    roof["algorithmic_bytes_per_launch"] = work[dom][0] / launches
    roof["algorithmic_flops_per_launch"] = work[dom][1] / launches
    roof["avg_ms"] = phase_ms[dom] / launches
    if roof["unit"] == "GB/s":
        try:
            roof["achievable"] = achievable_hbm(torch, dev, dp)
            roof["frac_of_achievable"] = roof["achieved"] / roof["achievable"]["read_gbs"]
            ab = work[dom][0]
            if N_SETS * ab < torch.cuda.mem_get_info()[0] // 2:
                roof["achievable_at_size"] = achievable_hbm_at(torch, dev, dp, ab)
            else:
                roof["achievable_at_size"] = achievable_hbm_tensors(torch, dp, batches[0])
            roof["frac_of_achievable_at_size"] = roof["achieved"] / roof["achievable_at_size"]["read_gbs"]
        except torch.cuda.OutOfMemoryError:
            pass
    if has_stored:
        roof["stored_gradient_blocks"] = {
            "bytes_written": work["stored_write"], "bytes_read": work["stored_read"],
            "note": "per-record gradient blocks [d_in x d_out] fp32 that the norm kernel writes "
                    "and the fused sum + noise kernel reads back instead of re-reading A and G "
                    "(the STORED clipped-sum strategy); not algorithmic bytes"}

    cpu = None
    if not args.no_cpu_baseline:
        del batches, cycle, calls, flat_batches, marsh
        torch.cuda.empty_cache()
        cpu = cpu_baseline(w, args.cpu_seconds)

    line = {"metric": METRIC, "value": w.logical_B / (ms * 1e-3), "unit": "records/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": datagen.configs.DTYPE_NAMES[w.dtype],
            "data": "synthetic",
            "config": {"workload": w.name, "layers": L, "params": w.n_params,
                       "records_per_step": w.logical_B, "physical_batches": w.n_phys,
                       "tokens": w.T, "C": w.C, "sigma": w.sigma,
                       "sum_policy": args.sum,
                       "sum_strategy": ("stored" if has_stored and not has_gemm else
                                        "gemm" if has_gemm and not has_stored else "mixed"),
                       "parallelism": "single GPU",
                       "descent": {"lr": DESCENT_LR, "normalizer": DESCENT_L} if args.descent else None},
            "roofline": roof, "cpu_baseline": cpu,
            "phases_ms": phase_ms, "kernels": kernels,
            "gpu_ms_per_step": gpu_ms / args.steps, "wall_ms_per_step": wall_ms / args.steps,
            "input_batches": n_cycle}
    print(json.dumps(line), flush=True)
    if args.manifest:
        man = {"git": subprocess.run(["git", "rev-parse", "HEAD"], cwd=ROOT, capture_output=True,
                                     text=True).stdout.strip() or None,
               "torch": torch.__version__, "hip": torch.version.hip,
               "device": torch.cuda.get_device_name(0),
               "cu": torch.cuda.get_device_properties(0).multi_processor_count,
               "host_cpu": platform.processor(), "nproc": os.cpu_count(),
               "plan_paths": [plan.layer_info(l) for l in range(L)], "workload": w.name}
        with open(args.manifest, "w") as f:
            json.dump(man, f, indent=1)


def graph_timed(torch, stream, call, reps):
    """Milliseconds per call of `call(stream_handle)`: `reps` calls captured once into a HIP graph
    (on a capture stream of default priority), the graph replayed between two HIP events on
    `stream`, so that the host's per-call cost does not pace a phase of a few microseconds."""
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        for _ in range(reps):
            call(cap.cuda_stream)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / reps


def kernel_mode(args, w, torch, dev, dp, datagen):
    """Only the dominant kernel's phase (or --phase), --warmup + --steps times over the workload's
    first physical batch: the command the HBM byte counters are collected on."""
    sum_policy = SUM_POLICIES[args.sum]
    plan = dp.Plan(w.layers, w.dtype, w.B, w.T, dp.PATH_AUTO, sum_policy)
    ws = plan.workspace(dev)
    out = [torch.empty(di * do, dtype=torch.float32, device=dev) for di, do in w.layers]
    As, Gs = device_inputs(w, datagen, torch, dev, 0, w.B)
    work = algorithmic_work(w, plan, dp)
    phase = args.phase or ("clipped_sum" if work["clipped_sum"][0] > 0 else "norms")
    L = w.n_layers
    if phase == "clipped_sum":
        dp.norms(plan, w.B, 0, L, As, Gs, ws)
        dp.clip(plan, w.B, w.C, ws)
    for _ in range(args.warmup + args.steps):
        if phase == "norms":
            dp.norms(plan, w.B, 0, L, As, Gs, ws)
        elif phase == "clipped_sum":
            dp.clipped_sum(plan, w.B, 0, L, As, Gs, None, out, ws)
        else:
            dp.noise(plan, out, w.C, w.sigma, w.noise_seed, 0, ws=ws)
    torch.cuda.synchronize()
    launches = (norm_launches(w, plan, dp) if phase == "norms" else
                sum_launches(w, plan, dp) if phase == "clipped_sum" else None)
    print(json.dumps({"mode": "kernel", "workload": w.name, "phase": phase, "sum_policy": args.sum,
                      "calls": args.warmup + args.steps, "launches_per_call": launches,
                      "algorithmic_bytes_per_call": work[phase][0],
                      "src_hash": kernel_src_hash(PHASE_SOURCES.get(phase, NORM_KERNEL_SOURCES))}),
          flush=True)


def achievable_hbm_tensors(torch, dp, batch, reps=3):
    """The streaming read (dpsgd_hbm_read) over the workload's own input tensors, one launch per
    tensor in turn, best of `reps` passes timed with HIP events: the read rate of the same bytes
    when the workload is too large to copy for distinct buffers."""
    As, Gs = batch
    ts = [t for t in As + Gs if (t.numel() * t.element_size()) % 16 == 0]
    nb = sum(t.numel() * t.element_size() for t in ts)
    sink = torch.empty(dp.HBM_READ_SINK_WORDS, dtype=torch.int32, device=ts[0].device)
    best = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for t in ts:
            dp.hbm_read(t.data_ptr(), t.numel() * t.element_size(), sink.data_ptr())
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b) * 1e-3)
    return {"read_gbs": nb / best / 1e9, "bytes": nb, "us": best * 1e6,
            "how": f"dpsgd_hbm_read over the workload's {len(ts)} input tensors in turn "
                   f"({nb / 1e9:.1f} GB), best of {reps} passes"}


def sample_line(args, torch, dev, dp):
    """Poisson sampling of 2^27 records at q = 0.01 (the page's accountant example rate): K draws
    (one per step index) between HIP events; the oracle's sampler on a 2^22-record sample for the
    host rate; the library accountant's host time for the page's 300-step epsilon."""
    import time
    n, q = 1 << 27, 0.01
    idx = torch.empty(n, dtype=torch.int64, device=dev)
    cnt = torch.empty(1, dtype=torch.int64, device=dev)
    ws = torch.empty(dp.poisson_ws_bytes(n) // 8, dtype=torch.int64, device=dev)
    mask = torch.empty(n, dtype=torch.uint8, device=dev)
    for s in range(args.warmup):
        dp.poisson_sample(1, s, q, n, idx, cnt, ws, mask=mask)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for s in range(args.steps):
        dp.poisson_sample(1, s, q, n, idx, cnt, ws, mask=mask)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    sel = int(cnt.item())
    from oracle import accountant as acc       # host baseline only
    m = 1 << 22
    t0 = time.perf_counter()
    acc.poisson_sample(1, 0, q, m)
    cpu_rate = m / (time.perf_counter() - t0)
    t0 = time.perf_counter()
    per = dp.rdp_sampled_gaussian(q, 1.0, acc.DEFAULT_ORDERS)
    eps, order = dp.rdp_to_epsilon(acc.DEFAULT_ORDERS, [300 * r for r in per], 1e-5)
    host_ms = (time.perf_counter() - t0) * 1e3
    line = {"metric": "records/sec Poisson-sampled (inclusion mask + index list)", "value": n / (ms * 1e-3),
            "unit": "records/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "u32", "data": "synthetic",
            "config": {"workload": "poisson_sampler", "population": n, "q": q, "selected_last": sel},
            "bytes_written_GBps": (n + 8 * sel) / (ms * 1e-3) / 1e9,
            "roofline": {"bound": "alu", "achieved": SAMPLE_OPS_PER_RECORD * n / (ms * 1e-3) / 1e12,
                         "peak": VALU_PEAK_TOPS, "unit": "T lane-ops/s",
                         "frac": SAMPLE_OPS_PER_RECORD * n / (ms * 1e-3) / 1e12 / VALU_PEAK_TOPS,
                         "traffic": None,
                         "kernel": "k_sample_count + k_sample_scan + k_sample_write (one draw)",
                         "algorithmic_ops_per_launch": SAMPLE_OPS_PER_RECORD * n, "avg_ms": ms,
                         "how": "Philox4x32-10 per 4 records: 10 rounds of two 32x32->64-bit products "
                                "and two XORs; one comparison per record; against the 32-bit VALU "
                                "lane-op rate, the draw's three launches timed together"},
            "cpu_baseline": {"value": cpu_rate, "unit": "records/s", "cores": 1, "kind": "oracle",
                             "sample": f"{m} records, one draw"},
            "accountant": {"epsilon_300_steps": eps, "order": order, "host_ms": host_ms}}
    print(json.dumps(line), flush=True)


def users_line(args, w, torch, dev, dp, datagen):
    """User-level clipping on workload 2's layers: 16 users, user u holding 1 + (u mod 4) of the
    generator's 128-token records, each user's rows concatenated (40 records, 5,120 token rows,
    at most 512 per user); one step clips each user's summed gradient."""
    import numpy as np
    recs = [1 + (u % 4) for u in range(16)]
    lens = [r * w.T for r in recs]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    n_users, T_max, n_rec = len(lens), max(lens), sum(recs)
    plan = dp.Plan(w.layers, w.dtype, n_users, T_max, segments=True)
    ws = plan.workspace(dev)
    dp.ws_segments(plan, ws, offs)
    As, Gs = device_inputs(w, datagen, torch, dev, 0, n_rec)          # records 0..39, contiguous
    As = [a.reshape(-1, a.shape[2]) for a in As]
    Gs = [g.reshape(-1, g.shape[2]) for g in Gs]
    out = [torch.empty(di * do, dtype=torch.float32, device=dev) for di, do in w.layers]
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    call = dp.StepCall(plan, As, Gs, out, ws, w.C, w.sigma, w.noise_seed, 0)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    assert dp.status(plan, ws) == dp.OK
    a, b = ev(), ev()
    a.record(stream)
    for _ in range(args.steps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    # the norm phase alone, its C call's arguments marshalled once so that the host does not pace it
    lib = dp.load()
    pa, pg, wsp, sp = dp._ptr_array(As), dp._ptr_array(Gs), ws.data_ptr(), stream.cuda_stream
    x0, x1 = ev(), ev()
    x0.record(stream)
    for _ in range(args.steps):
        rc = lib.dpsgd_norms(plan.handle, n_users, 0, w.n_layers, pa, pg, wsp, sp)
        if rc:
            dp._check(rc)
    x1.record(stream)
    torch.cuda.synchronize()
    norm_ms = x0.elapsed_time(x1) / args.steps
    rows = int(offs[-1])
    in_bytes = rows * sum(di + do for di, do in w.layers) * 4          # A and G read once
    gbs = in_bytes / (norm_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "traffic": stored_traffic(f"{w.name}_segments{n_users}", "norms", "users"),
            "kernel": "k_norm_direct (ghost_norm, direct path, segment plan)",
            "phase": "norms", "launches_per_phase": 1, "algorithmic_bytes_per_launch": in_bytes,
            "avg_ms": norm_ms,
            "stored_gradient_blocks": {"bytes_written": n_users * w.n_params * 4,
                                       "bytes_read": n_users * w.n_params * 4,
                                       "note": "each user's gradient block, written by the norm kernel "
                                               "and read back by the fused sum + noise kernel; not "
                                               "algorithmic bytes"}}
    line = {"metric": "users/sec per DP-SGD step with user-level clipping", "value": n_users / (ms * 1e-3),
            "unit": "users/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": datagen.configs.DTYPE_NAMES[w.dtype], "data": "synthetic",
            "config": {"workload": w.name + "_users", "users": n_users, "records": n_rec,
                       "token_rows": rows, "max_rows_per_user": T_max, "layers": w.n_layers,
                       "params": w.n_params, "parallelism": "single GPU"},
            "phases_ms": {"norms": norm_ms, "rest_of_step": ms - norm_ms},
            "roofline": roof,
            "cpu_baseline": None if args.no_cpu_baseline else users_cpu_baseline(w, recs, args.cpu_seconds)}
    print(json.dumps(line), flush=True)


def users_cpu_baseline(w, recs, seconds):
    """The oracle on the same users: each user's records' rows concatenated into one record of its own
    length (the oracle's gradient rows sum over them), one oracle step per user, all layers, repeated
    for about `seconds` on the host's threads; users/s."""
    import datagen
    import oracle
    cores = oracle.num_threads()
    users, first = [], 0
    for r in recs:
        A = [datagen.host_tensor(w, l, 0, first, r).reshape(1, r * w.T, -1) for l in range(w.n_layers)]
        G = [datagen.host_tensor(w, l, 1, first, r).reshape(1, r * w.T, -1) for l in range(w.n_layers)]
        users.append((A, G))
        first += r
    reps, t0 = 0, time.perf_counter()
    while True:
        for A, G in users:
            oracle.step(A, G, w.C, w.sigma, w.noise_seed, 0)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": len(recs) * reps / el, "unit": "users/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} x all {len(recs)} users ({sum(recs)} records of {w.T} tokens) over all "
                      f"{w.n_layers} layers, one oracle step per user on its concatenated rows (its noise "
                      f"over all {w.n_params} parameters included); input generation excluded; "
                      f"{el:.1f} s wall"}


I8_PEAK_TOPS = 5000.0   # dense INT8 MFMA, ops/s x 1e-12
# 32-bit VALU lane operations per second x 1e-12: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (the vendor's
# 157.3 TFLOP/s fp32 vector figure is this rate x 2 for a fused multiply-add x 2 for packed pairs)
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# the sampler's algorithmic 32-bit operations per record: Philox4x32-10 serves four records with
# 10 rounds of two 32x32->64-bit products and two XORs (40 / 4), plus one comparison
SAMPLE_OPS_PER_RECORD = 11


def int8_model(torch, dev, dp, seed=0):
    """The frozen OPT-125M backbone's 72 INT8 layers (12 blocks x q, k, v, out: 768 -> 768, fc1:
    768 -> 3072, fc2: 3072 -> 768) over one physical batch of B = 16 records x T = 256 tokens.
    q, k and v read the same input: their frozen weights are stacked into one 2304 x 768 weight
    (row-wise codes and scales are per output feature, so every output is the one the separate
    layers give), leaving four INT8 forwards per block.  Synthetic activations with three shared
    outlier columns and record-owned ones (datagen.int8), weights ~ N(0, 0.02)."""
    import numpy as np
    from datagen import int8 as gen
    B, T, H, F = 16, 256, 768, 3072
    offsets = gen.lengths_offsets([T] * B)
    n = int(offsets[-1])
    layers = []
    for blk in range(12):
        for j, (K, N, n_proj) in enumerate(((H, H, 3), (H, H, 1), (H, F, 1), (F, H, 1))):
            A, _, _, _ = gen.activations(1000 * seed + 10 * blk + j, [T] * B, K)
            W = np.concatenate([gen.weights(100 * blk + 10 * j + p, N, K) for p in range(n_proj)])
            W = torch.from_numpy(W).to(dev)
            Nt = N * n_proj
            wq = torch.empty((Nt, dp.i8_pitch(K)), dtype=torch.int8, device=dev)
            sw = torch.empty(Nt, dtype=torch.float32, device=dev)
            dp.i8_quantize_weight(W, Nt, K, wq, sw)
            del W
            Y = torch.empty((n, Nt), dtype=torch.float16, device=dev)
            layers.append({"A": torch.from_numpy(A).to(dev), "K": K, "N": Nt, "wq": wq, "sw": sw,
                           "Y": Y, "projections": n_proj})
    torch.cuda.synchronize()
    return {"B": B, "T": T, "n": n, "offsets": offsets, "layers": layers}


def int8_line(args, torch, dev, dp):
    """Record-owned LLM.int8 forward of the OPT-125M backbone (72 INT8 layers, one physical batch
    of 16 x 256 tokens per step): eager and HIP-graph timings of the whole forward, the GEMM's
    roofline from HIP events around back-to-back dpsgd_i8_matmul calls of each layer, the batched
    LLM.int8 variant (one record spanning the batch: the same kernels with the batch-wide union)
    for comparison, and the oracle's rate on one layer of each shape."""
    import ctypes
    import numpy as np
    m = int8_model(torch, dev, dp)
    n, B = m["n"], m["B"]
    plan = dp.I8Plan(n, B, 3072)
    ws = plan.workspace(dev)
    ws_b = plan.workspace(dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    lib = dp.load()
    tau = ctypes.c_float(6.0)

    def marshal(w, n_rec, st):
        """The block's four INT8 forwards (qkv, out, fc1, fc2) as C calls."""
        return [(lib.dpsgd_i8_forward, (plan.handle, w.data_ptr(), n, n_rec, L["A"].data_ptr(),
                                        L["K"], L["wq"].data_ptr(), L["sw"].data_ptr(), L["N"],
                                        tau, L["Y"].data_ptr(), st)) for L in m["layers"]]

    calls = marshal(ws, B, sp)
    calls_b = marshal(ws_b, 1, sp)
    dp.i8_set_records(plan, ws, m["offsets"], stream)
    dp.i8_set_records(plan, ws_b, [0, n], stream)

    def forward(cs):
        for f, c in cs:
            rc = f(*c)
            if rc:
                dp._check(rc)

    for _ in range(args.warmup):
        forward(calls)
        forward(calls_b)
    torch.cuda.synchronize()

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return max(e0.elapsed_time(e1), (time.perf_counter() - t0) * 1e3) / reps

    eager_ms = timed(lambda: (dp.i8_set_records(plan, ws, m["offsets"], stream), forward(calls)),
                     args.steps)
    batched_eager_ms = timed(lambda: forward(calls_b), args.steps)

    # the same forward captured once into a HIP graph (record offsets set outside it)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        forward(marshal(ws, B, torch.cuda.current_stream().cuda_stream))
    gb = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gb):
        forward(marshal(ws_b, 1, torch.cuda.current_stream().cuda_stream))
    for _ in range(3):
        g.replay()
        gb.replay()
    graph_ms = timed(g.replay, args.steps)
    batched_graph_ms = timed(gb.replay, args.steps)

    # dominant kernel: the INT8 GEMM of every layer, timed like every other phase: back-to-back
    # dpsgd_i8_matmul calls of one layer between two HIP events on the stream they run on (the
    # routing kernels of that layer run untimed before them).  Inside the forward the same GEMMs
    # run longer: by then the other layers' weights have evicted theirs from the L2.
    ops = 0
    gemm_ms = 0.0
    per = max(3, args.steps // 5)
    launches = 0
    abytes = 0   # codes + weight codes read, fp16 outputs written (outlier corrections aside)
    for L in m["layers"]:
        dp.i8_route(plan, ws, n, B, L["A"], L["K"], 6.0, stream)
        mm = (plan, ws, n, B, L["A"], L["K"], L["wq"], L["sw"], L["N"], L["Y"], stream)
        dp.i8_matmul(*mm)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(per):
            dp.i8_matmul(*mm)
        e1.record(stream)
        torch.cuda.synchronize()
        gemm_ms += e0.elapsed_time(e1)
        ops += per * 2 * n * L["K"] * L["N"]
        abytes += per * ((n + L["N"]) * dp.i8_pitch(L["K"]) + 2 * n * L["N"])
        launches += per
    avg_ms = gemm_ms / launches
    achieved = ops / (gemm_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": achieved, "peak": I8_PEAK_TOPS, "unit": "TOP/s",
            "frac": achieved / I8_PEAK_TOPS, "traffic": stored_i8_traffic(),
            "kernel": "k_i8_gemm (INT8 MFMA, dequantisation + record-owned FP16 correction)",
            "algorithmic_ops_per_launch": ops / launches, "algorithmic_bytes_per_launch": abytes / launches,
            "avg_ms": avg_ms, "launches": launches,
            "timing": "back-to-back launches of each layer's GEMM between two HIP events"}

    # the same kernels on one 7B-shaped frozen projection (4096 -> 4096) over 16 records x 512
    # tokens, where the INT8 product is large enough for the GEMM's MFMA efficiency to show
    from datagen import int8 as gen
    lens7, K7, N7 = [512] * 16, 4096, 4096
    A7, off7, _, _ = gen.activations(77, lens7, K7)
    n7 = int(off7[-1])
    dA7 = torch.from_numpy(A7).to(dev)
    W7 = torch.from_numpy(gen.weights(77, N7, K7)).to(dev)
    wq7 = torch.empty((N7, dp.i8_pitch(K7)), dtype=torch.int8, device=dev)
    sw7 = torch.empty(N7, dtype=torch.float32, device=dev)
    dp.i8_quantize_weight(W7, N7, K7, wq7, sw7)
    Y7 = torch.empty((n7, N7), dtype=torch.float16, device=dev)
    plan7 = dp.I8Plan(n7, len(lens7), K7)
    ws7 = plan7.workspace(dev)
    dp.i8_set_records(plan7, ws7, off7, stream)
    for _ in range(3):
        dp.i8_forward(plan7, ws7, n7, len(lens7), dA7, K7, wq7, sw7, N7, 6.0, Y7, stream)
    g7_ms, f7_ms = 0.0, 0.0
    reps7 = max(3, args.steps // 5)
    for _ in range(reps7):
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        dp.i8_route(plan7, ws7, n7, len(lens7), dA7, K7, 6.0, stream)
        e1.record(stream)
        dp.i8_matmul(plan7, ws7, n7, len(lens7), dA7, K7, wq7, sw7, N7, Y7, stream)
        e2.record(stream)
        torch.cuda.synchronize()
        f7_ms += e0.elapsed_time(e2)
        g7_ms += e1.elapsed_time(e2)
    ops7 = 2 * n7 * K7 * N7
    large = {"shape": f"{n7} x {K7} -> {N7} (16 records x 512 tokens)", "forward_ms": f7_ms / reps7,
             "gemm_ms": g7_ms / reps7, "gemm_TOPs": ops7 / (g7_ms / reps7 * 1e-3) / 1e12,
             "gemm_frac": ops7 / (g7_ms / reps7 * 1e-3) / 1e12 / I8_PEAK_TOPS}
    del dA7, W7, wq7, Y7, ws7

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import int8_forward as o8      # host baseline only
        shapes = []
        for K, N in ((768, 2304), (768, 768), (768, 3072), (3072, 768)):
            L = next(x for x in m["layers"] if x["K"] == K and x["N"] == N)
            W = np.random.default_rng(K + N).standard_normal((N, K)).astype(np.float16)
            Wq, sW, _ = o8.quantize_weight(W)
            shapes.append((L["A"].cpu().numpy(), Wq, sW))
        t_start = time.perf_counter()
        reps = 0
        while True:     # whole passes over the four shapes (one block), at least cpu_seconds
            for A, Wq, sW in shapes:
                o8.forward(A, m["offsets"], Wq, sW, 6.0)
            reps += 1
            if time.perf_counter() - t_start >= args.cpu_seconds:
                break
        step_s = 12 * (time.perf_counter() - t_start) / reps
        try:
            import threadpoolctl
            threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info())
        except Exception:
            threads = os.cpu_count()
        cpu = {"value": B / step_s, "unit": "records/s", "cores": threads, "kind": "oracle",
               "sample": f"{reps} passes over one block's four forwards (qkv 768->2304, out "
                         "768->768, fc1 768->3072, fc2 3072->768) on the 16 x 256-token batch, "
                         "times the 12 blocks "
                         f"({time.perf_counter() - t_start:.1f} s wall; numpy, BLAS threads)"}

    line = {"metric": "records/sec, record-owned LLM.int8 forward of a frozen backbone",
            "value": B / (graph_ms * 1e-3), "unit": "records/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": graph_ms,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
            "data": "synthetic",
            "config": {"workload": "opt125m_int8_forward", "int8_layers": 72,
                       "forwards_per_step": len(m["layers"]), "qkv_fused": True,
                       "records": B, "tokens": m["T"], "rows": n, "tau": 6.0,
                       "timing": "HIP graph of the 48 forwards; record offsets set before"},
            "roofline": roof, "cpu_baseline": cpu,
            "eager_ms_per_step": eager_ms, "large_layer": large,
            "batched_union": {"graph_ms_per_step": batched_graph_ms,
                              "eager_ms_per_step": batched_eager_ms},
            "tokens_per_s": n / (graph_ms * 1e-3)}
    print(json.dumps(line), flush=True)


def achievable_hbm(torch, dev, dp, mib=2048, reps=10):
    """The HBM read rate that a plain streaming read with 16-byte loads reaches on this device
    (dpsgd_hbm_read over a 2 GiB buffer, best of `reps` launches timed with HIP events): the
    measured reference beside the vendor peak."""
    nbytes = mib << 20
    x = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(dp.HBM_READ_SINK_WORDS, dtype=torch.int32, device=dev)
    dp.hbm_read(x.data_ptr(), nbytes, sink.data_ptr())
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dp.hbm_read(x.data_ptr(), nbytes, sink.data_ptr())
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b) * 1e-3)
    del x, sink
    return {"read_gbs": nbytes / best / 1e9,
            "how": f"dpsgd_hbm_read: streaming 16-byte loads over {mib} MiB, best of {reps}"}


def achievable_hbm_at(torch, dev, dp, nbytes, n_bufs=N_SETS, reps=40):
    """The same streaming read at a kernel's own size: dpsgd_hbm_read over `n_bufs` distinct
    buffers of `nbytes` each, launched in turn (so that no launch re-reads what the last-level
    cache kept), median of `reps` launches timed one by one with HIP events.  Launch ramp-up and
    drain weigh more at tens of microseconds than over 2 GiB; this is the read rate a kernel of
    that size can expect."""
    nb = nbytes // 16 * 16
    bufs = [torch.ones(nb // 4, dtype=torch.int32, device=dev) for _ in range(n_bufs)]
    sink = torch.empty(dp.HBM_READ_SINK_WORDS, dtype=torch.int32, device=dev)
    for b in bufs:
        dp.hbm_read(b.data_ptr(), nb, sink.data_ptr())
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record()
        dp.hbm_read(bufs[i % n_bufs].data_ptr(), nb, sink.data_ptr())
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e-3 for a, b in evs)[reps // 2]
    del bufs, sink
    return {"read_gbs": nb / t / 1e9, "bytes": nb, "us": t * 1e6,
            "how": f"dpsgd_hbm_read over {n_bufs} distinct {nb / 1e6:.0f} MB buffers in turn, "
                   f"median of {reps} launches"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD, choices=[1, 2, 3, 4, 5],
                    help="3 (default): the largest configuration that fits one GPU")
    ap.add_argument("--sum", default="auto", choices=sorted(SUM_POLICIES),
                    help="clipped-sum strategy: auto (per-record gradient blocks kept by the norm "
                         "pass where that moves fewer bytes), gemm (A^T diag(c) G re-reading A and "
                         "G), stored")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--manifest", default=None, help="write a run manifest JSON here")
    ap.add_argument("--mode", default="step", choices=["step", "kernel", "copy", "sample", "int8"],
                    help="step: the benchmark; kernel: only the dominant kernel's phase (or "
                         "--phase), --warmup + --steps times (for counter collection); copy: a "
                         "plain device copy of --copy-mib MiB (the reference for scaling HBM byte "
                         "counters)")
    ap.add_argument("--phase", default=None, choices=["norms", "clipped_sum", "noise"])
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--users", action="store_true",
                    help="workload 2's layers with user-level clipping: 16 users of 1-4 records each "
                         "(variable-length records, rows concatenated per user)")
    ap.add_argument("--descent", action="store_true",
                    help="fuse the descent step theta -= lr * noised sum / L into the timed step, with "
                         "lr 0.01 and L 1 (the sensitivity paper's release audit settings)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path (sharding of "
              "the step across GPUs is a design note, not built). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import datagen
    import differentially_private_amd as dp

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.mode == "copy":
        n = args.copy_mib * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        print(json.dumps({"mode": "copy", "bytes_read": 4 * n, "bytes_written": 4 * n,
                          "ms": ms, "GBps": 8 * n / ms / 1e6}), flush=True)
        return
    if args.mode == "sample":
        return sample_line(args, torch, dev, dp)
    if args.mode == "int8":
        return int8_line(args, torch, dev, dp)
    w = datagen.workload(args.workload)
    if args.users:
        return users_line(args, datagen.workload(2), torch, dev, dp, datagen)
    if args.mode == "kernel":
        return kernel_mode(args, w, torch, dev, dp, datagen)
    return step_line(args, w, torch, dev, dp, datagen)


if __name__ == "__main__":
    main()
