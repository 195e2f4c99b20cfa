#!/usr/bin/env python3
"""Benchmark of the DP-SGD private-gradient step (ghost per-record norms -> clip -> clipped sum ->
Gaussian noise) on one MI355X, through the library's C ABI.

Default workload: the OPT-125M-shaped rank-8 LoRA on q,v of 12 blocks (48 linear layers,
294,912 trainables), 16 records x 128 tokens, fp32 activations and output gradients ~ N(0,1),
C = 1, sigma = 1.  Inputs are synthetic (the seeded generator, written straight into HBM) and
resident before timing.  A step is one pass of the whole path over one batch.

Prints one JSON line: records/s over --steps timed steps, the roofline of the dominant kernel
(its average duration from HIP events recorded around it inside the timed loop), and the CPU
oracle timed on the host's cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_work(w, plan, dp):
    """Per-phase algorithmic HBM bytes / flops for one physical batch of w."""
    e = 4 if w.dtype == 0 else 2
    B, T = w.B, w.T
    norm_bytes = norm_flops = sum_bytes = sum_flops = 0
    for l, (di, do) in enumerate(w.layers):
        path, sm = plan.layer_info(l)
        in_bytes = B * T * (di + do) * e
        norm_bytes += in_bytes
        if path == dp.PATH_GRAM:
            norm_flops += 2 * B * T * T * (di + do)
        else:
            norm_flops += 2 * B * T * di * do
        if sm == dp.SUM_STORED:
            norm_bytes += B * di * do * 4            # the per-record gradient blocks written once
            sum_bytes += B * di * do * 4 + di * do * 4
        else:
            sum_bytes += in_bytes + di * do * 4
            sum_flops += 2 * B * T * di * do
    return {"norms": (norm_bytes, norm_flops), "clipped_sum": (sum_bytes, sum_flops),
            "noise": (8 * w.n_params, 0)}


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


# sources the ghost-norm kernels are compiled from: a stored HBM-traffic record applies only while
# these are unchanged
NORM_KERNEL_SOURCES = ("ghost_norm.hip", "tile_direct.h", "device_common.h", "internal.h")


# sources the INT8 forward's kernels are compiled from (same rule for its traffic record)
I8_KERNEL_SOURCES = ("int8_forward.hip", "int8.h", "device_common.h", "internal.h")


def kernel_src_hash(names=NORM_KERNEL_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "differentially_private_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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
    import numpy as np  # noqa: F401
    import datagen
    import oracle
    As = [datagen.host_tensor(w, l, 0) for l in range(w.n_layers)]
    Gs = [datagen.host_tensor(w, l, 1) for l in range(w.n_layers)]
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.step(As, Gs, w.C, w.sigma, w.noise_seed, 0)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    cores = oracle.num_threads()
    # the same oracle on one thread, on a shorter sample (at least one step)
    oracle.set_num_threads(1)
    reps1 = 0
    t0 = time.perf_counter()
    try:
        while True:
            oracle.step(As, Gs, w.C, w.sigma, w.noise_seed, 0)
            reps1 += 1
            el1 = time.perf_counter() - t0
            if el1 >= seconds / 3:
                break
    finally:
        oracle.set_num_threads(cores)
    return {"value": w.B * reps / el, "unit": "records/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{reps} full steps of the workload ({w.B} records x {w.n_layers} layers, "
                      f"noise included, input generation excluded), {el:.1f} s wall",
            "single_thread": {"value": w.B * reps1 / el1, "unit": "records/s", "cores": 1,
                              "sample": f"{reps1} full steps, {el1:.1f} s wall"}}


def sum_roofline(work, w, phase):
    """Algorithmic rate of the clipped-sum phase when it was timed alone (GEMM strategy: flops
    against the bf16/fp32 MFMA peak; STORED: bytes against HBM)."""
    if "clipped_sum" not in phase:
        return None
    sb, sf = work["clipped_sum"]
    t = phase["clipped_sum"] * 1e-3
    if sf:
        peak = MFMA_PEAK_TFLOPS[w.dtype]
        return {"TFLOPs": sf * w.n_phys / t / 1e12, "mfma_frac": sf * w.n_phys / t / 1e12 / peak}
    return {"hbm_GBps": sb * w.n_phys / t / 1e9, "hbm_frac": sb * w.n_phys / t / 1e9 / HBM_PEAK_GBS}


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
    x0, x1 = ev(), ev()
    x0.record(stream)
    for _ in range(args.steps):
        dp.norms(plan, n_users, 0, w.n_layers, As, Gs, ws)
    x1.record(stream)
    torch.cuda.synchronize()
    norm_ms = x0.elapsed_time(x1) / args.steps
    rows = int(offs[-1])
    norm_bytes = rows * sum(di + do for di, do in w.layers) * 4 + n_users * w.n_params * 4
    line = {"metric": "users/sec per DP-SGD step with user-level clipping", "value": n_users / (ms * 1e-3),
            "unit": "users/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": datagen.configs.DTYPE_NAMES[w.dtype], "data": "synthetic",
            "config": {"workload": w.name + "_users", "users": n_users, "records": n_rec,
                       "token_rows": rows, "max_rows_per_user": T_max, "layers": w.n_layers,
                       "params": w.n_params, "parallelism": "single GPU"},
            "phases_ms": {"norms": norm_ms, "rest_of_step": ms - norm_ms},
            "norms_roofline": {"hbm_GBps": norm_bytes / (norm_ms * 1e-3) / 1e9,
                               "hbm_frac": norm_bytes / (norm_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                               "algorithmic_bytes": norm_bytes}}
    print(json.dumps(line), flush=True)


def secondary(args, w, torch, dev, dp, datagen):
    """Secondary lines for workloads 1, 3, 4, 5: one step = all physical batches of a logical
    batch (virtual batching: norms/clip/sum per physical batch, noise once), inputs resident in
    HBM; workload 3 streams layer chunks when all inputs do not fit beside the workspace, and then
    times only the device phases (staging excluded).  Per-phase times come from HIP events."""
    import numpy as np
    L = w.n_layers
    plan = dp.Plan(w.layers, w.dtype, w.B, w.T)
    ws = plan.workspace(dev)
    out = [torch.empty(di * do, dtype=torch.float32, device=dev) for di, do in w.layers]
    theta = ([torch.zeros(di * do, dtype=torch.float32, device=dev) for di, do in w.layers]
             if args.descent else None)
    e = 4 if w.dtype == 0 else 2
    in_bytes = w.input_bytes_per_batch()
    free = torch.cuda.mem_get_info()[0]
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    phase = {"norms": 0.0, "rest_of_step": 0.0}
    note = ""
    n_cycle = 1
    if w.n_phys * in_bytes < free - (8 << 30):
        batches = [device_inputs(w, datagen, torch, dev, p * w.B, w.B) for p in range(w.n_phys)]
        # one physical batch: the timed steps cycle through N_SETS distinct batches when they fit,
        # so that no step re-reads inputs a previous step left in the last-level cache
        cycle = [batches]
        if w.n_phys == 1 and N_SETS * in_bytes < (free - (8 << 30)) // 2:
            cycle += [[device_inputs(w, datagen, torch, dev, k * w.B, w.B)] for k in range(1, N_SETS)]
        turn = [0]
        n_cycle = len(cycle)

        def step():
            bs = cycle[turn[0] % len(cycle)]
            turn[0] += 1
            for p, (As, Gs) in enumerate(bs):
                flags = (dp.NO_NOISE if w.n_phys > 1 else 0) | (dp.ACCUMULATE if p else 0)
                last = w.n_phys == 1
                dp.step(plan, As, Gs, out, ws, w.C, w.sigma, w.noise_seed, 0, flags=flags,
                        params=theta if last else None, lr=DESCENT_LR, normalizer=DESCENT_L)
            if w.n_phys > 1:
                dp.noise(plan, out, w.C, w.sigma, w.noise_seed, 0, ws=ws, params=theta,
                         lr=DESCENT_LR, normalizer=DESCENT_L)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(args.steps):
            step()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / args.steps
        As, Gs = batches[0]

        def timed(fn):
            x0, x1 = ev(), ev()
            x0.record(stream)
            for _ in range(args.steps):
                fn()
            x1.record(stream)
            torch.cuda.synchronize()
            return x0.elapsed_time(x1) / args.steps
        # each phase alone on physical batch 0 (K back-to-back calls between HIP events), with
        # the C calls' arguments marshalled once so that the host does not pace the GPU
        lib = dp.load()
        arr_a, arr_g, arr_o = dp._ptr_array(As), dp._ptr_array(Gs), dp._ptr_array(out)
        wsp, sp = ws.data_ptr(), stream.cuda_stream

        def checked(rc):
            if rc:
                dp._check(rc)
        phase["norms"] = timed(lambda: checked(lib.dpsgd_norms(plan.handle, w.B, 0, L, arr_a, arr_g,
                                                               wsp, sp))) * w.n_phys
        phase["clip"] = timed(lambda: checked(lib.dpsgd_clip(plan.handle, w.B, w.C, 0, wsp, None,
                                                             None, sp))) * w.n_phys
        phase["clipped_sum"] = timed(lambda: checked(lib.dpsgd_clipped_sum(
            plan.handle, w.B, 0, L, arr_a, arr_g, None, arr_o, 0, wsp, sp))) * w.n_phys
        phase["noise"] = timed(lambda: dp.noise(plan, out, w.C, w.sigma, w.noise_seed, 0, ws=ws,
                                                params=theta, lr=DESCENT_LR, normalizer=DESCENT_L))
        phase["rest_of_step"] = ms - phase["norms"]   # residual: the step minus the norms timed alone
    else:
        # layer-chunk streaming: chunks of inputs filled (untimed), norms timed per chunk
        note = "layer-chunk streaming, staging excluded"
        chunk = 32
        ms_norm = 0.0
        for l0 in range(0, L, chunk):
            l1 = min(L, l0 + chunk)
            As = [None] * (l1 - l0)
            Gs = [None] * (l1 - l0)
            for l in range(l0, l1):
                for tensor, lst in ((0, As), (1, Gs)):
                    scale, heavy = datagen.record_params(w, l, tensor, 0, w.B)
                    ds = torch.from_numpy(scale).to(dev)
                    dh = torch.from_numpy(heavy.astype(np.uint8)).to(dev)
                    d = w.layers[l][0] if tensor == 0 else w.layers[l][1]
                    buf = torch.empty((w.B, w.T, d), dtype=torch.int16 if e == 2 else torch.float32, device=dev)
                    datagen.device_fill(w, l, tensor, buf.data_ptr(), 0, w.B, ds.data_ptr(), dh.data_ptr(),
                                        stream.cuda_stream)
                    lst[l - l0] = buf
            torch.cuda.synchronize()
            for _ in range(max(1, args.warmup // 4)):
                dp.norms(plan, w.B, l0, l1, As, Gs, ws)
            x0, x1 = ev(), ev()
            x0.record(stream)
            for _ in range(args.steps):
                dp.norms(plan, w.B, l0, l1, As, Gs, ws)
            x1.record(stream)
            torch.cuda.synchronize()
            ms_norm += x0.elapsed_time(x1) / args.steps
            del As, Gs
        y0, y1 = ev(), ev()
        y0.record(stream)
        for _ in range(args.steps):
            dp.clip(plan, w.B, w.C, ws)
            dp.clipped_sum(plan, w.B, 0, L, None, None, None, out, ws)
            dp.noise(plan, out, w.C, w.sigma, w.noise_seed, 0, ws=ws, params=theta, lr=DESCENT_LR,
                     normalizer=DESCENT_L)
        y1.record(stream)
        torch.cuda.synchronize()
        phase["norms"] = ms_norm
        phase["rest_of_step"] = y0.elapsed_time(y1) / args.steps
        ms = ms_norm + phase["rest_of_step"]
    assert dp.status(plan, ws) == dp.OK
    work = algorithmic_work(w, plan, dp)
    nb, nf = work["norms"]
    nb *= w.n_phys
    nf *= w.n_phys
    try:
        ach = achievable_hbm(torch, dev, dp)
    except torch.cuda.OutOfMemoryError:
        ach = None
    norm_gbs = nb / (phase["norms"] * 1e-3) / 1e9
    line = {"metric": METRIC, "value": w.logical_B / (ms * 1e-3), "unit": "records/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": datagen.configs.DTYPE_NAMES[w.dtype],
            "data": "synthetic",
            "config": {"workload": w.name, "layers": L, "params": w.n_params,
                       "records_per_step": w.logical_B, "physical_batches": w.n_phys, "tokens": w.T,
                       "parallelism": "single GPU", "note": note,
                       "descent": {"lr": DESCENT_LR, "normalizer": DESCENT_L} if args.descent else None},
            "phases_ms": phase, "input_batches": n_cycle,
            "norms_roofline": {"hbm_GBps": norm_gbs, "hbm_frac": norm_gbs / HBM_PEAK_GBS,
                               "frac_of_achievable": norm_gbs / ach["read_gbs"] if ach else None,
                               "TFLOPs": nf / (phase["norms"] * 1e-3) / 1e12},
            "hbm_achievable": ach,
            "clipped_sum_roofline": sum_roofline(work, w, phase),
            "clipped_sum_bytes": work["clipped_sum"][0] * w.n_phys}
    print(json.dumps(line), flush=True)


N_SETS = 4   # distinct input batches the headline's timed steps cycle through
I8_PEAK_TOPS = 5000.0   # dense INT8 MFMA, ops/s x 1e-12


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
    roofline from HIP events around each dpsgd_i8_matmul, the batched LLM.int8 variant (one
    record spanning the batch: the same kernels with the batch-wide union) for comparison, and
    the oracle's rate on one layer of each shape."""
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

    # dominant kernel: the INT8 GEMM of every layer, HIP events around dpsgd_i8_matmul (the
    # routing kernels of that layer run untimed just before it)
    ops = 0
    gemm_ms = 0.0
    reps = max(1, args.steps // 10)
    launches = 0
    abytes = 0   # codes + weight codes read, fp16 outputs written (outlier corrections aside)
    for _ in range(reps):
        for L in m["layers"]:
            dp.i8_route(plan, ws, n, B, L["A"], L["K"], 6.0, stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dp.i8_matmul(plan, ws, n, B, L["A"], L["K"], L["wq"], L["sw"], L["N"], L["Y"], stream)
            e1.record(stream)
            torch.cuda.synchronize()
            gemm_ms += e0.elapsed_time(e1)
            ops += 2 * n * L["K"] * L["N"]
            abytes += (n + L["N"]) * dp.i8_pitch(L["K"]) + 2 * n * L["N"]
            launches += 1
    avg_ms = gemm_ms / launches
    achieved = ops / (gemm_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": achieved, "peak": I8_PEAK_TOPS, "unit": "TOP/s",
            "frac": achieved / I8_PEAK_TOPS, "traffic": stored_i8_traffic(),
            "kernel": "k_i8_gemm (INT8 MFMA, dequantisation + record-owned FP16 correction)",
            "algorithmic_ops_per_launch": ops / launches, "algorithmic_bytes_per_launch": abytes / launches,
            "avg_ms": avg_ms, "launches": launches}

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
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5],
                    help="2 (default) is the configuration the metric is quoted on; the others "
                         "print secondary lines")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", default=None,
                    help="JSON file with measured HBM bytes per launch of the dominant kernel")
    ap.add_argument("--manifest", default=None, help="write a run manifest JSON here")
    ap.add_argument("--mode", default="step", choices=["step", "kernel", "copy", "sample", "int8"],
                    help="step: the benchmark; kernel: only the dominant kernel, --steps times "
                         "(for counter collection); copy: a plain device copy of --copy-mib MiB "
                         "(the reference for scaling HBM byte counters)")
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
    if args.mode == "step" and args.users:
        return users_line(args, w, torch, dev, dp, datagen)
    if args.mode == "step" and args.workload != 2:
        return secondary(args, w, torch, dev, dp, datagen)
    plan = dp.Plan(w.layers, w.dtype, w.B, w.T)
    ws = plan.workspace(dev)
    As, Gs = device_inputs(w, datagen, torch, dev, 0, w.B)
    out = [torch.empty(di * do, dtype=torch.float32, device=dev) for di, do in w.layers]
    L = w.n_layers
    stream = torch.cuda.current_stream()
    # the timed steps cycle through N_SETS distinct batches (records k B .. k B + B - 1 of the
    # generator), so that no step re-reads inputs a previous step left in the last-level cache
    sets = [(As, Gs)] + ([device_inputs(w, datagen, torch, dev, k * w.B, w.B) for k in range(1, N_SETS)]
                         if args.mode == "step" else [])

    if args.mode == "kernel":
        for _ in range(args.warmup + args.steps):
            dp.norms(plan, w.B, 0, L, As, Gs, ws)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "kernel", "workload": w.name, "launches": args.warmup + args.steps,
                          "algorithmic_bytes": algorithmic_work(w, plan, dp)["norms"][0]}), flush=True)
        return

    theta = ([torch.zeros(di * do, dtype=torch.float32, device=dev) for di, do in w.layers]
             if args.descent else None)
    calls = [dp.StepCall(plan, A, G, out, ws, w.C, w.sigma, w.noise_seed, 0, params=theta,
                         lr=DESCENT_LR, normalizer=DESCENT_L) for A, G in sets]
    for i in range(max(args.warmup, len(calls))):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    assert dp.status(plan, ws) == dp.OK

    # timed region 1: K whole steps (dpsgd_step: norms -> clip -> clipped sum -> noise), each on
    # the next batch of the cycle
    def timed_steps(cs):
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for i in range(args.steps):
            cs[i % len(cs)]()
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop), time.perf_counter() - t0
    gpu_ms, wall = timed_steps(calls)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps
    assert dp.status(plan, ws) == dp.OK
    # the same batch every step, for comparison (its inputs partly stay in the last-level cache)
    gpu1, wall1 = timed_steps(calls[:1])
    same_ms = max(gpu1, wall1 * 1e3) / args.steps

    # timed region 2: the dominant kernel (the norm launch of the same step, same buffers, the
    # same cycle of batches), K launches back to back between two HIP events on the stream they
    # run on: the average holds the kernel and the gap to the next dispatch, not the events'
    # own recording
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        A, G = sets[i % len(sets)]
        dp.norms(plan, w.B, 0, L, A, G, ws)
    e1.record(stream)
    torch.cuda.synchronize()
    phase_ms = {"norms": e0.elapsed_time(e1) / args.steps}
    phase_ms["rest_of_step"] = max(ms_per_step - phase_ms["norms"], 0.0)

    work = algorithmic_work(w, plan, dp)
    dom = "norms"
    nbytes, nflops = work[dom]
    dur_s = phase_ms[dom] * 1e-3
    if nflops and nflops / max(nbytes, 1) > MFMA_PEAK_TFLOPS[w.dtype] * 1e12 / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": nflops / dur_s / 1e12,
                "peak": MFMA_PEAK_TFLOPS[w.dtype], "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": nbytes / dur_s / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    tpath = args.traffic or os.path.join(ROOT, "profiles", "norm_kernel_traffic.json")
    if os.path.exists(tpath):
        # HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled by a plain copy of
        # known size), valid only while the kernel sources are the ones it was measured on
        tr = json.load(open(tpath))
        if (tr.get("kernel_phase") == dom and tr.get("workload") == w.name
                and tr.get("src_hash") == kernel_src_hash()):
            roof["traffic"] = tr.get("bytes_per_launch")
    if roof["unit"] == "GB/s":
        roof["achievable"] = achievable_hbm(torch, dev, dp)
        roof["frac_of_achievable"] = roof["achieved"] / roof["achievable"]["read_gbs"]
        in_bytes = sum(t.numel() * t.element_size() for t in As + Gs)
        roof["achievable_at_size"] = achievable_hbm_at(torch, dev, dp, in_bytes)
        roof["frac_of_achievable_at_size"] = roof["achieved"] / roof["achievable_at_size"]["read_gbs"]
    roof["kernel"] = {"norms": "k_norm_direct (ghost_norm, direct path)",
                      "clipped_sum": "clipped_sum", "noise": "k_noise"}[dom]
    roof["algorithmic_bytes"] = nbytes
    roof["avg_ms"] = phase_ms[dom]

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)

    value = w.B / (ms_per_step * 1e-3)
    line = {
        "metric": METRIC, "value": value, "unit": "records/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": datagen.configs.DTYPE_NAMES[w.dtype], "data": "synthetic",
        "config": {"workload": w.name, "layers": w.n_layers, "params": w.n_params,
                   "records_per_step": w.B, "tokens": w.T, "C": w.C, "sigma": w.sigma,
                   "parallelism": "single GPU",
                   "descent": {"lr": DESCENT_LR, "normalizer": DESCENT_L} if args.descent else None},
        "roofline": roof, "cpu_baseline": cpu,
        "phases_ms": phase_ms, "gpu_ms_per_step": gpu_ms / args.steps,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "input_batches": len(sets),
        "same_batch": {"value": w.B / (same_ms * 1e-3), "ms_per_step": same_ms,
                       "note": "every timed step on one batch; its inputs partly stay in the last-level cache"},
    }
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


if __name__ == "__main__":
    main()
