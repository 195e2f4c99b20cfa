"""Workloads 3, 4 and 5 at full size, in the configuration the benchmark runs.  The oracle's full
run of workloads 3 and 5 would take hours, so they are checked two ways:

- whole outputs: the step exactly as the benchmark runs it (every layer, every record, every
  physical batch), with two layers carrying the generator's inputs and every other layer's A and
  G pointing at one all-zero buffer.  The record norms then come from those two layers, so the
  oracle computes every output: n and c of every record, the two layers' pre-noise and noised
  sums whole, every other layer exactly 0 before the noise and sigma C Z after it;
- sampled outputs on the real inputs: per-(record, layer) squared norms and the joint norm /
  clip factor of sampled records; entries of the clipped sum for caller-supplied factors (both
  factor 1 and factors below 1), from gathered input columns; the noise of every coordinate.
Workload 4 runs its full-width step on four records against the whole oracle, and its 64-record
sum with caller factors on one entry of every 256 x 256 output tile.  Inputs are filled directly
in HBM by the device generator, which is checked bit for bit against the host generator the
oracle uses.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import datagen  # noqa: E402
import differentially_private_amd as dp  # noqa: E402
import oracle  # noqa: E402
from _helpers import (TOL, device_tensor, flat, max_rel, oracle_record_layer_norm2,  # noqa: E402
                      oracle_sum_entry, rel_err)
from datagen import BF16  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("idx,layer,first,n", [(3, 0, 99, 3), (3, 1, 0, 2), (2, 5, 3, 4), (4, 2, 10, 1)])
def test_device_generator_matches_host(idx, layer, first, n):
    w = datagen.workload(idx)
    say("generator", w.name, layer, first, n)
    for tensor in (0, 1):
        d = device_tensor(w, layer, tensor, first, n, DEV).cpu().numpy()
        h = datagen.host_tensor(w, layer, tensor, first, n)
        assert np.array_equal(d.view(h.dtype), h)


def _layer_norms(plan, n_rec, L, ws):
    out = torch.empty(L * n_rec, dtype=torch.float32, device=DEV)
    dp.layer_norm2(plan, n_rec, 0, L, ws, out)
    return out.cpu().numpy().reshape(L, n_rec)


def _check_sum_entries(w, S_gpu_layers, c, picks, tol, first=0, n=None):
    """Each picked entry within tol of the oracle's, relative to the larger of its own magnitude
    and the rms of the oracle's picked entries of the same layer (the per-entry form of the
    relative Frobenius bound: an entry that happens to cancel is not held to a tighter one)."""
    wants = [oracle_sum_entry(w, l, j, k, c, first, n) for (l, j, k) in picks]
    rms = {}
    for (l, _, _), v in zip(picks, wants):
        rms.setdefault(l, []).append(v * v)
    rms = {l: math.sqrt(sum(v) / len(v)) for l, v in rms.items()}
    for (l, j, k), want in zip(picks, wants):
        got = float(S_gpu_layers[l][j * w.layers[l][1] + k])
        scale = max(abs(want), rms[l], 1e-30)
        assert abs(got - want) <= tol * scale, (l, j, k, got, want, rms[l])


def test_workload3_full_layer_streaming():
    """7B-shaped LoRA, 256 records x 512 tokens x 256 layers (276 GB of inputs): norms in layer
    chunks (inputs regenerated per chunk), then clip, the clipped sum from the kept gradient
    blocks (no second read of the inputs) and the noise."""
    w = datagen.workload(3)
    L, B = w.n_layers, w.B
    plan = dp.Plan(w.layers, w.dtype, B, w.T)
    assert all(plan.layer_info(l)[1] == dp.SUM_STORED for l in range(L))
    ws = plan.workspace(DEV)
    chunk = 32
    for l0 in range(0, L, chunk):
        say("workload 3 norms, layers", l0, l0 + chunk)
        As = [device_tensor(w, l, 0, 0, B, DEV) for l in range(l0, l0 + chunk)]
        Gs = [device_tensor(w, l, 1, 0, B, DEV) for l in range(l0, l0 + chunk)]
        dp.norms(plan, B, l0, l0 + chunk, As, Gs, ws)
        torch.cuda.synchronize()
        del As, Gs
    nrm = torch.empty(B, dtype=torch.float32, device=DEV)
    cf = torch.empty(B, dtype=torch.float32, device=DEV)
    dp.clip(plan, B, w.C, ws, norms_out=nrm, clip_out=cf)
    assert dp.status(plan, ws) == dp.OK
    n_gpu, c_gpu = nrm.cpu().numpy(), cf.cpu().numpy()
    ln = _layer_norms(plan, B, L, ws)
    tol = TOL[BF16]
    # record 0 (heavy-tailed, Student-t) over all 256 layers: joint norm and clip factor
    say("workload 3 oracle record 0")
    want = oracle_record_layer_norm2(w, 0, range(L))
    assert max_rel(ln[:, 0], want) <= tol
    n_o = math.sqrt(want.sum())
    c_o = oracle.clip_factor(want.sum(), w.C)
    assert abs(n_gpu[0] - n_o) <= tol * n_o and abs(c_gpu[0] - c_o) <= tol * c_o
    # a light record on a spread of layers
    lay = list(range(0, L, 17))
    want = oracle_record_layer_norm2(w, 131, lay)
    assert max_rel(ln[lay, 131], want) <= tol
    # clipped sum from the kept blocks with caller factors (A and G no longer needed)
    c_test = (0.05 + 0.9 * (np.arange(B) % 7) / 6).astype(np.float32)
    out = [torch.empty(a * b, dtype=torch.float32, device=DEV) for a, b in w.layers]
    dp.clipped_sum(plan, B, 0, L, None, None, torch.from_numpy(c_test).to(DEV), out, ws)
    torch.cuda.synchronize()
    S = [o.cpu().numpy() for o in out]
    rng = np.random.default_rng(3)
    picks = [(int(l), int(rng.integers(w.layers[l][0])), int(rng.integers(w.layers[l][1])))
             for l in rng.choice(L, 12, replace=False)]
    say("workload 3 sum entries", picks[:3], "...")
    _check_sum_entries(w, S, c_test.astype(np.float64), picks, tol)
    # noise once over all 16.8M coordinates
    pre = flat(S)
    dp.noise(plan, out, w.C, w.sigma, 0, 0, ws=ws)
    torch.cuda.synchronize()
    z_gpu = (flat([o.cpu().numpy() for o in out]) - pre) / (w.sigma * w.C)
    z = oracle.gauss(0, 0, 0, z_gpu.size)
    assert np.max(np.abs(z_gpu - z) / (1 + np.abs(z) + np.abs(pre) / (w.sigma * w.C))) <= 16 * 2.0 ** -24
    assert abs(np.linalg.norm(z_gpu) - math.sqrt(z.size)) < 5


def test_workload4_full_gram_and_direct():
    """Four dense 4096x4096 layers, 64 records x 256 tokens: the Gram path (the one the rule
    picks) against the oracle and against the forced direct path on the same data; the GEMM
    clipped sum for caller factors; the whole step's status."""
    w = datagen.workload(4)
    L, B = w.n_layers, w.B
    As = [device_tensor(w, l, 0, 0, B, DEV) for l in range(L)]
    Gs = [device_tensor(w, l, 1, 0, B, DEV) for l in range(L)]
    res = {}
    for path in (dp.PATH_AUTO, dp.PATH_DIRECT):
        say("workload 4 norms, path", path)
        plan = dp.Plan(w.layers, w.dtype, B, w.T, path)
        ws = plan.workspace(DEV)
        dp.norms(plan, B, 0, L, As, Gs, ws)
        res[path] = _layer_norms(plan, B, L, ws)
    plan = dp.Plan(w.layers, w.dtype, B, w.T)
    assert plan.layer_info(0)[0] == dp.PATH_GRAM
    tol = TOL[BF16]
    assert max_rel(res[dp.PATH_DIRECT], res[dp.PATH_AUTO]) <= tol
    for rec in (0, 63):
        say("workload 4 oracle record", rec)
        want = oracle_record_layer_norm2(w, rec, range(L))
        assert max_rel(res[dp.PATH_AUTO][:, rec], want) <= tol
        assert max_rel(res[dp.PATH_DIRECT][:, rec], want) <= tol
    # GEMM clipped sum with caller factors, sampled entries
    ws = plan.workspace(DEV)
    c_test = np.linspace(0.2, 1.0, B).astype(np.float32)
    out = [torch.empty(a * b, dtype=torch.float32, device=DEV) for a, b in w.layers]
    dp.ws_init(plan, ws)
    dp.clipped_sum(plan, B, 0, L, As, Gs, torch.from_numpy(c_test).to(DEV), out, ws)
    torch.cuda.synchronize()
    S = [o.cpu().numpy() for o in out]
    rng = np.random.default_rng(4)
    picks = [(l, 256 * tm + int(rng.integers(256)), 256 * tn + int(rng.integers(256)))
             for l in range(L) for tm in range(16) for tn in range(16)]   # one per 256 x 256 tile
    say("workload 4 sum entries, one per output tile:", len(picks))
    _check_sum_entries(w, S, c_test.astype(np.float64), picks, tol)
    # the whole step on this data: status OK and every record clipped (n ~ 131 >> C)
    nrm = torch.empty(B, dtype=torch.float32, device=DEV)
    dp.step(plan, As, Gs, out, ws, w.C, w.sigma, 0, 0, norms_out=nrm)
    assert dp.status(plan, ws) == dp.OK
    n = nrm.cpu().numpy()
    assert np.all(n > w.C) and np.all(np.isfinite(flat([o.cpu().numpy() for o in out])))


def test_workload5_full_virtual_batch():
    """4096 logical records in 16 physical batches of 256 (6.5 GB of inputs each), every layer
    carrying the generator's inputs: per physical batch the norms and the clip factors at the
    workload's C = 1 (every record clipped: c_i n_i <= C (1 + 4 * 2^-24) on all 4096), then the
    clipped sum with caller factors that take both branches' values (1 for every third record,
    below 1 otherwise), accumulated over the 16 batches; norms of records from several batches
    against the oracle; sampled sum entries over all 4096 records; the noise drawn once."""
    w = datagen.workload(5)
    L, B = w.n_layers, w.B
    plan = dp.Plan(w.layers, w.dtype, B, w.T)
    ws = plan.workspace(DEV)
    out = [torch.empty(a * b, dtype=torch.float32, device=DEV) for a, b in w.layers]
    r_all = np.arange(w.logical_B)
    c_test = np.where(r_all % 3 == 0, 1.0, 0.05 + 0.9 * (r_all % 7) / 6).astype(np.float32)
    sampled = {0: None, 1000: None, 4095: None}
    ns, cs = [], []
    for p in range(w.n_phys):
        say("workload 5 physical batch", p)
        As = [device_tensor(w, l, 0, p * B, B, DEV) for l in range(L)]
        Gs = [device_tensor(w, l, 1, p * B, B, DEV) for l in range(L)]
        nrm = torch.empty(B, dtype=torch.float32, device=DEV)
        cf = torch.empty(B, dtype=torch.float32, device=DEV)
        acc = dp.ACCUMULATE if p else 0
        dp.norms(plan, B, 0, L, As, Gs, ws)
        dp.clip(plan, B, w.C, ws, flags=acc, norms_out=nrm, clip_out=cf)
        dc = torch.from_numpy(c_test[p * B:(p + 1) * B]).to(DEV)
        dp.clipped_sum(plan, B, 0, L, As, Gs, dc, out, ws, flags=acc)
        torch.cuda.synchronize()
        ns.append(nrm.cpu().numpy())
        cs.append(cf.cpu().numpy())
        for r in sampled:
            if p * B <= r < (p + 1) * B:
                sampled[r] = float(ns[-1][r - p * B])
        del As, Gs
    assert dp.status(plan, ws) == dp.OK
    n_all, c_all = np.concatenate(ns).astype(np.float64), np.concatenate(cs).astype(np.float64)
    assert np.all(n_all > w.C) and np.all(c_all < 1.0)
    assert np.all(c_all * n_all <= w.C * (1 + 4 * 2.0 ** -24))
    S = [o.cpu().numpy() for o in out]
    rng = np.random.default_rng(5)
    picks = [(int(l), int(rng.integers(w.layers[l][0])), int(rng.integers(w.layers[l][1])))
             for l in rng.choice(L, 6, replace=False)]
    say("workload 5 sum entries over 4096 records", picks)
    _check_sum_entries(w, S, c_test.astype(np.float64), picks, TOL[BF16], 0, w.logical_B)
    for r, n_gpu in sampled.items():
        n2 = oracle_record_layer_norm2(w, r, range(L)).sum()
        want = math.sqrt(n2)
        assert abs(n_gpu - want) <= TOL[BF16] * want, (r, n_gpu, want)
        c_o = oracle.clip_factor(n2, w.C)
        assert abs(c_all[r] - c_o) <= TOL[BF16] * c_o
    pre = flat(S)
    dp.noise(plan, out, w.C, w.sigma, 7, 3, ws=ws)
    torch.cuda.synchronize()
    z_gpu = (flat([o.cpu().numpy() for o in out]) - pre) / (w.sigma * w.C)
    z = oracle.gauss(7, 3, 0, z_gpu.size)
    assert np.max(np.abs(z_gpu - z) / (1 + np.abs(z) + np.abs(pre) / (w.sigma * w.C))) <= 16 * 2.0 ** -24


# ------------------------------------------------------------------------------------------
# whole outputs of the benchmark's step

def _live_inputs(w, live, first, n, zero):
    """Device A and G per layer: generator inputs for records [first, first + n) of the layers in
    `live`, the shared all-zero buffer for every other layer."""
    dA, dG = [zero] * w.n_layers, [zero] * w.n_layers
    for l in live:
        dA[l] = device_tensor(w, l, 0, first, n, DEV)
        dG[l] = device_tensor(w, l, 1, first, n, DEV)
    return dA, dG


def _check_whole(w, plan, live, ref, pre, noised, seed, step, tol):
    """pre / noised: per-layer GPU outputs (numpy) before and after the noise; ref: the oracle's
    logical step over the live layers (no noise).  Live layers whole against the oracle; every
    other layer exactly 0 before the noise and sigma C Z (the oracle's stream at the layer's flat
    offset) after it."""
    offs = np.cumsum([0] + [a * b for a, b in w.layers])
    z = oracle.gauss(seed, step, 0, int(offs[-1]))
    sc = w.sigma * w.C
    for k, l in enumerate(live):
        e_pre = rel_err(pre[l], ref["S"][k].reshape(-1))
        want = ref["S"][k].reshape(-1) + sc * z[offs[l]:offs[l + 1]]
        e_noised = rel_err(noised[l], want)
        say(f"  layer {l} {w.layers[l]}: pre-noise {e_pre:.2e}, noised {e_noised:.2e}")
        assert e_pre <= tol and e_noised <= tol
    dead = [l for l in range(w.n_layers) if l not in live]
    assert all(np.all(pre[l] == 0.0) for l in dead)
    zg = np.concatenate([noised[l].astype(np.float64) / sc for l in dead])
    zo = np.concatenate([z[offs[l]:offs[l + 1]] for l in dead])
    assert np.max(np.abs(zg - zo) / (1 + np.abs(zo))) <= 8 * 2.0 ** -24


def test_workload3_step_whole_outputs():
    """Workload 3 (256 LoRA layers, 256 records x 512 tokens, the STORED plan: norms, the clip
    factors, then the fused sum + noise kernel) through dpsgd_step exactly as the benchmark calls
    it; layers 100 (4096 -> 16) and 201 (16 -> 4096) carry inputs, including the heavy-tailed
    records 0, 100 and 200."""
    w = datagen.workload(3)
    L, B = w.n_layers, w.B
    live = (100, 201)
    plan = dp.Plan(w.layers, w.dtype, B, w.T)
    assert all(plan.layer_info(l)[1] == dp.SUM_STORED for l in range(L))
    ws = plan.workspace(DEV)
    zero = torch.zeros(B * w.T * 4096, dtype=torch.int16, device=DEV)
    dA, dG = _live_inputs(w, live, 0, B, zero)
    out = [torch.full((a * b,), float("nan"), dtype=torch.float32, device=DEV) for a, b in w.layers]
    nrm = torch.empty(B, dtype=torch.float32, device=DEV)
    cf = torch.empty(B, dtype=torch.float32, device=DEV)
    say("workload 3 whole step, pre-noise")
    dp.step(plan, dA, dG, out, ws, w.C, w.sigma, 0, 0, flags=dp.NO_NOISE, norms_out=nrm, clip_out=cf)
    assert dp.status(plan, ws) == dp.OK
    pre = [o.cpu().numpy() for o in out]
    n_gpu, c_gpu = nrm.cpu().numpy(), cf.cpu().numpy()
    say("workload 3 whole step, noised")
    dp.step(plan, dA, dG, out, ws, w.C, w.sigma, 0, 0)
    assert dp.status(plan, ws) == dp.OK
    noised = [o.cpu().numpy() for o in out]
    del dA, dG, zero, ws
    say("workload 3 oracle over the live layers")
    As = [datagen.host_tensor(w, l, 0) for l in live]
    Gs = [datagen.host_tensor(w, l, 1) for l in live]
    ref = oracle.step(As, Gs, w.C, w.sigma, 0, 0, noise=False)
    del As, Gs
    tol = TOL[BF16]
    assert max_rel(n_gpu, ref["n"]) <= tol and max_rel(c_gpu, ref["c"]) <= tol
    assert np.all(ref["c"] < 1.0)          # every record clipped (n around 3 against C = 0.5)
    _check_whole(w, plan, live, ref, pre, noised, 0, 0, tol)


def test_workload4_full_width_few_records_whole():
    """Workload 4's four 4096 x 4096 layers at full width and T = 256 on four records (Gram norms,
    the dense MFMA clipped sum), every output against the oracle: n, c, the whole pre-noise sum and
    the whole noised sum."""
    w = datagen.workload(4).with_(B=4, logical_B=4)
    L, B = w.n_layers, w.B
    say("workload 4, 4 records, whole outputs")
    As = [datagen.host_tensor(w, l, 0) for l in range(L)]
    Gs = [datagen.host_tensor(w, l, 1) for l in range(L)]
    from _helpers import gpu_step
    r0 = gpu_step(w, As, Gs, DEV, flags=dp.NO_NOISE)
    r = gpu_step(w, As, Gs, DEV, plan=r0["plan"], ws=r0["ws"])
    assert r0["plan"].layer_info(0)[0] == dp.PATH_GRAM
    assert r0["status"] == dp.OK and r["status"] == dp.OK
    say("workload 4 oracle")
    ref = oracle.step(As, Gs, w.C, w.sigma, 0, 0)
    tol = TOL[BF16]
    assert max_rel(r["n"], ref["n"]) <= tol and max_rel(r["c"], ref["c"]) <= tol
    e0 = rel_err(flat(r0["out"]), flat(ref["S"]))
    e1 = rel_err(flat(r["out"]), flat(ref["S_noised"]))
    say(f"  pre-noise {e0:.2e}, noised {e1:.2e}")
    assert e0 <= tol and e1 <= tol


def test_workload4_full_width_long_records_whole():
    """Workload 4's four 4096 x 4096 layers at full width with records of 512 tokens (two records):
    the Gram norms take the 128-token block-pair kernel (T > 256), the dense clipped sum 16 k-steps
    per record; n, c, the whole pre-noise sum and the whole noised sum against the oracle."""
    w = datagen.workload(4).with_(B=2, logical_B=2, T=512)
    L = w.n_layers
    say("workload 4 layers, 2 records x 512 tokens, whole outputs")
    As = [datagen.host_tensor(w, l, 0) for l in range(L)]
    Gs = [datagen.host_tensor(w, l, 1) for l in range(L)]
    from _helpers import gpu_step
    r0 = gpu_step(w, As, Gs, DEV, flags=dp.NO_NOISE)
    r = gpu_step(w, As, Gs, DEV, plan=r0["plan"], ws=r0["ws"])
    assert r0["plan"].layer_info(0)[0] == dp.PATH_GRAM
    assert r0["status"] == dp.OK and r["status"] == dp.OK
    say("workload 4 long records oracle")
    ref = oracle.step(As, Gs, w.C, w.sigma, 0, 0)
    tol = TOL[BF16]
    assert max_rel(r["n"], ref["n"]) <= tol and max_rel(r["c"], ref["c"]) <= tol
    e0 = rel_err(flat(r0["out"]), flat(ref["S"]))
    e1 = rel_err(flat(r["out"]), flat(ref["S_noised"]))
    say(f"  pre-noise {e0:.2e}, noised {e1:.2e}")
    assert e0 <= tol and e1 <= tol


def test_workload5_virtual_step_whole_outputs():
    """Workload 5 (48 LoRA layers, 4096 logical records in 16 physical batches of 256, C = 1) as the
    benchmark runs it: dpsgd_step with NO_NOISE per physical batch (ACCUMULATE after the first),
    then the noise once; layers 10 (1024 -> 8) and 37 (8 -> 1024) carry inputs."""
    w = datagen.workload(5)
    L, B = w.n_layers, w.B
    live = (10, 37)
    plan = dp.Plan(w.layers, w.dtype, B, w.T)
    ws = plan.workspace(DEV)
    zero = torch.zeros(B * w.T * 1024, dtype=torch.int16, device=DEV)
    out = [torch.full((a * b,), float("nan"), dtype=torch.float32, device=DEV) for a, b in w.layers]
    ns, cs = [], []
    for p in range(w.n_phys):
        say("workload 5 whole step, physical batch", p)
        dA, dG = _live_inputs(w, live, p * B, B, zero)
        nrm = torch.empty(B, dtype=torch.float32, device=DEV)
        cf = torch.empty(B, dtype=torch.float32, device=DEV)
        dp.step(plan, dA, dG, out, ws, w.C, w.sigma, 0, 0,
                flags=dp.NO_NOISE | (dp.ACCUMULATE if p else 0), norms_out=nrm, clip_out=cf)
        ns.append(nrm.cpu().numpy())
        cs.append(cf.cpu().numpy())
        del dA, dG
    assert dp.status(plan, ws) == dp.OK
    pre = [o.cpu().numpy() for o in out]
    dp.noise(plan, out, w.C, w.sigma, 0, 0, ws=ws)
    assert dp.status(plan, ws) == dp.OK
    noised = [o.cpu().numpy() for o in out]
    say("workload 5 oracle over the live layers, 16 physical batches")
    batches = [([datagen.host_tensor(w, l, 0, p * B, B) for l in live],
                [datagen.host_tensor(w, l, 1, p * B, B) for l in live]) for p in range(w.n_phys)]
    ref = oracle.step(None, None, w.C, w.sigma, 0, 0, batches=batches, noise=False)
    del batches
    tol = TOL[BF16]
    assert max_rel(np.concatenate(ns), ref["n"]) <= tol and max_rel(np.concatenate(cs), ref["c"]) <= tol
    assert np.all(ref["c"] < 1.0)
    _check_whole(w, plan, live, ref, pre, noised, 0, 0, tol)
