"""Workloads 3, 4 and 5 at full size, in the configuration the benchmark runs, checked on sampled
outputs that the oracle computes one at a time (its full-size run would take hours):

- per-(record, layer) squared norms and the joint norm / clip factor of sampled records;
- entries of the clipped sum for caller-supplied factors, from gathered input columns;
- the noise added to every coordinate (all of them, against the oracle's stream);
- accumulation across all physical batches of the virtual batch (workload 5), with C = 1e30 so
  that every factor is 1 and any entry is a plain sum over all 4096 records.
Inputs are filled directly in HBM by the device generator, which is checked bit for bit against
the host generator the oracle uses.
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
    for (l, j, k) in picks:
        want = oracle_sum_entry(w, l, j, k, c, first, n)
        got = float(S_gpu_layers[l][j * w.layers[l][1] + k])
        scale = max(abs(want), 1e-30)
        assert abs(got - want) <= tol * scale + 1e-6 * tol, (l, j, k, got, want)


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
    picks = [(int(rng.integers(L)), int(rng.integers(4096)), int(rng.integers(4096))) for _ in range(24)]
    _check_sum_entries(w, S, c_test.astype(np.float64), picks, tol)
    # the whole step on this data: status OK and every record clipped (n ~ 131 >> C)
    nrm = torch.empty(B, dtype=torch.float32, device=DEV)
    dp.step(plan, As, Gs, out, ws, w.C, w.sigma, 0, 0, norms_out=nrm)
    assert dp.status(plan, ws) == dp.OK
    n = nrm.cpu().numpy()
    assert np.all(n > w.C) and np.all(np.isfinite(flat([o.cpu().numpy() for o in out])))


def test_workload5_full_virtual_batch():
    """4096 logical records in 16 physical batches of 256 (6.5 GB of inputs each): accumulation
    across all batches (C = 1e30: every factor 1, each entry a plain sum over 4096 records), norms
    of records from several batches, and noise drawn once."""
    w = datagen.workload(5)
    L, B = w.n_layers, w.B
    plan = dp.Plan(w.layers, w.dtype, B, w.T)
    ws = plan.workspace(DEV)
    out = [torch.empty(a * b, dtype=torch.float32, device=DEV) for a, b in w.layers]
    sampled = {0: None, 1000: None, 4095: None}
    for p in range(w.n_phys):
        say("workload 5 physical batch", p)
        As = [device_tensor(w, l, 0, p * B, B, DEV) for l in range(L)]
        Gs = [device_tensor(w, l, 1, p * B, B, DEV) for l in range(L)]
        nrm = torch.empty(B, dtype=torch.float32, device=DEV)
        flags = dp.NO_NOISE | (dp.ACCUMULATE if p else 0)
        dp.step(plan, As, Gs, out, ws, 1e30, w.sigma, 0, 0, flags=flags, norms_out=nrm)
        torch.cuda.synchronize()
        for r in sampled:
            if p * B <= r < (p + 1) * B:
                sampled[r] = float(nrm.cpu().numpy()[r - p * B])
        del As, Gs
    assert dp.status(plan, ws) == dp.OK
    S = [o.cpu().numpy() for o in out]
    rng = np.random.default_rng(5)
    picks = [(int(l), int(rng.integers(w.layers[l][0])), int(rng.integers(w.layers[l][1])))
             for l in rng.choice(L, 6, replace=False)]
    say("workload 5 sum entries over 4096 records", picks)
    _check_sum_entries(w, S, np.ones(w.logical_B), picks, TOL[BF16], 0, w.logical_B)
    for r, n_gpu in sampled.items():
        want = math.sqrt(oracle_record_layer_norm2(w, r, range(L)).sum())
        assert abs(n_gpu - want) <= TOL[BF16] * want, (r, n_gpu, want)
    pre = flat(S)
    dp.noise(plan, out, w.C, w.sigma, 7, 3, ws=ws)
    torch.cuda.synchronize()
    z_gpu = (flat([o.cpu().numpy() for o in out]) - pre) / (w.sigma * w.C)
    z = oracle.gauss(7, 3, 0, z_gpu.size)
    assert np.max(np.abs(z_gpu - z) / (1 + np.abs(z) + np.abs(pre) / (w.sigma * w.C))) <= 16 * 2.0 ** -24
