"""Random plans through dpsgd_step against the oracle: 1-5 layers of random widths (narrow,
LoRA-like and wide), fp32 or bf16, 1-39 records, T of 1-139 tokens or whole 32-token steps, every
path policy and sum policy, C spanning clipped and unclipped records.  Norms, clip factors, the
pre-noise sum and the noised sum must meet the fp32 / bf16 bounds.  DPSGD_FUZZ_CASES (default 60)
and DPSGD_FUZZ_SEED (default 100) set the number of plans and the first seed.  Twelve more plans
run as virtual batches (2-5 physical batches, the last one shorter, noise once)."""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import datagen  # noqa: E402
import differentially_private_amd as dp  # noqa: E402
import oracle  # noqa: E402
from _helpers import TOL, flat, gpu_step, host_inputs, max_rel, rel_err, to_device  # noqa: E402
from datagen import BF16, F32  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
N_CASES = int(os.environ.get("DPSGD_FUZZ_CASES", "60"))
SEED0 = int(os.environ.get("DPSGD_FUZZ_SEED", "100"))


def _plan(i):
    rng = np.random.default_rng(SEED0 + i)
    dtype = F32 if rng.random() < 0.5 else BF16
    layers = []
    for _ in range(int(rng.integers(1, 6))):
        r = rng.random()
        if r < 0.3:
            layers.append((int(rng.integers(1, 20)), int(rng.integers(1, 20))))
        elif r < 0.7:
            layers.append((int(rng.integers(1, 400)), int(rng.integers(1, 24))))
        else:
            layers.append((int(rng.integers(17, 260)), int(rng.integers(17, 260))))
    if rng.random() < 0.25:
        layers = [(b, a) for a, b in layers]
    B = int(rng.integers(1, 40))
    T = int(rng.choice([int(rng.integers(1, 140)), 32 * int(rng.integers(1, 5))]))
    path = int(rng.choice([dp.PATH_AUTO, dp.PATH_GRAM, dp.PATH_DIRECT]))
    sum_policy = int(rng.choice([dp.SUM_AUTO, dp.SUM_GEMM, dp.SUM_STORED]))
    C = float(rng.choice([0.1, 1.0, 50.0]))
    return dtype, tuple(layers), B, T, path, sum_policy, C


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_plan(i):
    dtype, layers, B, T, path, sum_policy, C = _plan(i)
    print("fuzz", SEED0 + i, dtype, path, sum_policy, B, T, C, layers, flush=True)
    w = datagen.Workload(name=f"fuzz{i}", layers=layers, layer_names=tuple(f"l{l}" for l in range(len(layers))),
                         dtype=dtype, B=B, logical_B=B, T=T, C=C, sigma=0.4, data_seed=20000 + SEED0 + i)
    As, Gs = host_inputs(w)
    ref = oracle.step(As, Gs, w.C, w.sigma, 6, 1)
    r0 = gpu_step(w, As, Gs, DEV, seed=6, step=1, path=path, sum_policy=sum_policy, flags=dp.NO_NOISE)
    r = gpu_step(w, As, Gs, DEV, seed=6, step=1, path=path, sum_policy=sum_policy)
    tol = TOL[dtype]
    assert r["status"] == dp.OK and r0["status"] == dp.OK
    assert max_rel(r["n"], ref["n"]) <= tol and max_rel(r["c"], ref["c"]) <= tol
    assert rel_err(flat(r0["out"]), flat(ref["S"])) <= tol
    assert rel_err(flat(r["out"]), flat(ref["S_noised"])) <= tol


@pytest.mark.parametrize("i", range(12))
def test_random_virtual_batches(i):
    """A random plan run as 2-5 physical batches (the last one shorter) accumulated into one
    output, noise drawn once at the end: equal to the oracle's logical step."""
    dtype, layers, B, T, path, sum_policy, C = _plan(1000 + i)
    rng = np.random.default_rng(SEED0 + 5000 + i)
    n_phys = int(rng.integers(2, 6))
    last = int(rng.integers(1, B + 1))
    sizes = [B] * (n_phys - 1) + [last]
    print("virtual", dtype, path, sum_policy, B, T, C, layers, sizes, flush=True)
    w = datagen.Workload(name=f"vfuzz{i}", layers=layers, layer_names=tuple(f"l{l}" for l in range(len(layers))),
                         dtype=dtype, B=B, logical_B=sum(sizes), T=T, C=C, sigma=0.4,
                         data_seed=40000 + SEED0 + i)
    plan = dp.Plan(layers, dtype, B, T, path, sum_policy)
    ws = plan.workspace(DEV)
    out = [torch.empty(a * b, dtype=torch.float32, device=DEV) for a, b in layers]
    batches, ns, cs, first = [], [], [], 0
    for p, nb in enumerate(sizes):
        As, Gs = host_inputs(w, first=first, n=nb)
        first += nb
        batches.append((As, Gs))
        nrm = torch.empty(B, dtype=torch.float32, device=DEV)
        cf = torch.empty(B, dtype=torch.float32, device=DEV)
        flags = dp.NO_NOISE | (dp.ACCUMULATE if p else 0)
        dp.step(plan, [to_device(a, DEV) for a in As], [to_device(g, DEV) for g in Gs], out, ws, C,
                w.sigma, 2, 5, n_records=nb, flags=flags, norms_out=nrm, clip_out=cf)
        ns.append(nrm.cpu().numpy()[:nb])
        cs.append(cf.cpu().numpy()[:nb])
    pre = flat([o.cpu().numpy() for o in out])
    dp.noise(plan, out, C, w.sigma, 2, 5, ws=ws)
    assert dp.status(plan, ws) == dp.OK
    ref = oracle.step(None, None, C, w.sigma, 2, 5, batches=batches)
    tol = TOL[dtype]
    assert max_rel(np.concatenate(ns), ref["n"]) <= tol
    assert max_rel(np.concatenate(cs), ref["c"]) <= tol
    assert rel_err(pre, flat(ref["S"])) <= tol
    assert rel_err(flat([o.cpu().numpy() for o in out]), flat(ref["S_noised"])) <= tol


def _plan_many(i):
    rng = np.random.default_rng(SEED0 + 9000 + i)
    dtype = F32 if rng.random() < 0.5 else BF16
    layers = [(int(rng.integers(1, 65)), int(rng.integers(1, 17))) for _ in range(int(rng.integers(1, 4)))]
    if rng.random() < 0.5:
        layers = [(b, a) for a, b in layers]
    B = int(rng.integers(65, 401))
    T = int(rng.integers(1, 65))
    path = int(rng.choice([dp.PATH_AUTO, dp.PATH_GRAM, dp.PATH_DIRECT]))
    sum_policy = int(rng.choice([dp.SUM_AUTO, dp.SUM_GEMM, dp.SUM_STORED]))
    C = float(rng.choice([0.1, 1.0, 50.0]))
    return dtype, tuple(layers), B, T, path, sum_policy, C


@pytest.mark.parametrize("i", range(12))
def test_random_plan_many_records(i):
    """65-400 records: the clip factors go over many workgroups (the last one partly filled), each
    record's reduction the same as in one workgroup; small layers keep the oracle fast."""
    dtype, layers, B, T, path, sum_policy, C = _plan_many(i)
    print("fuzz many", dtype, path, sum_policy, B, T, C, layers, flush=True)
    w = datagen.Workload(name=f"fuzzm{i}", layers=layers, layer_names=tuple(f"l{l}" for l in range(len(layers))),
                         dtype=dtype, B=B, logical_B=B, T=T, C=C, sigma=0.4, data_seed=60000 + SEED0 + i)
    As, Gs = host_inputs(w)
    ref = oracle.step(As, Gs, w.C, w.sigma, 6, 1)
    r0 = gpu_step(w, As, Gs, DEV, seed=6, step=1, path=path, sum_policy=sum_policy, flags=dp.NO_NOISE)
    r = gpu_step(w, As, Gs, DEV, seed=6, step=1, path=path, sum_policy=sum_policy)
    tol = TOL[dtype]
    assert r["status"] == dp.OK and r0["status"] == dp.OK
    assert max_rel(r["n"], ref["n"]) <= tol and max_rel(r["c"], ref["c"]) <= tol
    assert rel_err(flat(r0["out"]), flat(ref["S"])) <= tol
    assert rel_err(flat(r["out"]), flat(ref["S_noised"])) <= tol
    # every record's norm and factor bitwise the same when its batch runs at 64 records or fewer
    # (one clip workgroup) as at B (many)
    k = min(64, B)
    small = gpu_step(w, [a[:k] for a in As], [g[:k] for g in Gs], DEV, seed=6, step=1, path=path,
                     sum_policy=sum_policy, flags=dp.NO_NOISE)
    assert np.array_equal(small["n"], r["n"][:k]) and np.array_equal(small["c"], r["c"][:k])


def test_nonfinite_status_across_physical_batches_many_records():
    """Three physical batches of 200 records (clip factors over many workgroups), the second with a
    NaN record: the status stays NONFINITE through the third (ACCUMULATE ORs it), the sums and the
    noise are skipped, and the next logical step's first batch (no ACCUMULATE) clears it."""
    w = datagen.reduced(2).with_(B=200, logical_B=600, T=8)
    plan = dp.Plan(w.layers, w.dtype, w.B, w.T)
    ws = plan.workspace(DEV)
    out = [torch.full((a * b,), 7.0, dtype=torch.float32, device=DEV) for a, b in w.layers]
    for p in range(3):
        As, Gs = host_inputs(w, first=p * w.B, n=w.B)
        if p == 1:
            As[0] = As[0].copy()
            As[0][57, 3, :] = np.nan
        flags = dp.NO_NOISE | (dp.ACCUMULATE if p else 0)
        dp.step(plan, [to_device(a, DEV) for a in As], [to_device(g, DEV) for g in Gs], out, ws, w.C,
                w.sigma, 0, 0, flags=flags)
        assert dp.status(plan, ws) == (dp.OK if p == 0 else dp.ERR_NONFINITE)
    before = flat([o.cpu().numpy() for o in out])
    dp.noise(plan, out, w.C, w.sigma, 0, 0, ws=ws)
    assert np.array_equal(flat([o.cpu().numpy() for o in out]), before)
    As, Gs = host_inputs(w, first=3 * w.B, n=w.B)
    dp.step(plan, [to_device(a, DEV) for a in As], [to_device(g, DEV) for g in Gs], out, ws, w.C, w.sigma,
            0, 0, flags=dp.NO_NOISE)
    assert dp.status(plan, ws) == dp.OK
