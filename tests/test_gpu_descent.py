"""GPU parity of the fused descent step (phase 5: theta <- theta - lr * noised sum / L, applied in
the noise epilogue) against the oracle.

Parameters are fp32 and updated in place, so the GPU result is compared with the oracle's
float64 update within the step's tolerance (1e-5 fp32 / 2e-3 bf16, relative to the update's
Frobenius norm) plus the fp32 rounding of the parameters themselves.  Both epilogues are
covered: the fused clip + sum + noise kernel (layers that keep gradient blocks) and the noise
kernel (GEMM layers), plus virtual batching, an empty batch at the page's parameters, and a
nonfinite norm (parameters untouched).
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
from _helpers import TOL, flat, host_inputs, rel_err, to_device  # noqa: E402
from datagen import F32  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
LR = 0.01


def say(*a):
    print(*a, flush=True)


def thetas(w, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((a, b)).astype(np.float32) for a, b in w.layers]


def check_params(got, theta0, ref_theta, tol):
    """||theta_gpu - theta_oracle|| within tol of the update's norm plus the fp32 spacing of the
    parameters (the GPU's parameters are fp32)."""
    g = flat(got)
    o = flat(ref_theta)
    upd = o - flat(theta0)
    spacing = np.spacing(np.abs(o).astype(np.float32)).astype(np.float64)
    err = np.linalg.norm(g - o)
    bound = tol * np.linalg.norm(upd) + np.linalg.norm(spacing)
    say(f"  params err {err:.3e} bound {bound:.3e} (update norm {np.linalg.norm(upd):.3e})")
    assert err <= bound


def run(w, As, Gs, theta0, flags=0, sum_policy=dp.SUM_AUTO, descend=True, n=None):
    n = w.B if n is None else n
    plan = dp.Plan(w.layers, w.dtype, max(w.B, 1), w.T, dp.PATH_AUTO, sum_policy)
    ws = plan.workspace(DEV)
    dA = [to_device(a, DEV) for a in As]
    dG = [to_device(g, DEV) for g in Gs]
    out = [torch.full((a * b,), float("nan"), dtype=torch.float32, device=DEV) for a, b in w.layers]
    th = [torch.from_numpy(t.reshape(-1).copy()).to(DEV) for t in theta0]
    dp.step(plan, dA, dG, out, ws, w.C, w.sigma, 5, 3, n_records=n, flags=flags,
            params=th if descend else None, lr=LR, normalizer=float(max(w.B, 1)))
    st = dp.status(plan, ws)
    torch.cuda.synchronize()
    return ([o.cpu().numpy().reshape(a, b) for o, (a, b) in zip(out, w.layers)],
            [t.cpu().numpy().reshape(a, b) for t, (a, b) in zip(th, w.layers)], st)


@pytest.mark.parametrize("idx,sum_policy", [(2, dp.SUM_AUTO), (2, dp.SUM_GEMM), (3, dp.SUM_AUTO),
                                            (4, dp.SUM_AUTO), (1, dp.SUM_AUTO)])
def test_descent_matches_oracle(idx, sum_policy):
    w = datagen.reduced(idx).with_(logical_B=datagen.reduced(idx).B)
    say("descent", w.name, "sum", sum_policy)
    As, Gs = host_inputs(w)
    theta0 = thetas(w, idx)
    ref = oracle.step(As, Gs, w.C, w.sigma, 5, 3, descent_args=(theta0, LR, float(w.B)))
    out, th, st = run(w, As, Gs, theta0, sum_policy=sum_policy)
    assert st == dp.OK
    e = rel_err(flat(out), flat(ref["S_noised"]))
    say(f"  noised sum {e:.2e}")
    assert e <= TOL[w.dtype]
    check_params(th, theta0, ref["theta"], TOL[w.dtype])
    # descending does not change the released sum: out is bitwise the plain step's
    out_plain, th_plain, _ = run(w, As, Gs, theta0, sum_policy=sum_policy, descend=False)
    assert all(np.array_equal(a, b) for a, b in zip(out, out_plain))
    assert all(np.array_equal(a, b) for a, b in zip(th_plain, theta0))


def test_descent_virtual_batching():
    """Three physical batches accumulated without noise, then noise + descent once."""
    w = datagen.reduced(5)
    say("descent virtual batching", w.name)
    plan = dp.Plan(w.layers, w.dtype, w.B, w.T)
    ws = plan.workspace(DEV)
    out = [torch.empty(a * b, dtype=torch.float32, device=DEV) for a, b in w.layers]
    theta0 = thetas(w, 55)
    th = [torch.from_numpy(t.reshape(-1).copy()).to(DEV) for t in theta0]
    batches = []
    for p in range(w.n_phys):
        As, Gs = host_inputs(w, first=p * w.B)
        batches.append((As, Gs))
        dp.step(plan, [to_device(a, DEV) for a in As], [to_device(g, DEV) for g in Gs], out, ws,
                w.C, w.sigma, 9, 2, flags=dp.NO_NOISE | (dp.ACCUMULATE if p else 0))
    dp.noise(plan, out, w.C, w.sigma, 9, 2, ws=ws, params=th, lr=LR, normalizer=float(w.logical_B))
    assert dp.status(plan, ws) == dp.OK
    ref = oracle.step(None, None, w.C, w.sigma, 9, 2, batches=batches,
                      descent_args=(theta0, LR, float(w.logical_B)))
    e = rel_err(flat([o.cpu().numpy() for o in out]), flat(ref["S_noised"]))
    assert e <= TOL[w.dtype]
    check_params([t.cpu().numpy() for t in th], theta0, ref["theta"], TOL[w.dtype])


def test_descent_empty_batch_page_rms():
    """An empty batch releases noise only: from theta0 = 0 over d = 5e6 coordinates with sigma*C
    = 1, lr = 0.01, L = 128 the step's norm is the page's step-noise RMS 0.17 (within 5 standard
    deviations of lr * sqrt(d) / L), and matches the oracle's step."""
    di, do = 5000, 1000
    d = di * do
    w = datagen.Workload(name="pure_noise", layers=((di, do),), layer_names=("l0",), dtype=F32,
                         B=1, logical_B=1, T=1, C=1.0, sigma=1.0, data_seed=1)
    plan = dp.Plan(w.layers, F32, 1, 1)
    ws = plan.workspace(DEV)
    out = [torch.empty(d, dtype=torch.float32, device=DEV)]
    th = [torch.zeros(d, dtype=torch.float32, device=DEV)]
    dp.ws_init(plan, ws)
    dA = [torch.empty(di, dtype=torch.float32, device=DEV)]
    dG = [torch.empty(do, dtype=torch.float32, device=DEV)]
    dp.step(plan, dA, dG, out, ws, 1.0, 1.0, 0, 0, n_records=0, params=th, lr=0.01, normalizer=128.0)
    assert dp.status(plan, ws) == dp.OK
    t = th[0].cpu().numpy().astype(np.float64)
    norm = np.linalg.norm(t)
    say(f"pure-noise step norm {norm:.6f}")
    assert round(norm, 2) == 0.17
    assert abs(norm - 0.01 * math.sqrt(d) / 128) < 5 * 0.01 / (128 * math.sqrt(2))
    ref = oracle.step([np.zeros((0, 1, di))], [np.zeros((0, 1, do))], 1.0, 1.0, 0, 0,
                      descent_args=([np.zeros((di, do))], 0.01, 128.0))
    check_params([t.reshape(di, do)], [np.zeros((di, do))], ref["theta"], TOL[F32])


@pytest.mark.parametrize("idx", [2, 4])
def test_descent_skipped_on_nonfinite_norm(idx):
    """A NaN input makes a norm nonfinite: the status says so, and neither out nor the
    parameters are written."""
    w = datagen.reduced(idx).with_(logical_B=datagen.reduced(idx).B)
    As, Gs = host_inputs(w)
    As = [a.copy() for a in As]
    if As[0].dtype == np.uint16:
        As[0][1, 0, 0] = 0x7FC0      # bf16 NaN
    else:
        As[0][1, 0, 0] = np.nan
    theta0 = thetas(w, 7)
    out, th, st = run(w, As, Gs, theta0)
    assert st == dp.ERR_NONFINITE
    assert all(np.array_equal(a, b) for a, b in zip(th, theta0))
    assert all(np.isnan(o).all() for o in out)
