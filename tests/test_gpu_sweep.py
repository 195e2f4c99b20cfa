"""Seeded random sweeps of the HIP path against the oracle.

- The fused tail of plans whose layers all keep their gradient blocks (direct path, SUM_STORED): random layer
  shapes and counts give workgroups of one to eight wavefronts; layers whose sizes are not
  multiples of 4 take the element-wise variant; more than 1024 records put the clip factors in a
  separate launch; more than 48 layers split the tail into several launches.  Norms and clip
  factors (relative 1e-5 fp32 / 2e-3 bf16), the pre-noise sum and the noised sum (relative
  Frobenius, same bounds) are compared.
- The bf16 Gram path for records of at most 256 tokens (one workgroup per record and layer):
  random T, widths (multiples of 32) and record counts; per-layer squared norms against the
  oracle.
- The largest record count a plan accepts, on every path.
- The GEMM clipped sums (tile engine with record splits; dense kernels for wide bf16 layers, both
  the copy kernel and the register kernel) on random plans.
"""
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


def say(*a):
    print(*a, flush=True)


def _stored_case(i):
    rng = np.random.default_rng(7000 + i)
    dtype = F32 if i % 2 == 0 else BF16
    n_layers = int(rng.integers(1, 7))
    layers = []
    for _ in range(n_layers):
        if rng.random() < 0.5:   # sizes that are multiples of 4 (vector tail) or not
            layers.append((int(4 * rng.integers(1, 25)), int(4 * rng.integers(1, 25))))
        else:
            layers.append((int(rng.integers(1, 90)), int(rng.integers(1, 90))))
    return dict(dtype=dtype, layers=tuple(layers), B=int(rng.integers(1, 21)), T=int(rng.integers(1, 49)),
                seed=8000 + i)


STORED_CASES = [_stored_case(i) for i in range(12)] + [
    dict(dtype=F32, layers=((4, 4), (3, 5)), B=1100, T=2, seed=9001),        # clip factors outside
    dict(dtype=F32, layers=tuple((4, 8) if l % 3 else (5, 3) for l in range(50)), B=5, T=3,
         seed=9002),                                                          # two tail launches
    dict(dtype=BF16, layers=((768, 8), (8, 768), (1024, 8)), B=7, T=40, seed=9003),  # wide layers
    # stored-block order: whole 128-wide tiles kept in store order and the partial last tile in
    # natural order (wide dimension 300 or 260), rows moving (wide d_in) or, for bf16, 4-column
    # chunks moving (wide d_out), two 16-row blocks (d 36), and widths whose d_out is not a
    # multiple of 4 (natural order throughout)
    dict(dtype=F32, layers=((300, 8), (8, 300), (260, 12), (12, 260), (384, 36), (36, 384), (130, 6),
                            (6, 130)), B=6, T=20, seed=9004),
    dict(dtype=BF16, layers=((300, 8), (8, 300), (260, 12), (12, 260), (384, 36), (36, 384), (130, 6),
                             (6, 130)), B=6, T=40, seed=9005),
]


@pytest.mark.parametrize("case", range(len(STORED_CASES)))
def test_stored_tail_sweep(case):
    c = STORED_CASES[case]
    w = datagen.Workload(name=f"sweep{case}", layers=c["layers"],
                         layer_names=tuple(f"l{l}" for l in range(len(c["layers"]))), dtype=c["dtype"],
                         B=c["B"], logical_B=c["B"], T=c["T"], C=1.0, sigma=0.7, data_seed=c["seed"])
    say("stored sweep", case, "dtype", c["dtype"], "B", c["B"], "T", c["T"], "layers", len(c["layers"]),
        c["layers"][:4])
    As, Gs = host_inputs(w)
    ref = oracle.step(As, Gs, w.C, w.sigma, 3, 11)
    r = gpu_step(w, As, Gs, DEV, seed=3, step=11, path=dp.PATH_DIRECT, sum_policy=dp.SUM_STORED)
    tol = TOL[w.dtype]
    en, ec = max_rel(r["n"], ref["n"]), max_rel(r["c"], ref["c"])
    eS = rel_err(flat(r["out"]), flat(ref["S_noised"]))
    r0 = gpu_step(w, As, Gs, DEV, seed=3, step=11, path=dp.PATH_DIRECT, sum_policy=dp.SUM_STORED,
                  flags=dp.NO_NOISE)
    e0 = rel_err(flat(r0["out"]), flat(ref["S"]))
    say(f"  norm {en:.2e} clip {ec:.2e} noised {eS:.2e} pre-noise {e0:.2e}")
    assert r["status"] == dp.OK and r0["status"] == dp.OK
    assert en <= tol and ec <= tol and eS <= tol and e0 <= tol


def _gram_case(i):
    rng = np.random.default_rng(7100 + i)
    n_layers = int(rng.integers(1, 4))
    layers = tuple((int(32 * rng.integers(1, 9)), int(32 * rng.integers(1, 9))) for _ in range(n_layers))
    return dict(layers=layers, B=int(rng.integers(1, 7)), T=int(rng.integers(1, 257)), seed=8100 + i)


GRAM_CASES = [_gram_case(i) for i in range(10)]


@pytest.mark.parametrize("case", range(len(GRAM_CASES)))
def test_gram_per_record_sweep(case):
    c = GRAM_CASES[case]
    shapes, B, T = c["layers"], c["B"], c["T"]
    w = datagen.Workload(name=f"gsweep{case}", layers=shapes,
                         layer_names=tuple(f"l{l}" for l in range(len(shapes))), dtype=BF16, B=B,
                         logical_B=B, T=T, C=1.0, sigma=0.0, data_seed=c["seed"])
    say("gram sweep", case, "T", T, "B", B, "layers", shapes)
    As, Gs = host_inputs(w)
    want = np.stack([oracle.layer_norm2(a, g) for a, g in zip(As, Gs)])
    plan = dp.Plan(shapes, BF16, B, T, dp.PATH_GRAM)
    ws = plan.workspace(DEV)
    dA = [to_device(a, DEV) for a in As]
    dG = [to_device(g, DEV) for g in Gs]
    dp.ws_init(plan, ws)
    dp.norms(plan, B, 0, len(shapes), dA, dG, ws)
    out = torch.empty(len(shapes) * B, dtype=torch.float32, device=DEV)
    dp.layer_norm2(plan, B, 0, len(shapes), ws, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(len(shapes), B).astype(np.float64)
    e = max_rel(got, want)
    say(f"  rel {e:.2e}")
    assert e <= TOL[BF16]


# The largest record count a plan accepts (65535), on every path, with tiny layers: one
# workgroup row per record in the norm launches, clip factors in their own launch, the fused
# tail's record loop and the GEMM sums' record splits all at their widest.
MAX_RECORD_CASES = [
    (F32, dp.PATH_GRAM, dp.SUM_AUTO),
    (F32, dp.PATH_DIRECT, dp.SUM_STORED),
    (F32, dp.PATH_DIRECT, dp.SUM_GEMM),
    (BF16, dp.PATH_DIRECT, dp.SUM_STORED),
    (BF16, dp.PATH_GRAM, dp.SUM_AUTO),
]


@pytest.mark.parametrize("case", range(len(MAX_RECORD_CASES)))
def test_maximum_record_count(case):
    dtype, path, sum_policy = MAX_RECORD_CASES[case]
    B, T, layers = 65535, 2, ((4, 3), (3, 5))
    w = datagen.Workload(name=f"maxrec{case}", layers=layers, layer_names=("l0", "l1"), dtype=dtype,
                         B=B, logical_B=B, T=T, C=1.0, sigma=0.5, data_seed=9100 + case)
    say("max records", case, "dtype", dtype, "path", path, "sum", sum_policy, "B", B)
    As, Gs = host_inputs(w)
    ref = oracle.step(As, Gs, w.C, w.sigma, 5, 2)
    r = gpu_step(w, As, Gs, DEV, seed=5, step=2, path=path, sum_policy=sum_policy)
    r0 = gpu_step(w, As, Gs, DEV, seed=5, step=2, path=path, sum_policy=sum_policy, flags=dp.NO_NOISE)
    tol = TOL[dtype]
    en, ec = max_rel(r["n"], ref["n"]), max_rel(r["c"], ref["c"])
    eS = rel_err(flat(r["out"]), flat(ref["S_noised"]))
    e0 = rel_err(flat(r0["out"]), flat(ref["S"]))
    say(f"  norm {en:.2e} clip {ec:.2e} noised {eS:.2e} pre-noise {e0:.2e}")
    assert r["status"] == dp.OK and r0["status"] == dp.OK
    assert en <= tol and ec <= tol and eS <= tol and e0 <= tol


def _gemm_case(i):
    rng = np.random.default_rng(7200 + i)
    dtype = F32 if i % 2 == 0 else BF16
    n_layers = int(rng.integers(1, 4))
    layers = []
    for _ in range(n_layers):
        if rng.random() < 0.5:   # both widths above 16: the dense kernels for bf16
            layers.append((int(rng.integers(17, 300)), int(rng.integers(17, 300))))
        else:
            layers.append((int(rng.integers(1, 120)), int(rng.integers(1, 40))))
    T = int(32 * rng.integers(1, 4)) if rng.random() < 0.5 else int(rng.integers(1, 97))
    return dict(dtype=dtype, layers=tuple(layers), B=int(rng.integers(1, 25)), T=T, seed=8200 + i,
                path=dp.PATH_GRAM if i % 5 == 4 else dp.PATH_DIRECT)


GEMM_CASES = [_gemm_case(i) for i in range(14)] + [
    dict(dtype=BF16, layers=((256, 128), (64, 512)), B=9, T=64, seed=9201, path=dp.PATH_DIRECT),  # copy kernel
    dict(dtype=BF16, layers=((200, 136),), B=13, T=50, seed=9202, path=dp.PATH_DIRECT),           # register kernel
    # more layers than one launch takes: the record splits are chosen per launch (here 20 and 12,
    # every split a single record), each launch followed by its split reduce
    dict(dtype=F32, layers=tuple((64, 8) if l % 2 else (8, 64) for l in range(100)), B=20, T=16,
         seed=9203, path=dp.PATH_DIRECT),                                                        # 3 launches
    dict(dtype=BF16, layers=tuple((300, 12) if l % 2 else (12, 300) for l in range(60)) + ((64, 64),) * 3,
         B=12, T=32, seed=9204, path=dp.PATH_DIRECT),                                            # 2 + dense
]


@pytest.mark.parametrize("case", range(len(GEMM_CASES)))
def test_gemm_sum_sweep(case):
    """The GEMM clipped sums (the tile engine with its record splits, and for bf16 layers wider than
    16 in both dimensions the dense kernels) on random plans: norms, factors, pre-noise and noised
    sums against the oracle."""
    c = GEMM_CASES[case]
    w = datagen.Workload(name=f"gsum{case}", layers=c["layers"],
                         layer_names=tuple(f"l{l}" for l in range(len(c["layers"]))), dtype=c["dtype"],
                         B=c["B"], logical_B=c["B"], T=c["T"], C=1.0, sigma=0.3, data_seed=c["seed"])
    say("gemm sweep", case, "dtype", c["dtype"], "path", c["path"], "B", c["B"], "T", c["T"], c["layers"])
    As, Gs = host_inputs(w)
    ref = oracle.step(As, Gs, w.C, w.sigma, 4, 9)
    r = gpu_step(w, As, Gs, DEV, seed=4, step=9, path=c["path"], sum_policy=dp.SUM_GEMM)
    r0 = gpu_step(w, As, Gs, DEV, seed=4, step=9, path=c["path"], sum_policy=dp.SUM_GEMM,
                  flags=dp.NO_NOISE)
    tol = TOL[w.dtype]
    en, ec = max_rel(r["n"], ref["n"]), max_rel(r["c"], ref["c"])
    eS = rel_err(flat(r["out"]), flat(ref["S_noised"]))
    e0 = rel_err(flat(r0["out"]), flat(ref["S"]))
    say(f"  norm {en:.2e} clip {ec:.2e} noised {eS:.2e} pre-noise {e0:.2e}")
    assert r["status"] == dp.OK and r0["status"] == dp.OK
    assert en <= tol and ec <= tol and eS <= tol and e0 <= tol
