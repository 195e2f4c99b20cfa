"""GPU parity of variable-length records (segment plans: user-level clipping, each user's
records' token rows concatenated) against the oracle.

The oracle sees the same users as fixed-length records zero-padded to the longest user (zero
rows add nothing to A^T G), the GPU sees the rows concatenated with an offset array.  Covered:
the page's Alice/Bao example, random lengths including empty and full segments on the direct
(STORED and GEMM sum) and Gram paths in fp32 and bf16, 24 random plans (shapes, users, paths and
sum policies), and full-length segments giving bitwise the fixed-length plan's results on the
direct path.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import datagen  # noqa: E402
import differentially_private_amd as dp  # noqa: E402
import oracle  # noqa: E402
from _helpers import TOL, flat, host_inputs, max_rel, rel_err, to_device  # noqa: E402
from datagen import BF16, F32  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def run_segments(layers, dtype, T, lens, rows_A, rows_G, C, sigma, path=dp.PATH_AUTO,
                 sum_policy=dp.SUM_AUTO, flags=0, seed=3, step=1):
    """rows_A / rows_G: per layer [total rows, d] host arrays (fp32 or bf16 bits)."""
    B = len(lens)
    plan = dp.Plan(layers, dtype, max(B, 1), T, path, sum_policy, segments=True)
    ws = plan.workspace(DEV)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    dp.ws_segments(plan, ws, offs)
    dA = [to_device(a, DEV) for a in rows_A]
    dG = [to_device(g, DEV) for g in rows_G]
    out = [torch.full((a * b,), float("nan"), dtype=torch.float32, device=DEV) for a, b in layers]
    nrm = torch.full((max(B, 1),), -1.0, dtype=torch.float32, device=DEV)
    cf = torch.full((max(B, 1),), -1.0, dtype=torch.float32, device=DEV)
    dp.step(plan, dA, dG, out, ws, C, sigma, seed, step, n_records=B, flags=flags, norms_out=nrm,
            clip_out=cf)
    st = dp.status(plan, ws)
    torch.cuda.synchronize()
    return {"n": nrm.cpu().numpy()[:B], "c": cf.cpu().numpy()[:B], "status": st,
            "out": [o.cpu().numpy().reshape(a, b) for o, (a, b) in zip(out, layers)]}


def test_alice_bao_user_level_on_gpu():
    """The page's example: Alice's tickets 0.5 and 5.0 form one user, Bao's 0.25 another; C = 1,
    no noise: user-clipped 1.00 and 0.25, sum 1.25 (0.625 after the public normaliser 2), and
    0.25 without Alice (0.125): the change is C / 2."""
    A = np.ones((3, 1), dtype=np.float32)
    G = np.array([[0.5], [5.0], [0.25]], dtype=np.float32)
    r = run_segments([(1, 1)], F32, 2, [2, 1], [A], [G], 1.0, 0.0)
    assert r["status"] == dp.OK
    assert np.allclose(r["n"] * r["c"], [1.0, 0.25], rtol=1e-6)
    with_alice = r["out"][0][0, 0] / 2
    r1 = run_segments([(1, 1)], F32, 2, [1], [A[2:]], [G[2:]], 1.0, 0.0)
    without_alice = r1["out"][0][0, 0] / 2
    assert abs(with_alice - 0.625) < 1e-6 and abs(without_alice - 0.125) < 1e-7
    assert abs((with_alice - without_alice) - 0.5) < 1e-6


CASES = [
    ("lora_f32", ((64, 8), (8, 64)), F32, 40, dp.PATH_AUTO, dp.SUM_AUTO),
    ("lora_f32_gemm", ((64, 8), (8, 64)), F32, 40, dp.PATH_AUTO, dp.SUM_GEMM),
    ("bf16_gram", ((48, 40), (40, 48)), BF16, 24, dp.PATH_AUTO, dp.SUM_GEMM),
    ("bf16_direct_stored", ((48, 40), (40, 48)), BF16, 24, dp.PATH_DIRECT, dp.SUM_STORED),
    # gradient blocks of whole 128-wide tiles kept in store order, the partial last tile natural
    ("bf16_direct_stored_wide", ((300, 8), (8, 300)), BF16, 24, dp.PATH_DIRECT, dp.SUM_STORED),
    ("f32_direct_stored_wide", ((260, 12), (12, 260)), F32, 24, dp.PATH_DIRECT, dp.SUM_STORED),
    ("bf16_dense_gram", ((320, 272),), BF16, 48, dp.PATH_GRAM, dp.SUM_GEMM),
    ("f32_gram", ((96, 80),), F32, 33, dp.PATH_GRAM, dp.SUM_AUTO),
]


def _segment_case(name, layers, dtype, T, path, sum_policy, lens, C, sigma, data_seed):
    """The users of `lens` through a segment plan against the oracle on the same users zero-padded
    to T rows: norms, factors, noised and pre-noise sums."""
    B = len(lens)
    say("segments", name, "dtype", dtype, "path", path, "sum", sum_policy, "T", T, "lengths", list(lens))
    w = datagen.Workload(name=name, layers=layers, layer_names=tuple("l%d" % i for i in range(len(layers))),
                         dtype=dtype, B=B, logical_B=B, T=T, C=C, sigma=sigma, data_seed=data_seed)
    As, Gs = host_inputs(w)
    # oracle: users as fixed-length records, rows past each user's length zeroed
    zero = np.uint16(0) if dtype == BF16 else np.float32(0)
    Ap = [a.copy() for a in As]
    Gp = [g.copy() for g in Gs]
    for l in range(len(layers)):
        for i, n in enumerate(lens):
            Ap[l][i, n:] = zero
            Gp[l][i, n:] = zero
    ref = oracle.step(Ap, Gp, w.C, w.sigma, 3, 1)
    # GPU: each user's rows concatenated
    rows_A = [np.concatenate([a[i, :n] for i, n in enumerate(lens)]) for a in As]
    rows_G = [np.concatenate([g[i, :n] for i, n in enumerate(lens)]) for g in Gs]
    r = run_segments(layers, dtype, T, lens, rows_A, rows_G, w.C, w.sigma, path, sum_policy)
    assert r["status"] == dp.OK
    tol = TOL[dtype]
    en, ec = max_rel(r["n"], ref["n"]), max_rel(r["c"], ref["c"])
    eS = rel_err(flat(r["out"]), flat(ref["S_noised"]))
    say(f"  norm {en:.2e} clip {ec:.2e} noised sum {eS:.2e}")
    for i, n in enumerate(lens):
        if n == 0:
            assert r["n"][i] == 0.0 and r["c"][i] == 1.0        # an empty user
    assert en <= tol and ec <= tol and eS <= tol
    r0 = run_segments(layers, dtype, T, lens, rows_A, rows_G, w.C, w.sigma, path, sum_policy,
                      flags=dp.NO_NOISE)
    e0 = rel_err(flat(r0["out"]), flat(ref["S"]))
    say(f"  pre-noise sum {e0:.2e}")
    assert e0 <= tol


@pytest.mark.parametrize("name,layers,dtype,T,path,sum_policy", CASES)
def test_segments_match_oracle(name, layers, dtype, T, path, sum_policy):
    B = 7
    rng = np.random.default_rng(len(name) + T)
    lens = rng.integers(0, T + 1, B)
    lens[0], lens[1] = 0, T             # an empty user and a full-length one
    _segment_case(name, layers, dtype, T, path, sum_policy, lens, 0.7, 0.9, 700 + T)


def _random_segment_case(i):
    rng = np.random.default_rng(6100 + i)
    dtype = F32 if i % 2 == 0 else BF16
    layers = tuple((int(rng.integers(1, 200)), int(rng.integers(1, 40))) if rng.random() < 0.6
                   else (int(rng.integers(17, 200)), int(rng.integers(17, 200)))
                   for _ in range(int(rng.integers(1, 4))))
    T = int(rng.integers(1, 130))
    B = int(rng.integers(1, 25))
    lens = rng.integers(0, T + 1, B)
    if B > 2 and rng.random() < 0.5:
        lens[rng.integers(0, B)] = 0
    path = int(rng.choice([dp.PATH_AUTO, dp.PATH_GRAM, dp.PATH_DIRECT]))
    sum_policy = int(rng.choice([dp.SUM_AUTO, dp.SUM_GEMM, dp.SUM_STORED]))
    return dict(name=f"rseg{i}", layers=layers, dtype=dtype, T=T, path=path, sum_policy=sum_policy,
                lens=lens, C=float(rng.choice([0.2, 1.0, 30.0])), sigma=0.6, data_seed=6200 + i)


@pytest.mark.parametrize("i", range(24))
def test_random_segment_plans(i):
    """Random segment plans: 1-3 layers (LoRA-like or wide), fp32 and bf16, 1-24 users of 0-T rows,
    every path and sum policy."""
    _segment_case(**_random_segment_case(i))


def test_full_length_segments_equal_fixed_records():
    """Segments that all have T rows are the fixed-length layout: on the fp32 direct path the
    norms, factors and noised sum are bitwise those of the plan without segments."""
    w = datagen.reduced(2)
    As, Gs = host_inputs(w)
    lens = [w.T] * w.B
    rows_A = [a.reshape(-1, a.shape[2]) for a in As]
    rows_G = [g.reshape(-1, g.shape[2]) for g in Gs]
    r = run_segments(w.layers, w.dtype, w.T, lens, rows_A, rows_G, w.C, w.sigma)
    plan = dp.Plan(w.layers, w.dtype, w.B, w.T)
    ws = plan.workspace(DEV)
    out = [torch.empty(a * b, dtype=torch.float32, device=DEV) for a, b in w.layers]
    nrm = torch.empty(w.B, dtype=torch.float32, device=DEV)
    dp.step(plan, [to_device(a, DEV) for a in As], [to_device(g, DEV) for g in Gs], out, ws, w.C,
            w.sigma, 3, 1, norms_out=nrm)
    torch.cuda.synchronize()
    assert np.array_equal(r["n"], nrm.cpu().numpy())
    assert all(np.array_equal(a.reshape(-1), b.cpu().numpy()) for a, b in zip(r["out"], out))
