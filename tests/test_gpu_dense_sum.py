"""GPU parity of the clipped sum of dense bf16 layers (the MFMA GEMM kernels) against the oracle.

Both kernels are covered: the token-major copy kernel (T a multiple of 32, rows 16-byte aligned)
and the register-staging kernel (any T; also misaligned rows).  Cases span ragged tiles, one to
many record splits, accumulation, per-record factors over six orders of magnitude (the factors
are applied to the fp32 accumulator in Horner form, so their ratios matter), and more than 64
records in one split.  Tolerance: relative Frobenius error 2e-3 (bf16 inputs, fp32 accumulation).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import datagen  # noqa: E402
import differentially_private_amd as dp  # noqa: E402
import oracle  # noqa: E402
from _helpers import TOL, flat, host_inputs, oracle_sum_entry, rel_err, to_device  # noqa: E402
from datagen import BF16  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
SHAPES = ((320, 272), (264, 520), (256, 128), (24, 40))


def say(*a):
    print(*a, flush=True)


def factors(B, seed):
    rng = np.random.default_rng(seed)
    return rng.permutation(np.geomspace(1e-3, 1e3, B)).astype(np.float32)


def workload(shapes, B, T, seed):
    return datagen.Workload(name="dense_sum", layers=tuple(shapes),
                            layer_names=tuple("l%d" % i for i in range(len(shapes))), dtype=BF16,
                            B=B, logical_B=B, T=T, C=1.0, sigma=0.0, data_seed=seed)


def run_sum(w, dA, dG, c, flags=0, out=None):
    plan = dp.Plan(w.layers, BF16, w.B, w.T, dp.PATH_DIRECT, dp.SUM_GEMM)
    ws = plan.workspace(DEV)
    if out is None:
        out = [torch.full((a * b,), float("nan"), dtype=torch.float32, device=DEV)
               for a, b in w.layers]
    dp.ws_init(plan, ws)
    dp.clipped_sum(plan, w.B, 0, w.n_layers, dA, dG, torch.from_numpy(c).to(DEV), out, ws,
                   flags=flags)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("T", [32, 64, 96, 48])
@pytest.mark.parametrize("B", [1, 5, 70])
def test_dense_sum_small(T, B):
    w = workload(SHAPES, B, T, 1000 + T + B)
    say("dense sum", "T", T, "B", B)
    As, Gs = host_inputs(w)
    c = factors(B, T * B)
    want = flat([oracle.layer_clipped_sum(a, g, c.astype(np.float64)) for a, g in zip(As, Gs)])
    dA = [to_device(a, DEV) for a in As]
    dG = [to_device(g, DEV) for g in Gs]
    out = run_sum(w, dA, dG, c)
    e = rel_err(flat([o.cpu().numpy() for o in out]), want)
    say(f"  rel err {e:.2e}")
    assert e <= TOL[BF16]
    # accumulate on top: the result doubles
    out = run_sum(w, dA, dG, c, flags=dp.ACCUMULATE, out=out)
    e2 = rel_err(flat([o.cpu().numpy() for o in out]), 2 * want)
    say(f"  accumulate rel err {e2:.2e}")
    assert e2 <= TOL[BF16]


def test_dense_sum_misaligned_rows():
    """Rows one element past a 16-byte boundary take the register-staging kernel at T = 64."""
    w = workload(SHAPES[:2], 5, 64, 77)
    As, Gs = host_inputs(w)
    c = factors(5, 3)
    want = flat([oracle.layer_clipped_sum(a, g, c.astype(np.float64)) for a, g in zip(As, Gs)])

    def shifted(x):
        t = to_device(x.reshape(-1), DEV)
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
        buf[1:].copy_(t)
        return buf[1:]
    out = run_sum(w, [shifted(a) for a in As], [shifted(g) for g in Gs], c)
    e = rel_err(flat([o.cpu().numpy() for o in out]), want)
    say(f"misaligned rel err {e:.2e}")
    assert e <= TOL[BF16]


def test_dense_sum_one_split_many_records():
    """A 4096 x 4096 layer (512 tiles: one split) over 70 records of 32 tokens: every workgroup
    walks all 70 records (more than one 64-record window of factors).  Sampled entries against
    the oracle, computed from gathered columns of the generator."""
    w = workload(((4096, 4096),), 70, 32, 4242)
    say("one split, 70 records")
    c = factors(70, 11)
    dA = [to_device(datagen.host_tensor(w, 0, 0), DEV)]
    dG = [to_device(datagen.host_tensor(w, 0, 1), DEV)]
    out = run_sum(w, dA, dG, c)[0].view(4096, 4096)
    rng = np.random.default_rng(5)
    idx = [(0, 0), (4095, 4095), (255, 128), (256, 127)] + \
        [tuple(int(v) for v in rng.integers(0, 4096, 2)) for _ in range(28)]
    got = np.array([float(out[j, k]) for j, k in idx])
    want = np.array([oracle_sum_entry(w, 0, j, k, c.astype(np.float64)) for j, k in idx])
    e = rel_err(got, want)
    say(f"  sampled rel err {e:.2e}")
    assert e <= TOL[BF16]
