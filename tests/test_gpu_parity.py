"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Tolerances (relative): per-record norms and clip factors 1e-5 for fp32 inputs, 2e-3 for bf16;
clipped sum (pre-noise) and noised sum, relative Frobenius 1e-5 / 2e-3.  Philox words are compared
bit for bit; the normals Z within |dZ| <= 8 * 2^-24 * (1 + |Z|) (fp32 log/sqrt/sincos against the
oracle's fp64).  Integer, repeat and batch-invariance checks are bitwise.
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
from _helpers import TOL, flat, gpu_step, host_inputs, max_rel, rel_err, to_device  # noqa: E402
from datagen import BF16, F32  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------- noise stream

@pytest.mark.parametrize("seed,step,first,n", [(0, 0, 0, 1000), (0xDEADBEEF12345678, 7, 2**32 - 3, 777),
                                               (2**64 - 1, 2**64 - 1, 2**40, 513)])
def test_philox_raw_bitexact(seed, step, first, n):
    say("philox_raw", seed, step, first, n)
    out = torch.empty(4 * n, dtype=torch.int32, device=DEV)
    dp.philox_raw(seed, step, first, n, out)
    got = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, oracle.philox_words(seed, step, first, n))


def _noise_plan_and_out(layers, base=None):
    plan = dp.Plan(layers, dp.DTYPE_F32, 1, 1)
    out = [torch.zeros(a * b, dtype=torch.float32, device=DEV) for a, b in layers]
    if base is not None:
        for o, b in zip(out, base):
            o.copy_(torch.from_numpy(b))
    return plan, out


def test_noise_matches_oracle_ragged_layers():
    """Layers whose flat offsets are not multiples of 4 (blocks straddle layers)."""
    layers = [(3, 5), (7, 1), (64, 33), (1, 1), (130, 3), (8, 8)]
    say("noise ragged", layers)
    rng = np.random.default_rng(5)
    base = [rng.standard_normal(a * b).astype(np.float32) for a, b in layers]
    plan, out = _noise_plan_and_out(layers, base)
    sigma, C, seed, step = 1.3, 0.7, 12345, 3
    dp.noise(plan, out, C, sigma, seed, step)
    got = flat([o.cpu().numpy() for o in out])
    total = plan.n_params
    z = oracle.gauss(seed, step, 0, total)
    want = flat(base) + sigma * C * z
    z_gpu = (got - flat(base)) / (sigma * C)
    assert np.all(np.abs(z_gpu - z) <= 8 * 2.0 ** -24 * (1 + np.abs(z)) + 4e-7 * np.abs(flat(base)) / (sigma * C))
    assert rel_err(got, want) <= 1e-6


def test_noise_pure_z_and_statistics():
    """out = 0, sigma*C = 1 gives Z itself: per-element against the oracle, moments, and the
    page's sigma*C*sqrt(d) norm."""
    layers = [(768, 8), (8, 768)] * 24          # 294,912 coordinates
    say("noise pure z", len(layers))
    plan, out = _noise_plan_and_out(layers)
    dp.noise(plan, out, 1.0, 1.0, 0, 0)
    z_gpu = flat([o.cpu().numpy() for o in out])
    z = oracle.gauss(0, 0, 0, z_gpu.size)
    assert np.all(np.abs(z_gpu - z) <= 8 * 2.0 ** -24 * (1 + np.abs(z)))
    d = z.size
    assert abs(z_gpu.mean()) < 5 / math.sqrt(d)
    assert abs(z_gpu.var() - 1) < 5 * math.sqrt(2 / d)
    assert abs(np.linalg.norm(z_gpu) - math.sqrt(d)) < 5 / math.sqrt(2)


@pytest.mark.parametrize("descent", [False, True])
def test_noise_many_layers_several_launches(descent):
    """700 layers of 1-60 x 1-9 elements (ragged flat offsets): more layers than one noise launch
    takes (320, or 160 with the descent step), so the stream crosses launch boundaries; every
    coordinate against the oracle's, and the descent step on every parameter."""
    rng = np.random.default_rng(700 + descent)
    layers = [(int(rng.integers(1, 61)), int(rng.integers(1, 10))) for _ in range(700)]
    say("noise many layers", len(layers), "descent", descent)
    base = [rng.standard_normal(a * b).astype(np.float32) for a, b in layers]
    plan, out = _noise_plan_and_out(layers, base)
    sigma, C, seed, step, lr, L = 0.9, 1.7, 77, 5, 0.25, 4.0
    theta0 = [rng.standard_normal(a * b).astype(np.float32) for a, b in layers]
    theta = [torch.from_numpy(t).to(DEV) for t in theta0] if descent else None
    dp.noise(plan, out, C, sigma, seed, step, params=theta, lr=lr, normalizer=L)
    got = flat([o.cpu().numpy() for o in out])
    z = oracle.gauss(seed, step, 0, plan.n_params)
    z_gpu = (got - flat(base)) / (sigma * C)
    assert np.all(np.abs(z_gpu - z) <= 8 * 2.0 ** -24 * (1 + np.abs(z)) + 4e-7 * np.abs(flat(base)) / (sigma * C))
    if descent:
        # the oracle's update of its own noised sum; the GPU's within 1e-5 of the update's norm
        # plus the fp32 spacing of the parameters
        noised = flat(base) + sigma * C * z
        want = oracle.descent(flat(theta0), noised, lr, L)
        th = flat([t.cpu().numpy() for t in theta])
        spacing = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
        assert np.linalg.norm(th - want) <= 1e-5 * np.linalg.norm(want - flat(theta0)) + np.linalg.norm(spacing)


def test_noise_flat_index_past_2_32():
    """A 65,536 x 65,536 layer (2^32 parameters, cut into four launch pieces of 2^30) followed by a
    5 x 7 layer whose flat offsets start at 2^32: the Philox counter's upper word and the launch
    split by span.  Every coordinate of the small layer, and runs of coordinates at the start, the
    piece boundaries and the end of the large one, against the oracle's stream."""
    free = torch.cuda.mem_get_info()[0]
    if free < (20 << 30):
        pytest.skip("needs 20 GB of free device memory")
    layers = [(65536, 65536), (5, 7)]
    say("noise past 2^32")
    plan = dp.Plan(layers, dp.DTYPE_F32, 1, 1)
    big = torch.zeros(1 << 32, dtype=torch.float32, device=DEV)
    small = torch.zeros(35, dtype=torch.float32, device=DEV)
    sigma, C, seed, step = 1.5, 0.5, 0xABCDEF0123456789, 2**40 + 3
    dp.noise(plan, [big, small], C, sigma, seed, step)
    torch.cuda.synchronize()
    sc = sigma * C
    z = oracle.gauss(seed, step, 1 << 32, 35)
    got = small.cpu().numpy().astype(np.float64) / sc
    assert np.all(np.abs(got - z) <= 8 * 2.0 ** -24 * (1 + np.abs(z)))
    for start in (0, (1 << 30) - 37, (1 << 31) - 5, 3 * (1 << 30) - 64, (1 << 32) - 41):
        n = 101 if start + 101 <= (1 << 32) else (1 << 32) - start
        got = big[start:start + n].cpu().numpy().astype(np.float64) / sc
        want = oracle.gauss(seed, step, start, n)
        assert np.all(np.abs(got - want) <= 8 * 2.0 ** -24 * (1 + np.abs(want))), start
    del big


def test_noise_sigma_zero_and_step_change():
    layers = [(16, 16)]
    plan, out = _noise_plan_and_out(layers, [np.arange(256, dtype=np.float32)])
    dp.noise(plan, out, 1.0, 0.0, 1, 1)
    assert np.array_equal(out[0].cpu().numpy(), np.arange(256, dtype=np.float32))
    plan, o1 = _noise_plan_and_out([(512, 512)])
    plan, o2 = _noise_plan_and_out([(512, 512)])
    dp.noise(plan, o1, 1.0, 1.0, 9, 4)
    dp.noise(plan, o2, 1.0, 1.0, 9, 5)
    a, b = o1[0].cpu().numpy(), o2[0].cpu().numpy()
    assert abs(np.corrcoef(a, b)[0, 1]) < 5 / math.sqrt(a.size)


# ---------------------------------------------------------------- whole step, reduced workloads

def _oracle(w, As, Gs, C=None, sigma=None, seed=0, step=0, noise=True):
    return oracle.step(As, Gs, w.C if C is None else C, w.sigma if sigma is None else sigma,
                       seed, step, noise=noise)


def _check_step(w, r, ref, label):
    tol = TOL[w.dtype]
    en = max_rel(r["n"], ref["n"])
    ec = max_rel(r["c"], ref["c"])
    eS = rel_err(flat(r["out"]), flat(ref["S_noised"]))
    say(f"{label}: norm {en:.2e} clip {ec:.2e} noised-sum {eS:.2e}")
    assert r["status"] == dp.OK
    assert en <= tol and ec <= tol and eS <= tol


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("path,sum_policy", [(dp.PATH_AUTO, dp.SUM_AUTO), (dp.PATH_AUTO, dp.SUM_GEMM),
                                             (dp.PATH_GRAM, dp.SUM_AUTO), (dp.PATH_DIRECT, dp.SUM_STORED)])
def test_reduced_workload_step(idx, path, sum_policy):
    w = datagen.reduced(idx).with_(logical_B=datagen.reduced(idx).B)
    say("reduced workload", idx, w.name, "path", path, "sum", sum_policy)
    As, Gs = host_inputs(w)
    ref = _oracle(w, As, Gs)
    r = gpu_step(w, As, Gs, DEV, path=path, sum_policy=sum_policy)
    _check_step(w, r, ref, f"w{idx} p{path} s{sum_policy}")
    # pre-noise clipped sum (the noise would hide clipped-sum errors)
    r0 = gpu_step(w, As, Gs, DEV, path=path, sum_policy=sum_policy, flags=dp.NO_NOISE)
    e0 = rel_err(flat(r0["out"]), flat(ref["S"]))
    say(f"  pre-noise sum {e0:.2e}")
    assert e0 <= TOL[w.dtype]


def test_virtual_batching_reduced():
    """Three physical batches accumulated with one noise draw equal the oracle's logical step."""
    w = datagen.reduced(5)
    say("virtual batching", w.name, w.B, w.logical_B)
    plan = dp.Plan(w.layers, w.dtype, w.B, w.T)
    ws = plan.workspace(DEV)
    out = [torch.empty(a * b, dtype=torch.float32, device=DEV) for a, b in w.layers]
    batches, ns, cs = [], [], []
    for p in range(w.n_phys):
        As, Gs = host_inputs(w, first=p * w.B, n=w.B)
        batches.append((As, Gs))
        dA = [to_device(a, DEV) for a in As]
        dG = [to_device(g, DEV) for g in Gs]
        nrm = torch.empty(w.B, dtype=torch.float32, device=DEV)
        cf = torch.empty(w.B, dtype=torch.float32, device=DEV)
        flags = dp.NO_NOISE | (dp.ACCUMULATE if p else 0)
        dp.step(plan, dA, dG, out, ws, w.C, w.sigma, 0, 0, flags=flags, norms_out=nrm, clip_out=cf)
        ns.append(nrm.cpu().numpy())
        cs.append(cf.cpu().numpy())
    pre = flat([o.cpu().numpy() for o in out])
    dp.noise(plan, out, w.C, w.sigma, 0, 0, ws=ws)
    assert dp.status(plan, ws) == dp.OK
    ref = oracle.step(None, None, w.C, w.sigma, 0, 0, batches=batches)
    assert max_rel(np.concatenate(ns), ref["n"]) <= TOL[w.dtype]
    assert max_rel(np.concatenate(cs), ref["c"]) <= TOL[w.dtype]
    assert rel_err(pre, flat(ref["S"])) <= TOL[w.dtype]
    assert rel_err(flat([o.cpu().numpy() for o in out]), flat(ref["S_noised"])) <= TOL[w.dtype]


# ---------------------------------------------------------------- exactness and invariance

@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("T,shapes", [(8, [(16, 16), (16, 16)]), (5, [(12, 7), (7, 12)]),
                                      (8, [(3, 80), (80, 3)]), (1, [(1, 1)])])
def test_integer_inputs_exact(dtype, T, shapes):
    """Entries in {-3..3} with 81 T^2 d_in d_out L < 2^24: every partial sum is an exact integer,
    so the GPU's per-layer squared norms equal the oracle's exactly on both paths."""
    say("integer exact", dtype, T, shapes)
    rng = np.random.default_rng(7)
    B = 4
    As = [rng.integers(-3, 4, size=(B, T, a)).astype(np.float32) for a, _ in shapes]
    Gs = [rng.integers(-3, 4, size=(B, T, b)).astype(np.float32) for _, b in shapes]
    if dtype == BF16:
        As = [(a.view(np.uint32) >> 16).astype(np.uint16) for a in As]
        Gs = [(g.view(np.uint32) >> 16).astype(np.uint16) for g in Gs]
    want = np.stack([oracle.layer_norm2(a, g) for a, g in zip(As, Gs)])
    res = {}
    for path in (dp.PATH_GRAM, dp.PATH_DIRECT):
        plan = dp.Plan(shapes, dtype, B, T, path)
        ws = plan.workspace(DEV)
        dA = [to_device(a, DEV) for a in As]
        dG = [to_device(g, DEV) for g in Gs]
        dp.norms(plan, B, 0, len(shapes), dA, dG, ws)
        out = torch.empty(len(shapes) * B, dtype=torch.float32, device=DEV)
        dp.layer_norm2(plan, B, 0, len(shapes), ws, out)
        res[path] = out.cpu().numpy().reshape(len(shapes), B)
        assert np.array_equal(res[path].astype(np.float64), want), (path, res[path], want)
    assert np.array_equal(res[dp.PATH_GRAM], res[dp.PATH_DIRECT])


@pytest.mark.parametrize("idx", [2, 3])
def test_batch_invariance_and_repeat(idx):
    """Prop. 2 of 'Sensitivity Inflation ...' (record isolation): record i's norm and clip factor
    are bitwise identical alone, at another position, with a record added, under another plan
    capacity; two identical runs give bitwise identical outputs."""
    w = datagen.reduced(idx)
    say("batch invariance", w.name)
    As, Gs = host_inputs(w)
    B = w.B
    base = gpu_step(w, As, Gs, DEV)
    again = gpu_step(w, As, Gs, DEV, plan=base["plan"], ws=base["ws"])
    assert np.array_equal(base["n"], again["n"]) and np.array_equal(base["c"], again["c"])
    for o1, o2 in zip(base["out"], again["out"]):
        assert np.array_equal(o1, o2)
    big = dp.Plan(w.layers, w.dtype, B + 7, w.T)
    for i in range(B):
        alone = gpu_step(w, [a[i:i + 1] for a in As], [g[i:i + 1] for g in Gs], DEV, plan=big)
        assert alone["n"][0] == base["n"][i] and alone["c"][0] == base["c"][i]
    perm = np.arange(B)[::-1].copy()
    rev = gpu_step(w, [a[perm] for a in As], [g[perm] for g in Gs], DEV)
    assert np.array_equal(rev["n"], base["n"][perm]) and np.array_equal(rev["c"], base["c"][perm])
    extra = host_inputs(w, first=B, n=1)
    plus = gpu_step(w, [np.concatenate([a, e]) for a, e in zip(As, extra[0])],
                    [np.concatenate([g, e]) for g, e in zip(Gs, extra[1])], DEV, plan=big)
    assert np.array_equal(plus["n"][:B], base["n"]) and np.array_equal(plus["c"][:B], base["c"])


# ---------------------------------------------------------------- degenerate and error cases

@pytest.mark.parametrize("bad", [float("nan"), float("inf"), 1e30])
def test_nonfinite_norm_skips_sum_and_noise(bad):
    """A NaN/Inf input, or one whose norm overflows fp32, sets NONFINITE and leaves out untouched."""
    w = datagen.reduced(2)
    say("nonfinite", bad)
    As, Gs = host_inputs(w)
    As[1] = As[1].copy()
    Gs[1] = Gs[1].copy()
    As[1][2, 3, :] = bad
    Gs[1][2, 3, :] = bad
    plan = dp.Plan(w.layers, w.dtype, w.B, w.T)
    out = [torch.full((a * b,), 123.0, dtype=torch.float32, device=DEV) for a, b in w.layers]
    r = gpu_step(w, As, Gs, DEV, plan=plan, out=out)
    assert r["status"] == dp.ERR_NONFINITE
    for o in r["out"]:
        assert np.all(o == 123.0)
    # a following clean step on the same workspace clears the status
    As2, Gs2 = host_inputs(w)
    r2 = gpu_step(w, As2, Gs2, DEV, plan=plan, ws=r["ws"])
    assert r2["status"] == dp.OK


def test_empty_batch_releases_noise_only():
    """n_records = 0 (an empty Poisson sample): the clipped sum is 0 and the release is sigma*C*Z."""
    w = datagen.reduced(2)
    say("empty batch")
    plan = dp.Plan(w.layers, w.dtype, 4, w.T)
    ws = plan.workspace(DEV)
    out = [torch.full((a * b,), 5.0, dtype=torch.float32, device=DEV) for a, b in w.layers]
    dp.step(plan, None, None, out, ws, w.C, w.sigma, 3, 2, n_records=0)
    assert dp.status(plan, ws) == dp.OK
    got = flat([o.cpu().numpy() for o in out])
    z = oracle.gauss(3, 2, 0, got.size)
    assert np.all(np.abs(got - w.sigma * w.C * z) <= 8 * 2.0 ** -24 * (1 + np.abs(z)) * w.sigma * w.C)
    # with ACCUMULATE and NO_NOISE an empty batch leaves out unchanged
    dp.step(plan, None, None, out, ws, w.C, w.sigma, 3, 2, n_records=0,
            flags=dp.ACCUMULATE | dp.NO_NOISE)
    assert np.array_equal(flat([o.cpu().numpy() for o in out]), got)


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("path", [dp.PATH_AUTO, dp.PATH_GRAM, dp.PATH_DIRECT])
def test_ragged_shapes_and_misaligned_pointers(dtype, path):
    """Dimensions that are not multiples of the vector width or tile, T not a multiple of the
    MFMA k-step, and inputs starting one element past a 16-byte boundary."""
    say("ragged", dtype, path)
    shapes = [(37, 5), (5, 37), (130, 3), (19, 17), (200, 24), (1, 9)]
    T, B = 45, 3
    w = datagen.Workload(name="ragged", layers=tuple(shapes), layer_names=tuple("l%d" % i for i in range(6)),
                         dtype=dtype, B=B, logical_B=B, T=T, C=0.8, sigma=0.5, data_seed=99)
    As, Gs = host_inputs(w)
    ref = oracle.step(As, Gs, w.C, w.sigma, 1, 1)
    plan = dp.Plan(shapes, dtype, B, T, path)
    ws = plan.workspace(DEV)

    def shifted(x):
        t = to_device(x.reshape(-1), DEV)
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
        buf[1:].copy_(t)
        return buf[1:]
    dA = [shifted(a) for a in As]
    dG = [shifted(g) for g in Gs]
    out = [torch.empty(a * b, dtype=torch.float32, device=DEV) for a, b in shapes]
    nrm = torch.empty(B, dtype=torch.float32, device=DEV)
    dp.step(plan, dA, dG, out, ws, w.C, w.sigma, 1, 1, norms_out=nrm)
    assert dp.status(plan, ws) == dp.OK
    tol = TOL[dtype]
    assert max_rel(nrm.cpu().numpy(), ref["n"]) <= tol
    assert rel_err(flat([o.cpu().numpy() for o in out]), flat(ref["S_noised"])) <= tol


def test_clipped_sum_with_caller_factors():
    """dpsgd_clipped_sum with factors supplied by the caller, against the oracle's sum with the same
    factors, for both sum strategies."""
    w = datagen.reduced(3)
    say("caller factors", w.name)
    As, Gs = host_inputs(w)
    c = np.linspace(0.1, 1.0, w.B).astype(np.float32)
    want = flat([oracle.layer_clipped_sum(a, g, c.astype(np.float64)) for a, g in zip(As, Gs)])
    for sp in (dp.SUM_GEMM, dp.SUM_STORED):
        plan = dp.Plan(w.layers, w.dtype, w.B, w.T, dp.PATH_DIRECT, sp)
        ws = plan.workspace(DEV)
        dA = [to_device(a, DEV) for a in As]
        dG = [to_device(g, DEV) for g in Gs]
        out = [torch.empty(a * b, dtype=torch.float32, device=DEV) for a, b in w.layers]
        dp.ws_init(plan, ws)
        dp.norms(plan, w.B, 0, w.n_layers, dA, dG, ws)
        dc = torch.from_numpy(c).to(DEV)
        dp.clipped_sum(plan, w.B, 0, w.n_layers, dA, dG, dc, out, ws)
        torch.cuda.synchronize()
        assert rel_err(flat([o.cpu().numpy() for o in out]), want) <= TOL[w.dtype]


# ---------------------------------------------------------------- full-size workloads 1 and 2

@pytest.mark.parametrize("idx", [1, 2])
def test_full_workload_exact_oracle(idx):
    """Workloads 1 and 2 at full size, compared element by element with the full oracle."""
    w = datagen.workload(idx)
    say("full workload", idx, w.name)
    As, Gs = host_inputs(w)
    ref = _oracle(w, As, Gs)
    r = gpu_step(w, As, Gs, DEV)
    _check_step(w, r, ref, f"full w{idx}")
    # the pre-noise clipped sum (noise of norm sigma C sqrt(P) would hide its errors: about 543
    # against at most B C = 16 on workload 2), for the default plan and for the GEMM sum
    # A^T diag(c) G that re-reads the inputs instead of keeping per-record gradient blocks
    for sp in (dp.SUM_AUTO, dp.SUM_GEMM):
        r0 = gpu_step(w, As, Gs, DEV, flags=dp.NO_NOISE, sum_policy=sp)
        e0 = rel_err(flat(r0["out"]), flat(ref["S"]))
        say(f"  pre-noise sum (sum policy {sp}): {e0:.2e}")
        assert r0["status"] == dp.OK and e0 <= TOL[w.dtype]
        assert max_rel(r0["n"], ref["n"]) <= TOL[w.dtype] and max_rel(r0["c"], ref["c"]) <= TOL[w.dtype]
    if idx == 1:
        # workload 1 spans both clip branches: records 0-3 unclipped, 4-7 clipped
        assert np.all(ref["c"][:4] == 1.0) and np.all(ref["c"][4:] < 1.0)
        assert np.array_equal(r["c"][:4], np.ones(4, np.float32))
