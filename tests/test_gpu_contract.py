"""The DP contract on the library's own outputs, and the Gram path on records whose token
contributions cancel.

- Clipped norm: c_i n_i <= C (1 + 4 * 2^-24) on the fp32 n and c the library returns, and c_i = 1
  exactly when n_i <= C ("Privacy-Preserving Machine Learning", DP-SGD phase 3 and the remark
  after its clip_vector_l2 example that rounding can leave a clipped norm a hair above the bound).
- Sensitivity of the pre-noise clipped sum F(D) = sum_i c_i P_i (sigma = 0): adding or removing one
  record moves it by at most C, replacing one record by at most 2C ("Sensitivity Inflation from
  Cross-Record Precision Routing in Private Quantized Fine-Tuning", Sec. 2 Eq. 3 and Sec. 4.1
  Prop. 2; Sec. 5 "Measurement" takes the change in FP64 from the FP32 contributions with a 1e-4
  margin, as here).
- Gram path, near-cancelling tokens: tokens t and t + 64 share an activation row while their output
  gradients are (nearly) opposite, so the record's gradient sum_t a_t g_t^T is (nearly) zero while
  the Gram terms (a_t . a_s)(g_t . g_s) are not; their rounded fp32 sum may fall below zero.  The
  library must return status OK, a finite n >= 0 and c in (0, 1], with n^2 within the a-priori
  bound of the oracle's value (see gram_error_bound).
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import differentially_private_amd as dp  # noqa: E402
import oracle  # noqa: E402
from _helpers import TOL, flat, max_rel, rel_err, to_device  # noqa: E402
from datagen import BF16, F32  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
U = 2.0 ** -24      # fp32 unit roundoff


def say(*a):
    print(*a, flush=True)


def bf16_bits(x):
    """float32 values -> bf16 bit patterns, round to nearest even (input preparation only)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def as_f64(x):
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def run(layers, dtype, As, Gs, C, path=dp.PATH_AUTO, sum_policy=dp.SUM_AUTO, n=None):
    """dpsgd_step with sigma = 0 on the first n records; returns n, c, out (float64 flat), status."""
    n = As[0].shape[0] if n is None else n
    plan = dp.Plan(layers, dtype, max(n, 1), As[0].shape[1], path, sum_policy)
    ws = plan.workspace(DEV)
    dA = [to_device(np.ascontiguousarray(a[:n]), DEV) for a in As]
    dG = [to_device(np.ascontiguousarray(g[:n]), DEV) for g in Gs]
    out = [torch.full((a * b,), float("nan"), dtype=torch.float32, device=DEV) for a, b in layers]
    nrm = torch.full((max(n, 1),), -1.0, dtype=torch.float32, device=DEV)
    cf = torch.full((max(n, 1),), -1.0, dtype=torch.float32, device=DEV)
    dp.step(plan, dA, dG, out, ws, C, 0.0, 0, 0, n_records=n, norms_out=nrm, clip_out=cf)
    st = dp.status(plan, ws)
    return {"n": nrm.cpu().numpy()[:n], "c": cf.cpu().numpy()[:n], "status": st,
            "out": flat([o.cpu().numpy() for o in out]), "plan": plan, "ws": ws}


# ------------------------------------------------------------------------------------------
# Records of three kinds for the contract tests: ordinary ones (norm around the bound), ones far
# above it, and an all-zero record; shapes that take the direct path (LoRA-like), the Gram path and
# the dense bf16 GEMM sum.

CASES = {
    "direct_fp32_lora": ([(128, 8), (8, 128)], F32, 64, dp.PATH_AUTO, dp.SUM_AUTO),
    "direct_bf16_gemm": ([(256, 16), (16, 256)], BF16, 96, dp.PATH_AUTO, dp.SUM_GEMM),
    "gram_fp32": ([(256, 96)], F32, 40, dp.PATH_AUTO, dp.SUM_AUTO),
    "gram_bf16_dense": ([(256, 96), (96, 320)], BF16, 64, dp.PATH_AUTO, dp.SUM_AUTO),
}


def contract_inputs(layers, dtype, T, B, seed):
    rng = np.random.default_rng(seed)
    scale = np.exp(rng.uniform(np.log(0.02), np.log(50.0), size=B))
    scale[1] = 1e3          # far above the bound
    As, Gs = [], []
    for d_in, d_out in layers:
        a = rng.standard_normal((B, T, d_in)).astype(np.float32)
        g = (rng.standard_normal((B, T, d_out)) * scale[:, None, None]
             / math.sqrt(T * d_in * d_out * len(layers))).astype(np.float32)
        a[2] = 0.0          # a zero record: norm 0, factor 1
        if dtype == BF16:
            a, g = bf16_bits(a), bf16_bits(g)
        As.append(a)
        Gs.append(g)
    return As, Gs


@pytest.mark.parametrize("case", sorted(CASES))
def test_clipped_norm_bound_and_factors(case):
    layers, dtype, T, path, sp = CASES[case]
    B, C = 9, 1.0
    As, Gs = contract_inputs(layers, dtype, T, B, 11)
    say("clip bound", case)
    r = run(layers, dtype, As, Gs, C, path, sp)
    assert r["status"] == dp.OK
    n, c = r["n"].astype(np.float64), r["c"].astype(np.float64)
    assert np.all(np.isfinite(n)) and np.all(n >= 0) and np.all(c > 0) and np.all(c <= 1)
    assert np.all(c * n <= C * (1 + 4 * U)), np.max(c * n / C - 1)
    assert np.all(c[n <= C] == 1.0)
    assert n[2] == 0.0 and c[2] == 1.0
    assert np.any(n > C) and np.any(n <= C)         # both branches exercised
    ref = oracle.step(As, Gs, C, 0.0, 0, 0, noise=False)
    assert max_rel(n, ref["n"]) <= TOL[dtype] and max_rel(c, ref["c"]) <= TOL[dtype]
    assert rel_err(r["out"], flat(ref["S"])) <= TOL[dtype]


@pytest.mark.parametrize("case", sorted(CASES))
def test_sensitivity_add_remove_and_replace(case):
    """F(D u {x}) - F(D) and F(D with x replaced) - F(D), in FP64 from the library's fp32 sums."""
    layers, dtype, T, path, sp = CASES[case]
    B, C = 9, 0.5
    As, Gs = contract_inputs(layers, dtype, T, B + 1, 12)
    say("sensitivity", case)
    full = run(layers, dtype, As, Gs, C, path, sp)                 # D u {x}, x = the last record
    base = run(layers, dtype, As, Gs, C, path, sp, n=B)            # D
    assert full["status"] == dp.OK and base["status"] == dp.OK
    delta = np.linalg.norm(full["out"] - base["out"])
    say(f"  add/remove: {delta / C:.6f} C")
    assert delta <= C * (1 + 1e-4)
    # x placed first instead of last: the same bound
    perm = np.r_[B, np.arange(B)]
    first = run(layers, dtype, [a[perm] for a in As], [g[perm] for g in Gs], C, path, sp)
    assert np.linalg.norm(first["out"] - base["out"]) <= C * (1 + 1e-4)
    # removing the record far above the bound (record 1): exactly its clipped contribution, norm C
    keep = np.r_[0, np.arange(2, B)]
    rem = run(layers, dtype, [a[keep] for a in As], [g[keep] for g in Gs], C, path, sp)
    d1 = np.linalg.norm(base["out"] - rem["out"])
    say(f"  remove the large record: {d1 / C:.6f} C")
    assert abs(d1 - C) <= 1e-4 * C
    # replace record 4 of D by x: at most 2C
    rep = np.r_[np.arange(4), B, np.arange(5, B)]
    swapped = run(layers, dtype, [a[rep] for a in As], [g[rep] for g in Gs], C, path, sp)
    d2 = np.linalg.norm(swapped["out"] - base["out"])
    say(f"  replace: {d2 / C:.6f} C")
    assert d2 <= 2 * C * (1 + 1e-4)


# ------------------------------------------------------------------------------------------
# Gram path on near-cancelling tokens

def gram_error_bound(A, G):
    """A-priori bound on the rounding error of the Gram-path squared norm of one record (A [T,
    d_in], G [T, d_out] as float64): every token Gram entry is an fp32 sum of d products, every
    Hadamard term one more fp32 product, and the T^2 terms an fp32 sum, so the computed value is
    within gamma_{max(d_in, d_out) + T^2 + 1} * M of the exact one (Higham, "Accuracy and Stability of
    Numerical Algorithms", Sec. 3.1: the error of any summation order), with
    M = sum_{t,s} |a_t|.|a_s| |g_t|.|g_s| (entrywise absolute values).  Unlike the squared norm
    itself, M does not shrink when the token contributions cancel."""
    T, d_in = A.shape
    d_out = G.shape[1]
    Ma = np.abs(A) @ np.abs(A).T
    Mg = np.abs(G) @ np.abs(G).T
    n = max(d_in, d_out) + T * T + 1
    return n * U / (1 - n * U) * float(np.sum(Ma * Mg))


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_gram_near_cancelling_tokens(dtype):
    """Records of 128 tokens (two 64-token blocks) in one 256 -> 96 layer (Gram: 128^2 < 256 * 96;
    fp32 runs the register Gram kernel, bf16 the per-record copy kernel): token t + 64 repeats the
    activation row of token t and carries minus its gradient row, exactly (records 0-7), with a few
    gradient entries moved by one ulp (records 8-15), or scaled by 1 + 2^-12 (records 16-23; fp32
    only: bf16 keeps the exact negation there); records 24-27 are ordinary."""
    T, d_in, d_out, B = 128, 256, 96, 28
    rng = np.random.default_rng(2024 + dtype)
    a = rng.standard_normal((B, 64, d_in)).astype(np.float32)
    g = rng.standard_normal((B, 64, d_out)).astype(np.float32)
    if dtype == BF16:
        a = as_f64(bf16_bits(a)).astype(np.float32)
        g = as_f64(bf16_bits(g)).astype(np.float32)
    g2 = -g.copy()
    for i in range(8, 16):      # one-ulp moves of a few entries
        idx = rng.integers(0, 64, 5), rng.integers(0, d_out, 5)
        if dtype == BF16:
            bits = bf16_bits(g2[i][idx]).astype(np.int32) + 1
            g2[i][idx] = as_f64(bits.astype(np.uint16)).astype(np.float32)
        else:
            g2[i][idx] = np.nextafter(g2[i][idx], np.float32(np.inf))
    if dtype == F32:
        g2[16:24] *= np.float32(1 + 2.0 ** -12)
    A = np.concatenate([a, a], axis=1)
    G = np.concatenate([g, g2], axis=1)
    A[24:] = rng.standard_normal((4, T, d_in))
    G[24:] = rng.standard_normal((4, T, d_out))
    if dtype == BF16:
        A, G = bf16_bits(A), bf16_bits(G)
    layers = [(d_in, d_out)]
    say("gram near-cancel", dtype)
    plan = dp.Plan(layers, dtype, B, T)
    assert plan.layer_info(0)[0] == dp.PATH_GRAM
    r = run(layers, dtype, [A], [G], 1.0)
    assert r["status"] == dp.OK
    n, c = r["n"].astype(np.float64), r["c"].astype(np.float64)
    assert np.all(np.isfinite(n)) and np.all(n >= 0), n
    assert np.all(c > 0) and np.all(c <= 1) and np.all(np.isfinite(r["out"]))
    ln = torch.empty(B, dtype=torch.float32, device=DEV)
    dp.layer_norm2(r["plan"], B, 0, 1, r["ws"], ln)
    ln = ln.cpu().numpy().astype(np.float64)
    assert np.all(ln >= 0)
    want = oracle.layer_norm2(A, G)
    Af, Gf = as_f64(A), as_f64(G)
    worst = 0.0
    for i in range(B):
        bound = gram_error_bound(Af[i], Gf[i])
        worst = max(worst, abs(ln[i] - want[i]) / bound)
        assert abs(ln[i] - want[i]) <= bound + 4 * U * ln[i], (i, ln[i], want[i], bound)
        assert abs(n[i] ** 2 - want[i]) <= bound * (1 + 1e-6) + 4 * U * n[i] ** 2, (i, n[i], want[i])
    # the factors follow the returned norms (C = 1); a cancelling record's own contribution is
    # (nearly) zero, so its factor does not move the sum
    assert np.all(c[n <= 1.0] == 1.0) and np.all(c * n <= 1.0 + 4 * U)
    say(f"  worst error / bound {worst:.2e}; norms of the cancelling records: {n[:24].max():.3e} max")
    # the ordinary records keep the usual relative accuracy
    assert max_rel(n[24:], np.sqrt(want[24:])) <= TOL[dtype]
    # pre-noise sum against the oracle (its factors from its own norms).  Its entries are sums of
    # cancelling token products too, so their error is bounded entrywise by the sizes of the
    # summed products, sum_i c_i sum_t |a_t| |g_t|^T (an fp32 sum of B T terms, plus one rounding
    # per record of the factor applied to a running sum), and by the factors' own tolerance
    # times |P_i|; a relative Frobenius bound holds only where nothing cancels
    ref = oracle.step([A], [G], 1.0, 0.0, 0, 0, noise=False)
    got = r["out"].reshape(d_in, d_out)
    E = np.zeros((d_in, d_out))
    Pabs = np.zeros((d_in, d_out))
    for i in range(B):
        E += ref["c"][i] * (np.abs(Af[i]).T @ np.abs(Gf[i]))
        # a factor may differ from the oracle's as far as its norm may (checked above)
        Pabs += max(abs(c[i] - ref["c"][i]), TOL[dtype] * ref["c"][i]) * np.abs(Af[i].T @ Gf[i])
    n_terms = B * T + 2 * B + 2
    bound = n_terms * U / (1 - n_terms * U) * E + Pabs
    err = np.abs(got - ref["S"][0])
    say(f"  clipped sum: worst error / entrywise bound {np.max(err / bound):.2e}, "
        f"relative Frobenius error {rel_err(got, ref['S'][0]):.2e}")
    assert np.all(err <= bound)
