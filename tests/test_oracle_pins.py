"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test names the passage or the fact it pins.  A plausible mistake in the oracle (a dropped
term, a wrong sign or index, a transposed operand, a wrong clip branch, a wrong Philox round or
counter layout, a wrong Box-Muller pairing) fails at least one of them.
"""
import json
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

rng = np.random.default_rng(1234)


def one_layer(vectors, dtype=np.float64):
    """Scalar/vector records as a linear layer with T = 1, d_in = 1, A = [[1]]: P_i = G_i."""
    g = np.asarray(vectors, dtype=dtype)
    B, d = g.shape
    A = np.ones((B, 1, 1), dtype=dtype)
    G = g.reshape(B, 1, d)
    return A, G


def run_step(A, G, C, sigma=0.0, seed=0, step=0):
    return oracle.step([A], [G], C, sigma, seed, step, noise=sigma != 0.0)


# ---------------------------------------------------------------- clipping: the page's example

def test_p1_clip_example(golden_dir):
    """'Privacy-Preserving Machine Learning', DP-SGD section: clip_vector_l2 on three vectors."""
    g = json.load(open(os.path.join(golden_dir, "p1_clip_example.json")))
    A, G = one_layer(g["gradients"])
    r = run_step(A, G, g["C"])
    np.testing.assert_allclose(r["n"], g["norms"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r["c"], g["factors"], rtol=0, atol=1e-15)
    clipped = np.array(g["gradients"]) * r["c"][:, None]
    np.testing.assert_allclose(clipped, g["clipped"], rtol=0, atol=1e-15)
    S = r["S"][0].reshape(-1)
    assert [round(x, 2) for x in S] == g["clipped_sum_2dp"]
    np.testing.assert_allclose(S, [1.6, 1.9], rtol=0, atol=1e-15)
    # the same records stored as fp32, the precision the GPU consumes
    A32, G32 = one_layer(g["gradients"], np.float32)
    r32 = run_step(A32, G32, g["C"])
    np.testing.assert_allclose(r32["S"][0].reshape(-1), [1.6, 1.9], rtol=1e-7)


def test_p1_rounding_remark(golden_dir):
    """Same section: [1, 3] clipped has norm <= C unrounded; its 4-decimal display exceeds 1."""
    g = json.load(open(os.path.join(golden_dir, "p1_clip_example.json")))["rounding_remark"]
    A, G = one_layer([g["gradient"]])
    r = run_step(A, G, 1.0)
    clipped = np.array(g["gradient"]) * r["c"][0]
    assert np.linalg.norm(clipped) <= 1.0 * (1 + 4 * 2.0 ** -53)
    np.testing.assert_allclose(np.round(clipped, 4), g["rounded_clipped"], atol=0)
    assert math.hypot(*g["rounded_clipped"]) > 1.0


def test_p1_alice_bao_row_clipping(golden_dir):
    """Same section: example-level clipping of scalar gradients gives 1.50 (Alice), 0.25 (Bao)."""
    g = json.load(open(os.path.join(golden_dir, "p1_clip_example.json")))["alice_bao"]
    for user, want in (("alice", g["alice_row_clipped_sum"]), ("bao", g["bao_row_clipped_sum"])):
        A, G = one_layer([[x] for x in g[user]])
        r = run_step(A, G, g["C"])
        assert abs(r["S"][0][0, 0] - want) <= 1e-15
        # scalar clipping to [-C, C] is the 1-D case of the L2 clip
        assert abs(r["S"][0][0, 0] - sum(max(-g["C"], min(x, g["C"])) for x in g[user])) <= 1e-15


def test_clip_branches_and_tie():
    """Clip factor: 1 for n <= C (including n = 0 and n = C), C/n above; the exhibit's form
    g / max(1, ||g||/C) agrees with g * min(1, C/||g||)."""
    assert oracle.clip_factor(0.0, 1.0) == 1.0
    assert oracle.clip_factor(1.0, 1.0) == 1.0            # n == C stays unclipped
    assert oracle.clip_factor(0.25, 1.0) == 1.0
    assert oracle.clip_factor(4.0, 1.0) == 0.5
    assert oracle.clip_factor(25.0, 2.0) == 2.0 / 5.0
    for n in [1e-3, 0.7, 1.0, 1.3, 5.0, 1e6]:
        C = 1.1
        assert abs(oracle.clip_factor(n * n, C) - 1.0 / max(1.0, n / C)) <= 1e-15


def test_zero_gradient_unchanged():
    """A zero per-record gradient is left unchanged (no division by zero) and adds nothing."""
    A, G = one_layer([[0.0, 0.0], [3.0, 4.0]])
    r = run_step(A, G, 1.0)
    assert r["n"][0] == 0.0 and r["c"][0] == 1.0
    np.testing.assert_allclose(r["S"][0].reshape(-1), [0.6, 0.8], atol=1e-15)


# ---------------------------------------------------------------- the constructed witness

def test_p5_witness_exact_values(golden_dir):
    """'Sensitivity Inflation ...', App. A: seven records whose gradient flips sign between the
    neighbours (both larger than C_f) and one record clipped to +C_f in both; with per-record
    clipping the replacement distance is 14 C_f and the ratio to 2 C_f is 7."""
    w = json.load(open(os.path.join(golden_dir, "p5_witness.json")))
    Cf = w["C_f"]
    assert Cf == float(np.float32(0.005))
    big = 1.0                                  # the replaced record: clipped to +C_f in both
    D = [[w["grad_D"]]] * w["n_unchanged"] + [[big]]
    Dp = [[w["grad_Dprime"]]] * w["n_unchanged"] + [[big]]
    FD = run_step(*one_layer(D), Cf)["S"][0][0, 0]
    FDp = run_step(*one_layer(Dp), Cf)["S"][0][0, 0]
    assert abs(FD - (-6 * Cf)) <= 8 * np.spacing(Cf)
    assert abs(FDp - 8 * Cf) <= 8 * np.spacing(Cf)
    delta = abs(FDp - FD)
    assert abs(delta - w["delta"]) <= 16 * np.spacing(w["delta"])
    assert abs(delta / (2 * Cf) - w["delta_over_2C"]) <= 1e-14


# ---------------------------------------------------------------- norms: closed forms, brute force

def test_rank_one_closed_form():
    """T = 1: ||a g^T||_F = ||a|| ||g|| for any vectors."""
    for d_in, d_out in [(1, 1), (7, 3), (64, 32), (5, 300)]:
        a = rng.standard_normal((1, 1, d_in))
        g = rng.standard_normal((1, 1, d_out))
        n2 = oracle.layer_norm2(a, g)[0]
        want = np.linalg.norm(a) * np.linalg.norm(g)
        assert abs(math.sqrt(n2) - want) <= 1e-14 * want


@pytest.mark.parametrize("T,d_in,d_out", [(1, 1, 1), (3, 2, 5), (8, 4, 7), (5, 16, 1)])
def test_integer_brute_force_and_gram_identity(T, d_in, d_out):
    """Integer entries in [-3, 3]: every partial sum is an exact integer, so the oracle's squared
    norm must equal both the brute-force sum_{j,k}(sum_t a_tj g_tk)^2 and the Gram identity
    sum_{t,s}(a_t . a_s)(g_t . g_s), computed here in Python integers."""
    B = 3
    Ai = rng.integers(-3, 4, size=(B, T, d_in))
    Gi = rng.integers(-3, 4, size=(B, T, d_out))
    for dt in (np.float64, np.float32):
        got = oracle.layer_norm2(Ai.astype(dt), Gi.astype(dt))
        for i in range(B):
            a = Ai[i].tolist()
            g = Gi[i].tolist()
            brute = sum(sum(a[t][j] * g[t][k] for t in range(T)) ** 2
                        for j in range(d_in) for k in range(d_out))
            gram = sum(sum(a[t][j] * a[s][j] for j in range(d_in)) *
                       sum(g[t][k] * g[s][k] for k in range(d_out))
                       for t in range(T) for s in range(T))
            assert brute == gram
            assert got[i] == float(brute)


def test_bf16_inputs_widen_exactly():
    """bf16 bit patterns are widened exactly: 0x3F80 = 1.0, 0xC040 = -3.0, 0x3E80 = 0.25."""
    A = np.array([[[0x3F80, 0xC040]]], dtype=np.uint16)        # a = (1, -3)
    G = np.array([[[0x3E80]]], dtype=np.uint16)                # g = (0.25)
    n2 = oracle.layer_norm2(A, G)[0]
    assert n2 == (1 * 0.25) ** 2 + (-3 * 0.25) ** 2


def test_gradient_convention_autograd():
    """P_i = A_i^T G_i is the gradient of a loss summed over the record's tokens through
    y = x W with W in R^{d_in x d_out} (G = dLoss/dy), as autograd (float64) computes it."""
    torch = pytest.importorskip("torch")
    T, d_in, d_out = 6, 5, 3
    A = rng.standard_normal((T, d_in))
    G = rng.standard_normal((T, d_out))
    W = torch.zeros(d_in, d_out, dtype=torch.float64, requires_grad=True)
    y = torch.from_numpy(A) @ W
    loss = (y * torch.from_numpy(G)).sum()
    loss.backward()
    P = oracle.record_grad(A, G)
    np.testing.assert_allclose(P, W.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_no_clip_reduces_to_gemm():
    """With C = 1e30 nothing is clipped, so S = A^T G over all B*T rows (one library GEMM)."""
    B, T, d_in, d_out = 4, 9, 13, 6
    A = rng.standard_normal((B, T, d_in)).astype(np.float32)
    G = rng.standard_normal((B, T, d_out)).astype(np.float32)
    r = run_step(A, G, 1e30)
    assert np.all(r["c"] == 1.0)
    want = A.reshape(-1, d_in).astype(np.float64).T @ G.reshape(-1, d_out).astype(np.float64)
    np.testing.assert_allclose(r["S"][0], want, rtol=1e-12, atol=1e-12)


def test_joint_norm_over_layers():
    """One norm per record over the concatenated gradient of all layers (not per layer)."""
    B, T = 3, 4
    shapes = [(5, 2), (2, 5), (3, 3)]
    As = [rng.standard_normal((B, T, a)) for a, _ in shapes]
    Gs = [rng.standard_normal((B, T, b)) for _, b in shapes]
    r = oracle.step(As, Gs, 1.0, 0.0, 0, 0, noise=False)
    for i in range(B):
        flat = np.concatenate([(As[l][i].T @ Gs[l][i]).reshape(-1) for l in range(3)])
        assert abs(r["n"][i] - np.linalg.norm(flat)) <= 1e-12 * np.linalg.norm(flat)
        clipped_norm = np.linalg.norm(flat * r["c"][i])
        assert clipped_norm <= 1.0 * (1 + 1e-12)


# ---------------------------------------------------------------- sensitivity

def _F(As, Gs, C):
    r = oracle.step(As, Gs, C, 0.0, 0, 0, noise=False)
    return np.concatenate([s.reshape(-1) for s in r["S"]]), r


def test_sensitivity_add_remove_and_replace():
    """Separable bound of the clipped sum: adding/removing one record moves it by the record's
    own clipped contribution (norm <= C); replacing one moves it by <= 2C."""
    C = 0.7
    B, T = 6, 5
    shapes = [(4, 3), (3, 4)]
    As = [rng.standard_normal((B + 1, T, a)) for a, _ in shapes]
    Gs = [rng.standard_normal((B + 1, T, b)) for _, b in shapes]
    F_all, r_all = _F(As, Gs, C)
    F_less, _ = _F([a[:B] for a in As], [g[:B] for g in Gs], C)
    h = F_all - F_less
    x_flat = np.concatenate([(As[l][B].T @ Gs[l][B]).reshape(-1) for l in range(2)])
    np.testing.assert_allclose(h, x_flat * r_all["c"][B], rtol=1e-10, atol=1e-12)
    assert np.linalg.norm(h) <= C * (1 + 1e-12)
    # replacement of record 0
    As2 = [a[:B].copy() for a in As]
    Gs2 = [g[:B].copy() for g in Gs]
    for l in range(2):
        As2[l][0] = As[l][B]
        Gs2[l][0] = -Gs[l][B]
    F_rep, _ = _F(As2, Gs2, C)
    assert np.linalg.norm(F_rep - F_less) <= 2 * C * (1 + 1e-12)


def test_sensitivity_bounds_attained_in_1d():
    """1-D: a record clipped to +C added to an empty batch moves the sum by exactly C; replacing
    +5 by -5 moves it by exactly 2C."""
    C = 1.0
    F1 = run_step(*one_layer([[5.0]]), C)["S"][0][0, 0]
    assert F1 == C
    Fm = run_step(*one_layer([[-5.0]]), C)["S"][0][0, 0]
    assert abs(F1 - Fm) == 2 * C


def test_clip_the_mean_bug_gives_2C():
    """'Privacy-Preserving Machine Learning': clipping the batch mean instead of each record
    allows a 2C change between neighbours; per-record clipping (the oracle) gives C."""
    C = 1.0
    D = [[5.0]]
    Dp = [[5.0], [-50.0]]
    per_record = abs(run_step(*one_layer(Dp), C)["S"][0][0, 0] - run_step(*one_layer(D), C)["S"][0][0, 0])
    assert per_record == C

    def clip_mean(v):
        m = np.mean(v)
        return m * min(1.0, C / abs(m))
    assert abs(clip_mean(Dp) - clip_mean(D)) == 2 * C


def test_clipped_norm_bound_fp_rounding():
    """||c_i P_i|| <= C (1 + 4 * 2^-53) in double for heavy and light records."""
    B, T, d_in, d_out = 8, 7, 9, 5
    A = rng.standard_cauchy((B, T, d_in))
    G = rng.standard_normal((B, T, d_out))
    for C in [1e-3, 0.5, 1.0, 3.0]:
        r = run_step(A, G, C)
        for i in range(B):
            P = A[i].T @ G[i]
            assert np.linalg.norm(P * r["c"][i]) <= C * (1 + 4 * 2.0 ** -53) * (1 + 1e-13)


def test_virtual_batching_equals_one_batch():
    """Records split into physical batches: n and c are unchanged bitwise (each record's factor
    depends only on its own data), the accumulated sum equals the one-batch sum, noise once."""
    B, T = 6, 4
    shapes = [(5, 2), (2, 5)]
    As = [rng.standard_normal((B, T, a)).astype(np.float32) for a, _ in shapes]
    Gs = [rng.standard_normal((B, T, b)).astype(np.float32) for _, b in shapes]
    one = oracle.step(As, Gs, 0.5, 1.3, 7, 3)
    batches = [([a[p:p + 2] for a in As], [g[p:p + 2] for g in Gs]) for p in range(0, B, 2)]
    virt = oracle.step(None, None, 0.5, 1.3, 7, 3, batches=batches)
    assert np.array_equal(one["n"], virt["n"]) and np.array_equal(one["c"], virt["c"])
    for l in range(2):
        np.testing.assert_allclose(virt["S"][l], one["S"][l], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(virt["S_noised"][l], one["S_noised"][l], rtol=1e-13, atol=1e-13)


def test_sigma_zero_is_exact_sum():
    B, T = 3, 4
    A = rng.standard_normal((B, T, 6)).astype(np.float32)
    G = rng.standard_normal((B, T, 3)).astype(np.float32)
    r = oracle.step([A], [G], 0.3, 0.0, 5, 9, noise=True)
    assert np.array_equal(r["S_noised"][0], r["S"][0])


# ---------------------------------------------------------------- Philox and the Gaussian stream

def _rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand"):
        pytest.skip("hipcc / rocRAND headers not available")
    d = tmp_path_factory.mktemp("rocrand")
    exe = str(d / "philox_ref")
    src = os.path.join(os.path.dirname(__file__), "rocrand_philox_ref.cpp")
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-O1", "-o", exe, src],
                          stderr=subprocess.DEVNULL)
    return exe


@pytest.fixture(scope="module")
def rocrand_exe(tmp_path_factory):
    return _rocrand_ref(tmp_path_factory)


@pytest.mark.parametrize("seed,step,first,n", [(0, 0, 0, 8), (0x123456789ABCDEF, 5, 2, 6),
                                               (2**64 - 1, 2**64 - 1, 2**62 - 4, 4),
                                               (42, 1, 2**32 - 2, 5)])
def test_philox_matches_rocrand(rocrand_exe, seed, step, first, n):
    """Philox4x32-10 (SC'11) with key = seed and counter = (block, step) reproduces rocRAND's
    engine word for word, including 64-bit carries of the block index."""
    out = subprocess.check_output([rocrand_exe, str(seed), str(step), str(first), str(n)], text=True)
    want = np.array([int(x) for x in out.split()], dtype=np.uint32)
    got = oracle.philox_words(seed, step, first, n)
    assert np.array_equal(got, want)


def test_gauss_statistics_and_page_rms(golden_dir):
    """Noise over d = 5e6 coordinates with sigma*C = 1: ||Z|| matches the page's RMS 2236.07
    (sqrt(d)) within 5 standard deviations of ||Z||, mean and variance within 5 sigma, KS
    against the standard normal, and the page's step-noise RMS eta*sigma*C*sqrt(d)/L."""
    g = json.load(open(os.path.join(golden_dir, "p1_noise_rms.json")))
    d = g["d_adapter"]
    z = oracle.gauss(0, 0, 0, d)
    assert abs(np.linalg.norm(z) - g["adapter_sum_rms_2dp"]) < 5 * (1 / math.sqrt(2)) + 0.005
    assert round(g["learning_rate"] * math.sqrt(d) * g["sigma_c"] / g["normalizer"], 2) == \
        g["adapter_step_rms_2dp"]
    assert abs(z.mean()) < 5 / math.sqrt(d)
    assert abs(z.var() - 1) < 5 * math.sqrt(2 / d)
    stats = pytest.importorskip("scipy.stats")
    ks = stats.kstest(z[:1_000_000], "norm")
    assert ks.pvalue > 1e-4
    assert np.abs(z).max() <= math.sqrt(48 * math.log(2)) + 1e-12


def test_gauss_pairs_use_one_radius():
    """Box-Muller pairing: lanes (0,1) and (2,3) of each block share one radius, so
    z0^2 + z1^2 = -2 ln u1 of word 0; different pairs use different words."""
    w = oracle.philox_words(3, 4, 0, 16).reshape(16, 4)
    z = oracle.gauss(3, 4, 0, 64).reshape(16, 4)
    for b in range(16):
        for p in range(2):
            u1 = ((int(w[b, 2 * p]) >> 8) + 1) / 2 ** 24
            assert abs(z[b, 2 * p] ** 2 + z[b, 2 * p + 1] ** 2 - (-2 * math.log(u1))) < 1e-12
            u2 = (int(w[b, 2 * p + 1]) >> 8) / 2 ** 24
            ang = math.atan2(z[b, 2 * p + 1], z[b, 2 * p]) % (2 * math.pi)
            assert abs(ang - 2 * math.pi * u2) < 1e-9 or abs(ang - 2 * math.pi * u2) > 2 * math.pi - 1e-9


def test_gauss_offsets_and_decorrelation():
    """Z is a function of (seed, step, element): any window reproduces the full stream; a new
    step or seed gives an uncorrelated stream."""
    d = 400_000
    z = oracle.gauss(11, 2, 0, d)
    np.testing.assert_array_equal(oracle.gauss(11, 2, 1001, 5003), z[1001:6004])
    for other in (oracle.gauss(11, 3, 0, d), oracle.gauss(12, 2, 0, d)):
        rho = np.corrcoef(z, other)[0, 1]
        assert abs(rho) < 5 / math.sqrt(d)


def test_noise_added_to_every_coordinate():
    """Noise reaches every coordinate of every layer, including those where S is exactly 0."""
    As = [np.zeros((2, 3, 4), np.float32), np.ones((2, 3, 2), np.float32)]
    Gs = [np.zeros((2, 3, 5), np.float32), np.ones((2, 3, 3), np.float32)]
    r = oracle.step(As, Gs, 1.0, 1.0, 0, 0)
    flat = np.concatenate([s.reshape(-1) for s in r["S_noised"]])
    pre = np.concatenate([s.reshape(-1) for s in r["S"]])
    assert np.all(flat != pre)
    np.testing.assert_allclose(flat - pre, oracle.gauss(0, 0, 0, flat.size), rtol=1e-14, atol=1e-15)


def test_descent_worked_example(golden_dir):
    """Phase 5 on the page's clip_vector_l2 example (no noise): theta1 worked by hand from the
    printed clipped sum [1.60, 1.90] with eta = 0.5, L = 2."""
    g = json.load(open(os.path.join(golden_dir, "p1_clip_example.json")))
    d = json.load(open(os.path.join(golden_dir, "p1_descent_example.json")))
    grads = np.array(g["gradients"], dtype=np.float64)
    A = [np.ones((len(grads), 1, 1))]
    G = [grads.reshape(len(grads), 1, 2)]
    theta0 = [np.array(d["theta0"], dtype=np.float64).reshape(1, 2)]
    r = oracle.step(A, G, g["C"], 0.0, 0, 0, descent_args=(theta0, d["learning_rate"], d["normalizer"]))
    assert np.allclose(r["theta"][0].reshape(-1), d["theta1"], rtol=0, atol=1e-15)
    with pytest.raises(ValueError):
        oracle.step(A, G, g["C"], 0.0, 0, 0, noise=False, descent_args=(theta0, 0.5, 2.0))


def test_descent_step_noise_rms_page(golden_dir):
    """A pure-noise step (empty batch) from theta0 = 0 over d = 5e6 coordinates with the page's
    sigma*C = 1, eta = 0.01, L = 128: the step's norm is the page's step-noise RMS 0.17, within
    5 standard deviations of eta*sigma*C*||Z||/L around eta*sigma*C*sqrt(d)/L."""
    g = json.load(open(os.path.join(golden_dir, "p1_noise_rms.json")))
    d = g["d_adapter"]
    di, do = 5000, d // 5000
    A = [np.zeros((0, 1, di))]
    G = [np.zeros((0, 1, do))]
    lr, L = g["learning_rate"], g["normalizer"]
    r = oracle.step(A, G, 1.0, g["sigma_c"], 0, 0, descent_args=([np.zeros((di, do))], lr, L))
    step_norm = np.linalg.norm(r["theta"][0])
    assert round(step_norm, 2) == g["adapter_step_rms_2dp"]
    assert abs(step_norm - lr * g["sigma_c"] * math.sqrt(d) / L) < 5 * lr / (L * math.sqrt(2))


def _users_as_records(users, d_out=1):
    """Users as records: each user's token rows (one token per scalar gradient here) concatenated
    and zero-padded to the longest user; zero rows add nothing to A^T G."""
    T = max(len(u) for u in users)
    A = np.zeros((len(users), T, 1))
    G = np.zeros((len(users), T, d_out))
    for i, u in enumerate(users):
        A[i, :len(u), 0] = 1.0
        G[i, :len(u), 0] = u
    return [A], [G]


def test_user_level_clipping_page(golden_dir):
    """The page's sum-then-user-clip example: Alice's tickets 0.5 and 5.0 and Bao's 0.25 as two
    users (each user's gradient is the sum over its records' token rows), C = 1: user-clipped
    1.00 and 0.25; with the public normaliser 2 the sums are 0.625 with Alice and 0.125 without,
    a change of 0.500 = C / 2 (example-level clipping gives Alice 1.50)."""
    g = json.load(open(os.path.join(golden_dir, "p1_clip_example.json")))["alice_bao"]
    u = g["user_level"]
    A, G = _users_as_records([g["alice"], g["bao"]])
    r = oracle.step(A, G, g["C"], 0.0, 0, 0)
    assert np.allclose(r["n"] * r["c"], [u["alice_user_clipped"], u["bao_user_clipped"]], atol=1e-15)
    with_alice = r["S"][0][0, 0] / u["normalizer"]
    A1, G1 = _users_as_records([g["bao"]])
    without_alice = oracle.step(A1, G1, g["C"], 0.0, 0, 0)["S"][0][0, 0] / u["normalizer"]
    assert round(with_alice, 3) == u["with_alice"]
    assert round(without_alice, 3) == u["without_alice"]
    assert round(with_alice - without_alice, 3) == u["change"]
    assert abs(with_alice - without_alice) <= g["C"] / u["normalizer"] + 1e-15
    # example-level clipping of the same tickets gives Alice 1.50
    Ar, Gr = _users_as_records([[v] for v in g["alice"]])
    assert round(oracle.step(Ar, Gr, g["C"], 0.0, 0, 0)["S"][0][0, 0], 2) == g["alice_row_clipped_sum"]
