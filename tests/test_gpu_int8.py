"""GPU parity of the record-owned LLM.int8 forward ("Sensitivity Inflation from Cross-Record
Precision Routing in Private Quantized Fine-Tuning", Eq. 6 / Algorithm 1) against the oracle.

Both sides take every rounding decision in the same IEEE operations, so everything is compared
bit for bit: the weight codes and scales, the per-record outlier masks, row owners, row scales,
activation codes and the fp16 output.  Covered: the App. A witness (record-owned and batched
as a single record), the vector and scalar load paths (k % 8), ragged row and feature tails of
both GEMM tile shapes, empty records, one-row records (a tile spanning many records), more than
one correction chunk (more than 32 union columns in a tile), threshold zero, batch invariance
(a record alone vs in a batch, and with another record added) and the OPT-125M layer shapes at
B = 16, T = 256.
"""
import json
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import differentially_private_amd as dp  # noqa: E402
from datagen import int8 as gen  # noqa: E402
from oracle import int8_forward as o8  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
F16 = np.float16


def say(*a):
    print(*a, flush=True)


class Layer:
    """A frozen weight quantised on the GPU, checked against the oracle's quantisation."""

    def __init__(self, W: np.ndarray):
        self.N, self.K = W.shape
        self.W = W
        self.pitch = dp.i8_pitch(self.K)
        dW = torch.from_numpy(np.ascontiguousarray(W)).to(DEV)
        self.wq = torch.full((self.N, self.pitch), 99, dtype=torch.int8, device=DEV)
        self.sw = torch.full((self.N,), -1.0, dtype=torch.float32, device=DEV)
        dp.i8_quantize_weight(dW, self.N, self.K, self.wq, self.sw)
        torch.cuda.synchronize()
        self.Wq_ref, self.sW_ref, _ = o8.quantize_weight(W)
        wq = self.wq.cpu().numpy()
        assert np.array_equal(wq[:, :self.K], self.Wq_ref)
        assert np.all(wq[:, self.K:] == 0)
        assert np.array_equal(self.sw.cpu().numpy(), self.sW_ref)


def run(A: np.ndarray, offsets, layer: Layer, tau=6.0, plan=None, ws=None):
    n, K = A.shape
    n_rec = len(offsets) - 1
    if plan is None:
        plan = dp.I8Plan(max(n, 1), max(n_rec, 1), K)
        ws = plan.workspace(DEV)
    dA = torch.from_numpy(np.ascontiguousarray(A)).to(DEV)
    Y = torch.full((n, layer.N), float("nan"), dtype=torch.float16, device=DEV)
    dp.i8_set_records(plan, ws, offsets)
    dp.i8_forward(plan, ws, n, n_rec, dA, K, layer.wq, layer.sw, layer.N, tau, Y)
    q = torch.empty((n, layer.pitch), dtype=torch.int8, device=DEV)
    s = torch.empty(n, dtype=torch.float32, device=DEV)
    om = torch.empty((n_rec, (K + 31) // 32), dtype=torch.int32, device=DEV)
    own = torch.empty(n, dtype=torch.int32, device=DEV)
    dp.i8_intermediates(plan, ws, n, n_rec, K, q, s, om, own)
    torch.cuda.synchronize()
    omask = om.cpu().numpy().view(np.uint32)
    O = np.zeros((n_rec, K), dtype=bool)
    for j in range(K):
        O[:, j] = (omask[:, j // 32] >> np.uint32(j % 32)) & 1
    return {"Y": Y.cpu().numpy(), "Q": q.cpu().numpy(), "s": s.cpu().numpy(), "O": O,
            "own": own.cpu().numpy()}


def check(A, offsets, layer, tau=6.0, routing="record"):
    got = run(A, offsets, layer, tau)
    ref = o8.forward(A, offsets, layer.Wq_ref, layer.sW_ref, tau, routing)
    n, K = A.shape
    assert np.array_equal(got["own"], o8.row_owners(offsets))
    assert np.array_equal(got["O"], ref["O"])
    assert np.array_equal(got["s"], ref["s"])
    assert np.array_equal(got["Q"][:, :K], ref["Q"]) and np.all(got["Q"][:, K:] == 0)
    same = (got["Y"].view(np.uint16) == ref["Y"].view(np.uint16))
    if not same.all():
        bad = np.argwhere(~same)[:5]
        say("  mismatches", int((~same).sum()), "first", bad.tolist(),
            [(float(got["Y"][i, j]), float(ref["Y"][i, j])) for i, j in bad])
    assert same.all()
    say(f"  n={n} K={K} N={layer.N} records={len(offsets) - 1} union={int(ref['U'].sum())} "
        f"bit-exact")
    return got, ref


def witness_rows(golden_dir, key):
    g = json.load(open(os.path.join(golden_dir, "p5_int8_witness.json")))
    rows = [g["unchanged_row"]] * g["n_unchanged"] + [g[key]]
    return g, np.array(rows, dtype=F16), Layer(np.array(g["weight"], dtype=F16))


def test_app_a_witness_on_gpu(golden_dir):
    """App. A: eight one-row records.  Record-owned: the unchanged rows give the INT8 value
    1.220703125 in D and D'.  As one batch-wide record (batched LLM.int8) D' gives 1.234375."""
    say("App. A witness")
    g, A, L = witness_rows(golden_dir, "replaced_row_D")
    _, A2, _ = witness_rows(golden_dir, "replaced_row_Dprime")
    n = g["n_unchanged"]
    one_each = np.arange(n + 2)
    y1, _ = check(A, one_each, L)
    y2, _ = check(A2, one_each, L)
    assert np.all(y1["Y"][:n, 0] == g["out_int8_path"])
    assert np.array_equal(y1["Y"][:n], y2["Y"][:n])
    assert np.all(y1["Q"][:n, 0] == g["code_unchanged_col0"]) and np.all(y1["s"] == g["row_scale"])
    b1, _ = check(A, [0, n + 1], L, routing="batch")
    b2, _ = check(A2, [0, n + 1], L, routing="batch")
    assert np.all(b1["Y"][:n, 0] == g["out_int8_path"])
    assert np.all(b2["Y"][:n, 0] == g["out_fp16_path"])


CASES = [
    # name, lens, K, N, kwargs for the generator
    ("small_vec", [5, 3, 8, 1], 40, 24, {}),
    ("scalar_k", [5, 3, 8, 1], 37, 30, {}),
    ("empty_records", [0, 7, 0, 12, 2, 0], 96, 17, {"p_owned": 1.0}),
    ("one_row_records", [1] * 300, 64, 40, {"p_owned": 0.5}),
    ("ragged_small_tiles", [130, 97, 51], 200, 261, {"p_owned": 1.0}),
    ("big_tiles", [256] * 16, 72, 4096, {}),
    ("big_tiles_ragged_scalar", [300] * 13 + [137], 100, 4116, {"p_owned": 0.6}),
    # rows wider than one batch of the routing kernels' loads (3072 columns), ragged: a second,
    # partial batch; not a multiple of 8: the element-wise path; the largest K the plan takes
    ("wide_k_two_load_batches", [40, 25, 63], 5000, 96, {"p_owned": 1.0}),
    ("wide_k_scalar", [17, 30], 6147, 40, {}),
    ("max_k", [3, 5, 2], 32768, 24, {"p_owned": 1.0}),
]


@pytest.mark.parametrize("name,lens,K,N,kw", CASES, ids=[c[0] for c in CASES])
def test_forward_matches_oracle(name, lens, K, N, kw):
    say("int8 forward", name)
    A, offsets, _, _ = gen.activations(len(name) + K, lens, K, **kw)
    L = Layer(gen.weights(K + N, N, K))
    check(A, offsets, L)


def test_many_union_columns():
    """More than 32 union columns in a tile (several correction chunks), rows owning 0, a few,
    or 70 outlier columns; also exact threshold values."""
    rng = np.random.default_rng(21)
    K, N = 160, 72
    lens = [40, 30, 50, 8]
    offsets = gen.lengths_offsets(lens)
    A = rng.standard_normal((offsets[-1], K)).astype(np.float32)
    A[0:40:3, 10:80] = 7.5                        # record 0 owns 70 columns
    A[45, 100:105] = -9.0                         # record 1 owns 5
    A[80, 150] = 6.0                              # record 2: exactly tau
    A[81, 151] = 5.99609375                       # largest fp16 below tau: not an outlier
    A = A.astype(F16)
    L = Layer(gen.weights(3, N, K))
    got, ref = check(A, offsets, L)
    assert ref["O"][0].sum() == 70 and ref["O"][2, 150] and not ref["O"][2, 151]
    assert not ref["O"][3].any()


def test_threshold_zero():
    A, offsets, _, _ = gen.activations(5, [20, 30], 64, p_owned=1.0)
    L = Layer(gen.weights(5, 48, 64))
    got, ref = check(A, offsets, L, tau=0.0)
    assert not got["O"].any()


def test_batch_invariance():
    """Sec. 8's recommended check: each record's output alone equals its output in the batch
    (bitwise), and adding a record that owns a new outlier column changes no other row."""
    lens = [24, 40, 17, 33]
    A, offsets, shared, owned = gen.activations(31, lens, 128, p_owned=1.0)
    L = Layer(gen.weights(31, 96, 128))
    full = run(A, offsets, L)["Y"]
    for r in range(len(lens)):
        lo, hi = offsets[r], offsets[r + 1]
        alone = run(A[lo:hi], [0, hi - lo], L)["Y"]
        assert np.array_equal(alone.view(np.uint16), full[lo:hi].view(np.uint16))
    extra = np.random.default_rng(32).standard_normal((9, 128)).astype(F16)
    free = np.setdiff1d(np.arange(128), np.concatenate([shared, list(owned.values())]))[0]
    extra[4, free] = 11.0
    A2 = np.concatenate([A, extra])
    off2 = np.concatenate([offsets, [offsets[-1] + 9]])
    more = run(A2, off2, L)["Y"]
    assert np.array_equal(more[:offsets[-1]].view(np.uint16), full.view(np.uint16))
    # batched routing (one record over all rows) is not invariant here
    b1 = run(A, [0, offsets[-1]], L)["Y"]
    b2 = run(A2, [0, off2[-1]], L)["Y"]
    assert not np.array_equal(b1.view(np.uint16), b2[:offsets[-1]].view(np.uint16))


def test_workspace_reuse_across_shapes():
    """One plan and workspace for layers of different widths in a row (as in a model's forward):
    each call's masks are cleared and its codes laid out at its own pitch."""
    lens = [64, 64, 32]
    plan = dp.I8Plan(160, 3, 300)
    ws = plan.workspace(DEV)
    for K, N, seed in [(300, 40, 1), (96, 300, 2), (256, 64, 3)]:
        A, offsets, _, _ = gen.activations(seed, lens, K, p_owned=1.0)
        L = Layer(gen.weights(seed, N, K))
        got = run(A, offsets, L, plan=plan, ws=ws)
        ref = o8.forward(A, offsets, L.Wq_ref, L.sW_ref, 6.0)
        assert np.array_equal(got["Y"].view(np.uint16), ref["Y"].view(np.uint16))
        assert np.array_equal(got["O"], ref["O"])


@pytest.mark.parametrize("K,N", [(768, 768), (768, 3072), (3072, 768)])
def test_opt125m_layer_shapes(K, N):
    """The OPT-125M frozen layers (attention projections, the two feed-forward projections) at
    the pages' physical batch B = 16 of T = 256 tokens, full output compared."""
    say("OPT-125M layer", K, "->", N)
    A, offsets, _, _ = gen.activations(K * 7 + N, [256] * 16, K)
    L = Layer(gen.weights(K + 3 * N, N, K))
    check(A, offsets, L)


def test_graph_replay_matches_eager():
    """Three layers' forwards captured into one HIP graph: every replay (with eager work and
    synchronisations between replays) gives bitwise the eager outputs."""
    lens = [64] * 4
    shapes = [(256, 128), (128, 384), (384, 96)]
    plan = dp.I8Plan(256, 4, 384)
    ws = plan.workspace(DEV)
    A_dev, layers, Ys = [], [], []
    for idx, (K, N) in enumerate(shapes):
        A, offsets, _, _ = gen.activations(40 + idx, lens, K, p_owned=1.0)
        A_dev.append(torch.from_numpy(A).to(DEV))
        layers.append(Layer(gen.weights(40 + idx, N, K)))
        Ys.append(torch.empty((256, N), dtype=torch.float16, device=DEV))
    dp.i8_set_records(plan, ws, offsets)

    def fwd():
        for A, L, Y in zip(A_dev, layers, Ys):
            dp.i8_forward(plan, ws, 256, 4, A, A.shape[1], L.wq, L.sw, L.N, 6.0, Y)

    fwd()
    torch.cuda.synchronize()
    eager = [y.clone() for y in Ys]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    for rep in range(4):
        for y in Ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, e in zip(Ys, eager):
            assert torch.equal(y.view(torch.int16), e.view(torch.int16)), rep
        fwd()          # eager work between replays
        torch.cuda.synchronize()


def test_wide_layer_and_odd_features():
    """k = 16384 (512 mask words per record, tile unions over many words), 203 output features
    (no 8-byte output stores), records of 100-300 rows."""
    say("int8 wide layer")
    A, offsets, _, _ = gen.activations(61, [100, 300, 160], 16384, n_shared=5, p_owned=1.0)
    L = Layer(gen.weights(61, 203, 16384))
    check(A, offsets, L)


def test_misaligned_activations():
    """Activation rows whose base is 2 bytes past a 16-byte boundary take the element-wise load
    path even with k a multiple of 8; same results as the aligned buffer."""
    A, offsets, _, _ = gen.activations(62, [40, 25], 64, p_owned=1.0)
    L = Layer(gen.weights(62, 36, 64))
    n, K = A.shape
    plan = dp.I8Plan(n, 2, K)
    ws = plan.workspace(DEV)
    buf = torch.zeros(n * K + 8, dtype=torch.float16, device=DEV)
    buf[1:1 + n * K] = torch.from_numpy(A.reshape(-1)).to(DEV)
    mis = buf[1:1 + n * K]
    assert mis.data_ptr() % 16 != 0
    Y = torch.empty((n, L.N), dtype=torch.float16, device=DEV)
    dp.i8_set_records(plan, ws, offsets)
    dp.i8_forward(plan, ws, n, 2, mis, K, L.wq, L.sw, L.N, 6.0, Y)
    torch.cuda.synchronize()
    ref = o8.forward(A, offsets, L.Wq_ref, L.sW_ref, 6.0)
    assert np.array_equal(Y.cpu().numpy().view(np.uint16), ref["Y"].view(np.uint16))


def test_thousand_short_records():
    """1,000 records of 0-5 rows: the owner search over many records, tiles spanning hundreds of
    records (and empty ones between them)."""
    rng = np.random.default_rng(63)
    lens = rng.integers(0, 6, 1000)
    A, offsets, _, _ = gen.activations(63, lens, 96, p_owned=0.5)
    L = Layer(gen.weights(63, 72, 96))
    check(A, offsets, L)


def test_max_width():
    """The largest supported k (32768): mask words at the limit of a tile's union buffer."""
    say("int8 max width")
    A, offsets, _, _ = gen.activations(64, [20, 12], 32768, n_shared=8, p_owned=1.0)
    L = Layer(gen.weights(64, 40, 32768))
    check(A, offsets, L)


def _near_half_rows(K):
    """fp16 rows whose quotients 127 a / s fall on or next to half-integers: exact ties (s = 127/64,
    a = (k + 1/2)/64, so 127 a / s = k + 1/2) and, for other row maxima s, every fp16 value a in
    (0, s] whose quotient lies within 1e-3 of a half-integer, with both signs."""
    rows = []
    tie = np.array([(k + 0.5) / 64 for k in range(126)], dtype=np.float64)
    extra = np.random.default_rng(43).uniform(0.05, 5.99, 40)
    for s in [127 / 64, 1.0, 2.9921875, 5.99609375, 0.3330078125, 4.125, 0.0999755859375, *extra]:
        s16 = F16(s)
        grid = np.arange(1, 65536, dtype=np.uint16).view(F16).astype(np.float64)   # all positive fp16
        grid = grid[np.isfinite(grid) & (grid > 0) & (grid <= float(s16))]
        q = 127.0 * grid / float(s16)
        near = grid[np.abs(q - np.floor(q) - 0.5) < 1e-3]
        vals = np.concatenate([tie if s == 127 / 64 else near, [float(s16)]])
        vals = np.concatenate([vals, -vals[: len(vals) // 2]])
        for i in range(0, len(vals), K - 1):
            chunk = vals[i:i + K - 1]
            row = np.zeros(K, dtype=np.float64)
            row[: len(chunk)] = chunk
            row[-1] = float(s16)          # the row's maximum, below the outlier threshold
            rows.append(row)
    return np.array(rows).astype(F16)


def test_codes_near_half_integers():
    """Codes round(127 a / s) where the quotient is a tie or within 1e-3 of one (where the
    rounding of the division and ties-to-even decide the code): bit-exact with the oracle."""
    K = 256
    A = _near_half_rows(K)
    n = A.shape[0]
    offsets = [0, n // 3, n]
    say("int8 near-half codes", n, "rows")
    L = Layer(gen.weights(41, 64, K))
    check(A, offsets, L)


def _random_forward(i):
    rng = np.random.default_rng(90000 + i)
    K = int(rng.choice([int(rng.integers(1, 600)), 32 * int(rng.integers(1, 40))]))
    N = int(rng.integers(1, 700))
    lens = [int(x) for x in rng.integers(0, 90, int(rng.integers(1, 30)))]
    if sum(lens) == 0:
        lens[0] = 1
    tau = float(rng.choice([6.0, 3.0, 1.5, 0.0]))
    one_record = rng.random() >= 0.8
    return K, N, lens, tau, one_record, int(rng.integers(0, 5)), float(rng.random())


@pytest.mark.parametrize("i", range(20))
def test_random_forwards(i):
    """Random layers (K of 1-599 or whole 32-column groups, 1-699 features), 1-29 records of
    0-89 rows, thresholds 0-6, record-owned or one record over the batch: bit-exact."""
    K, N, lens, tau, one_record, n_shared, p_owned = _random_forward(i)
    say("int8 random", i, "K", K, "N", N, "records", len(lens), "tau", tau, "one record", one_record)
    A, offsets, _, _ = gen.activations(i, lens, K, tau=max(tau, 1.0), n_shared=n_shared, p_owned=p_owned)
    L = Layer(gen.weights(i, N, K))
    check(A, [0, int(offsets[-1])] if one_record else offsets, L, tau=tau)
