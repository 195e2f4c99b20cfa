"""Pins of the INT8-forward oracle (record-owned LLM.int8 of "Sensitivity Inflation from
Cross-Record Precision Routing in Private Quantized Fine-Tuning", Eq. 6 / Algorithm 1) against
what the pages and the mathematics fix.  No GPU.

A plausible mistake in the oracle fails at least one of these:
- a wrong outlier test, scale or code: the App. A witness values (code 31, scale 5,
  1.220703125 / 1.234375) and the exact-rational codes, ties included;
- a wrong owner (row masked with another record's set, or with the union): the
  one-record-at-a-time reference semantics of Sec. 4.2 and the per-row mask check;
- a dropped or transposed correction, a wrong dequantisation scale: the closed forms on exactly
  representable grids and the quantisation error bound against the fp64 product.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from datagen import int8 as gen
from oracle import int8_forward as o8

F16 = np.float16


def witness(golden_dir, replaced_key):
    g = json.load(open(os.path.join(golden_dir, "p5_int8_witness.json")))
    rows = [g["unchanged_row"]] * g["n_unchanged"] + [g[replaced_key]]
    A = np.array(rows, dtype=F16)
    W = np.array(g["weight"], dtype=F16)
    offsets = np.arange(len(rows) + 1)
    Wq, sW, _ = o8.quantize_weight(W)
    return g, A, offsets, Wq, sW


@pytest.mark.parametrize("key", ["replaced_row_D", "replaced_row_Dprime"])
def test_app_a_witness_batched(golden_dir, key):
    """Appendix A: under the batch-wide union the unchanged rows' output is the INT8 value
    1.220703125 (code 31, scale 5) in D and the FP16 value 1.234375 in D'."""
    g, A, off, Wq, sW = witness(golden_dir, key)
    r = o8.forward(A, off, Wq, sW, g["tau"], "batch")
    n = g["n_unchanged"]
    assert np.all(r["s"] == g["row_scale"])
    union = np.flatnonzero(r["U"]).tolist()
    if key == "replaced_row_D":
        assert union == g["union_D"]
        assert np.all(r["Q"][:n, 0] == g["code_unchanged_col0"])
        assert np.all(r["Y"][:n, 0] == g["out_int8_path"])
    else:
        assert union == g["union_Dprime"]
        assert np.all(r["Q"][:n, 0] == 0)
        assert np.all(r["Y"][:n, 0] == g["out_fp16_path"])


def test_app_a_witness_record_owned(golden_dir):
    """Eq. 6: with record-owned routing the unchanged records keep the INT8 value in both
    batches; only the replaced record (whose own set now holds column 0) takes the FP16 path."""
    g, A, off, Wq, sW = witness(golden_dir, "replaced_row_D")
    _, A2, _, _, _ = witness(golden_dir, "replaced_row_Dprime")
    n = g["n_unchanged"]
    y1 = o8.forward(A, off, Wq, sW, g["tau"])["Y"]
    r2 = o8.forward(A2, off, Wq, sW, g["tau"])
    assert np.all(y1[:n, 0] == g["out_int8_path"])
    assert np.array_equal(y1[:n], r2["Y"][:n])
    assert r2["O"][n].tolist() == [True, False, False, False] and not r2["O"][:n].any()
    assert r2["Y"][n, 0] == F16(6.1) * F16(1.0)


def test_owned_fp16_path_value(golden_dir):
    """A record whose own other row crosses tau routes the entry 1.234 to FP16 (1.234375)."""
    g = json.load(open(os.path.join(golden_dir, "p5_int8_witness.json")))
    A = np.array([g["unchanged_row"], g["replaced_row_Dprime"]], dtype=F16)
    Wq, sW, _ = o8.quantize_weight(np.array(g["weight"], dtype=F16))
    r = o8.forward(A, [0, 2], Wq, sW, g["tau"])
    assert r["Y"][0, 0] == g["out_fp16_path"]


def random_layer(seed, lens, K, N, **kw):
    L = gen.layer(seed, lens, K, N, **kw)
    Wq, sW, _ = o8.quantize_weight(L.W)
    return L, Wq, sW


@pytest.mark.parametrize("seed,lens,K,N", [(1, [5, 3, 8, 1], 40, 24), (2, [16] * 6, 64, 33),
                                           (3, [0, 7, 0, 12, 2], 96, 17)])
def test_record_owned_is_one_record_at_a_time(seed, lens, K, N):
    """Sec. 4.2: the reference semantics runs LLM.int8 on one record's tokens at a time; the
    batched record-owned forward gives bitwise the same rows."""
    L, Wq, sW = random_layer(seed, lens, K, N, p_owned=0.8)
    y = o8.forward(L.A, L.offsets, Wq, sW, 6.0)["Y"]
    ref = o8.forward_one_record_at_a_time(L.A, L.offsets, Wq, sW, 6.0)
    assert np.array_equal(y, ref)
    if L.owned:   # the batched union differs on some row of a record that does not own a column
        yb = o8.forward(L.A, L.offsets, Wq, sW, 6.0, "batch")["Y"]
        assert not np.array_equal(y, yb)


def test_singleton_batch_and_threshold_zero():
    """Sec. 4.2 'Simpler alternatives': a singleton batch and threshold zero both make the two
    routings agree; threshold zero has no FP16 path at all."""
    L, Wq, sW = random_layer(4, [9], 48, 20, p_owned=1.0)
    a = o8.forward(L.A, L.offsets, Wq, sW, 6.0)
    b = o8.forward(L.A, L.offsets, Wq, sW, 6.0, "batch")
    assert a["U"].any() and np.array_equal(a["Y"], b["Y"])
    L, Wq, sW = random_layer(5, [4, 6, 3], 48, 20, p_owned=1.0)
    for tau in (0.0, float("inf")):
        a = o8.forward(L.A, L.offsets, Wq, sW, tau)
        b = o8.forward(L.A, L.offsets, Wq, sW, tau, "batch")
        assert not a["U"].any() and np.all(a["corr16"] == 0)
        assert np.array_equal(a["Y"], b["Y"])
        assert np.array_equal(a["s"], np.abs(L.A.astype(np.float32)).max(axis=1))


def exact_round(x: Fraction) -> int:
    return round(x)          # Fraction rounding: nearest, ties to even


def test_codes_match_exact_rational():
    """round(127 a / s): the fp32 quotient gives the exactly rounded rational except within
    2^-16 of a half-integer; exact ties go to the even code."""
    rng = np.random.default_rng(6)
    A = (rng.standard_normal((50, 64)) * 2).astype(F16)
    M = o8.outlier_entries(A, 6.0)
    s = o8.row_scales(A, M)
    Q = o8.quant_codes(A, s)
    checked = 0
    for i in range(A.shape[0]):
        for j in range(A.shape[1]):
            if M[i, j]:
                continue
            x = Fraction(float(A[i, j])) * 127 / Fraction(float(s[i]))
            assert abs(Q[i, j] - x) <= Fraction(1, 2) + Fraction(1, 1 << 16)
            if abs(abs(x - int(x)) - Fraction(1, 2)) > Fraction(1, 1 << 16):
                assert Q[i, j] == exact_round(x)
                checked += 1
    assert checked > 2000
    # exact ties: s = 127/32, a = (2k+1)/64 gives 127 a / s = k + 1/2
    s_tie = np.float32(127 / 32)
    ks = np.arange(0, 127)
    a = ((2 * ks + 1) / 64).astype(F16)
    row = np.concatenate([[s_tie], a]).astype(F16)[None, :]
    q = o8.quant_codes(row, np.array([s_tie], dtype=np.float32))[0, 1:]
    want = [exact_round(Fraction(2 * k + 1, 2)) for k in ks]
    assert q.tolist() == want and q[0] == 0 and q[1] == 2     # 0.5 -> 0, 1.5 -> 2


def test_exact_grid_closed_form():
    """Activations and weights on the grid m/64 with a row maximum of 127/64: every code is m,
    both scales are 1/64, and Y is the exact product rounded once to fp16."""
    rng = np.random.default_rng(7)
    n, K, N = 12, 32, 10
    ma = rng.integers(-127, 128, (n, K))
    ma[:, 0] = 127
    mw = rng.integers(-127, 128, (N, K))
    mw[:, 3] = -127
    A = (ma / 64).astype(F16)
    W = (mw / 64).astype(F16)
    Wq, sW, What = o8.quantize_weight(W)
    assert np.array_equal(Wq, mw) and np.array_equal(What, W)
    r = o8.forward(A, [0, 5, n], Wq, sW, 6.0)
    assert not r["U"].any() and np.array_equal(r["Q"], ma)
    exact = (ma @ mw.T) / 4096.0          # exact in fp64 (integers over a power of two)
    assert np.array_equal(r["Y"], exact.astype(F16))


def test_all_outlier_rows_closed_form():
    """A record whose every column crosses tau runs entirely on the FP16 path: with integer
    activations and weights on the grid m/64 (row maximum 127/64, so What = W) the fp32 sum is
    exact."""
    rng = np.random.default_rng(8)
    K, N = 16, 8
    A = rng.integers(6, 40, (3, K)) * rng.choice([-1, 1], (3, K))
    A = A.astype(F16)
    mw = rng.integers(-127, 128, (N, K))
    mw[:, 0] = 127
    W = (mw / 64).astype(F16)
    Wq, sW, What = o8.quantize_weight(W)
    assert np.array_equal(What, W)
    r = o8.forward(A, [0, 3], Wq, sW, 6.0)
    assert r["O"].all() and np.all(r["s"] == 0) and np.all(r["Q"] == 0)
    exact = A.astype(np.float64) @ W.astype(np.float64).T
    assert np.array_equal(r["Y"], exact.astype(F16))


def test_owner_masks():
    """Steps 5-6: row i's codes are zero exactly on O_rho(i), and R holds A exactly there."""
    L, Wq, sW = random_layer(9, [6, 6, 6, 6, 6], 80, 12, p_owned=1.0, n_shared=2)
    r = o8.forward(L.A, L.offsets, Wq, sW, 6.0)
    for rec in range(5):
        lo, hi = L.offsets[rec], L.offsets[rec + 1]
        cols = set(L.shared.tolist()) | ({L.owned[rec]} if rec in L.owned else set())
        have = set(np.flatnonzero(r["O"][rec]).tolist())
        assert have <= cols and have >= {L.owned.get(rec, -1)} - {-1}
        for i in range(lo, hi):
            assert np.all(r["Q"][i, r["O"][rec]] == 0)
            assert np.array_equal(r["R"][i, r["O"][rec]], L.A[i, r["O"][rec]])
            assert np.all(r["R"][i, ~r["O"][rec]] == 0)
    assert sorted(np.flatnonzero(r["U"]).tolist()) == sorted(set(np.flatnonzero(r["O"].any(0))))


def test_weight_quantization():
    """Row-wise weight codes: the row maximum codes to +-127, every dequantised weight within
    half a code step (plus half an fp16 spacing) of the weight."""
    W = gen.weights(3, 40, 72)
    Wq, sW, What = o8.quantize_weight(W)
    Wf = W.astype(np.float64)
    assert np.all(np.abs(Wq).max(axis=1) == 127)
    assert np.array_equal(sW, np.abs(W.astype(np.float32)).max(axis=1))
    step = sW.astype(np.float64)[:, None] / 127
    err = np.abs(What.astype(np.float64) - Wf)
    assert np.all(err <= step / 2 * (1 + 1e-6) + np.spacing(np.abs(What).astype(F16)).astype(np.float64))


@pytest.mark.parametrize("routing", ["record", "batch"])
def test_quantization_error_bound(routing):
    """|Y - A W^T| within the quantisation bound: half a code step per entry of each operand,
    plus the fp16 roundings of the dequantised weight, the two partial outputs and their sum."""
    L, Wq, sW = random_layer(10, [20, 30, 14], 128, 48, p_owned=1.0)
    r = o8.forward(L.A, L.offsets, Wq, sW, 6.0, routing)
    A = L.A.astype(np.float64)
    W = L.W.astype(np.float64)
    What = o8.dequant_weight(Wq, sW).astype(np.float64)
    exact = A @ W.T
    own = o8.row_owners(L.offsets)
    rs = r["O"][own] if routing == "record" else np.broadcast_to(r["U"], A.shape)
    da = np.where(rs, 0.0, r["s"].astype(np.float64)[:, None] / 254)       # |a - a_hat|
    dw = np.abs(What - W)                                                   # |w - w_hat|
    bound = da @ np.abs(W).T + np.abs(A) @ dw.T + da @ dw.T
    y = r["Y"].astype(np.float64)
    parts = np.abs(r["dq16"].astype(np.float64)) + np.abs(r["corr16"].astype(np.float64))
    rnd = np.spacing((parts + np.abs(y)).astype(F16)).astype(np.float64) * 2
    err = np.abs(y - exact)
    assert np.all(err <= bound * (1 + 1e-5) + rnd)
    assert np.max(err) < 0.05 * np.max(np.abs(exact))


def test_batch_invariance_of_record_owned_routing():
    """Sec. 8 (recommendations): compare each record's output under batching with its output
    alone.  Adding a record that owns a new outlier column leaves every other record's
    record-owned output bitwise unchanged; the batched union changes them."""
    L, Wq, sW = random_layer(11, [10, 10, 10], 64, 16, p_owned=0.0)
    extra = np.array(np.random.default_rng(12).standard_normal((4, 64)), dtype=F16)
    free = np.setdiff1d(np.arange(64), L.shared)[0]
    extra[1, free] = 9.0
    A2 = np.concatenate([L.A, extra])
    off2 = np.concatenate([L.offsets, [L.offsets[-1] + 4]])
    n = L.A.shape[0]
    y1 = o8.forward(L.A, L.offsets, Wq, sW, 6.0)["Y"]
    y2 = o8.forward(A2, off2, Wq, sW, 6.0)["Y"]
    assert np.array_equal(y1, y2[:n])
    for r in range(3):
        lo, hi = L.offsets[r], L.offsets[r + 1]
        alone = o8.forward(L.A[lo:hi], [0, hi - lo], Wq, sW, 6.0)["Y"]
        assert np.array_equal(alone, y1[lo:hi])
    b1 = o8.forward(L.A, L.offsets, Wq, sW, 6.0, "batch")["Y"]
    b2 = o8.forward(A2, off2, Wq, sW, 6.0, "batch")["Y"]
    assert not np.array_equal(b1, b2[:n])


def test_threshold_is_inclusive():
    """Step 1 tests |a| >= tau: an entry of exactly 6 is an outlier (its column joins O_r and
    leaves the row scale), the largest fp16 below 6 (5.99609375) is not."""
    A = np.array([[6.0, 1.0, 0.5, -2.0], [5.99609375, 1.0, 0.5, -2.0], [-6.0, 0.0, 0.0, 3.0]],
                 dtype=F16)
    M = o8.outlier_entries(A, 6.0)
    assert M.tolist() == [[True, False, False, False], [False] * 4, [True, False, False, False]]
    s = o8.row_scales(A, M)
    assert s.tolist() == [2.0, 5.99609375, 3.0]
    r = o8.forward(A, [0, 1, 2, 3], *o8.quantize_weight(np.eye(4, dtype=F16))[:2], 6.0)
    assert r["O"][:, 0].tolist() == [True, False, True]
    assert r["Q"][1, 0] == 127 and r["Q"][0, 0] == 0 and r["Q"][2, 0] == 0
    assert r["Y"][0, 0] == 6.0 and r["Y"][2, 0] == -6.0


def test_integer_product_is_exact():
    """The INT8 accumulator equals the int64 product of the codes at the largest K (32768) with
    every code at +-127 (the extreme partial sums)."""
    rng = np.random.default_rng(13)
    K = 32768
    Q = rng.choice(np.array([-127, 127], dtype=np.int8), (3, K))
    Wq = rng.choice(np.array([-127, 127], dtype=np.int8), (2, K))
    Wq[0] = Q[0]
    A = (Q.astype(np.float32) / 64).astype(F16)          # row scale 127/64: codes are Q
    r = o8.forward(A, [0, 3], Wq, np.full(2, 127 / 64, dtype=np.float32), 6.0)
    assert np.array_equal(r["Q"], Q)
    assert np.array_equal(r["acc"], Q.astype(np.int64) @ Wq.astype(np.int64).T)
    assert r["acc"][0, 0] == 127 * 127 * K
