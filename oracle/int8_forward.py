"""Record-owned LLM.int8 forward of one frozen linear layer, written from the algorithm's steps.

TEST INFRASTRUCTURE ONLY: this module is the reference the library's INT8 forward is checked
against; only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline may use it.  It shares
no code with the library.

Source: "Sensitivity Inflation from Cross-Record Precision Routing in Private Quantized
Fine-Tuning", Sec. 1 Eq. 1 (the batch-wide outlier set O(D)), Sec. 2 (LLM.int8: row-local scales
over the entries below tau, outlier columns zeroed in the INT8 codes and recomputed in FP16, the
two partial products added), Sec. 4.2 Eq. 6 and Algorithm 1 (record-owned routing: each row is
masked with its own record's outlier set O_r; batched LLM.int8 is the case where every row uses
the union U), Appendix A (the constructed witness: its codes, scales and outputs).

Steps, in the algorithm's order (A: n x K fp16 activation rows; rho(i): the record owning row i;
record r owns rows [offsets[r], offsets[r+1])):
  1. M_ij = |A_ij| >= tau                             per-entry test
  2. O_r = {j : M_ij for some row i of record r}      per-record outlier columns
  3. U = union of the O_r                             (public columns to fetch)
  4. s_i = max |A_ij| over the j with M_ij false      row-local scale
  5. Q_ij = round(127 A_ij / s_i) if j not in O_rho(i), else 0
  6. R_ij = A_ij if j in O_rho(i), else 0
  7. Y = dequant(Q Wq^T; s, s_W) + R What^T
The weight is quantised row by row (one scale per output feature):
  s_W[o] = max_j |W_oj|, Wq_oj = round(127 W_oj / s_W[o]), What_oj = dequantised Wq.

Readings where the pages leave the arithmetic open (the library follows the same ones, and the
two sides take every rounding decision in the same IEEE fp32 operations, so results are
compared bit for bit):
  - tau <= 0 (or infinite) disables the outlier path: no entry is an outlier ("threshold zero"
    is the no-outlier control of Sec. 5).
  - round(.) is round-to-nearest, ties to even, of the fp32 value fl(fl(127 A) / s), where
    127 A is exact and the division is correctly rounded.  s = 0 (no nonzero entry below tau)
    gives code 0.  Weights use the same rule with their own scale.
  - dequantisation scales are fl(s / 127) per row and fl(s_W / 127) per output feature:
    the INT8 path's output is fp16(fl(fl(float(acc) * fl(s_i/127)) * fl(s_W/127))), acc being
    the exact integer product; the dequantised weight is What = fp16(fl(Wq * fl(s_W/127))).
  - the FP16 correction accumulates fl(A_ij * What_oj) (exact: fp16 x fp16 fits fp32) in fp32
    over the row owner's outlier columns in ascending order and rounds once to fp16; the two
    fp16 partial outputs are added and rounded to fp16: Y = fp16(dq16 + corr16).
"""
from __future__ import annotations

import math

import numpy as np

F16, F32 = np.float16, np.float32


def _no_outliers(tau: float) -> bool:
    return not (tau > 0) or math.isinf(tau)


def outlier_entries(A: np.ndarray, tau: float) -> np.ndarray:
    """Step 1: the per-entry test |A_ij| >= tau (all false when the outlier path is off)."""
    if _no_outliers(tau):
        return np.zeros(A.shape, dtype=bool)
    return np.abs(A.astype(F32)) >= F32(tau)


def record_outlier_sets(M: np.ndarray, offsets) -> np.ndarray:
    """Step 2: O[r, j] = some row of record r has M true in column j."""
    n_rec = len(offsets) - 1
    O = np.zeros((n_rec, M.shape[1]), dtype=bool)
    for r in range(n_rec):
        lo, hi = int(offsets[r]), int(offsets[r + 1])
        if hi > lo:
            O[r] = M[lo:hi].any(axis=0)
    return O


def row_owners(offsets) -> np.ndarray:
    """rho(i) for every row."""
    n = int(offsets[-1])
    own = np.empty(n, dtype=np.int64)
    for r in range(len(offsets) - 1):
        own[int(offsets[r]):int(offsets[r + 1])] = r
    return own


def row_scales(A: np.ndarray, M: np.ndarray) -> np.ndarray:
    """Step 4: s_i = max |A_ij| over the entries that are not outliers (0 if there are none)."""
    a = np.abs(A.astype(F32))
    a[M] = 0
    return a.max(axis=1) if a.shape[1] else np.zeros(a.shape[0], dtype=F32)


def quant_codes(X: np.ndarray, s: np.ndarray) -> np.ndarray:
    """round(127 x / s) per row in fp32 (ties to even); code 0 where s = 0."""
    x = X.astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (F32(127) * x) / s.astype(F32)[:, None]
    q = np.rint(v)
    q[s == 0, :] = 0
    return q.astype(np.int8)


def quantize_weight(W: np.ndarray):
    """Row-wise weight quantisation: (Wq int8, s_W float32, What fp16)."""
    Wf = W.astype(F32)
    sW = np.abs(Wf).max(axis=1) if Wf.shape[1] else np.zeros(Wf.shape[0], dtype=F32)
    Wq = quant_codes(W, sW)
    What = dequant_weight(Wq, sW)
    return Wq, sW.astype(F32), What


def dequant_weight(Wq: np.ndarray, sW: np.ndarray) -> np.ndarray:
    sb = sW.astype(F32) / F32(127)
    return (Wq.astype(F32) * sb[:, None]).astype(F16)


def forward(A: np.ndarray, offsets, Wq: np.ndarray, sW: np.ndarray, tau: float,
            routing: str = "record") -> dict:
    """Algorithm 1 for one layer.  A: [n, K] fp16; offsets: record boundaries (length n_rec + 1,
    offsets[-1] = n); Wq: [N, K] int8; sW: [N] float32.  routing="record" masks each row with
    its owner's O_r (Eq. 6); routing="batch" uses U for every row (batched LLM.int8, Eq. 1).
    Returns the intermediates and Y ([n, N] fp16)."""
    A = np.asarray(A, dtype=F16)
    n, K = A.shape
    N = Wq.shape[0]
    offsets = np.asarray(offsets, dtype=np.int64)
    assert offsets[0] == 0 and offsets[-1] == n and np.all(np.diff(offsets) >= 0)
    M = outlier_entries(A, tau)                                   # step 1
    O = record_outlier_sets(M, offsets)                           # step 2
    U = O.any(axis=0)                                             # step 3
    s = row_scales(A, M)                                          # step 4
    own = row_owners(offsets)
    if routing == "record":
        row_set = O[own] if n else np.zeros((0, K), dtype=bool)   # O_rho(i) per row
    elif routing == "batch":
        row_set = np.broadcast_to(U, (n, K))
    else:
        raise ValueError(routing)
    Q = quant_codes(A, s)                                         # step 5
    Q[row_set] = 0
    R = np.where(row_set, A, F16(0))                              # step 6
    # step 7, INT8 part: the exact integer product (in fp64: every partial sum is an integer of
    # magnitude <= 127^2 K < 2^53, so any summation order is exact), then the dequantisation
    acc = np.rint(Q.astype(np.float64) @ Wq.astype(np.float64).T).astype(np.int64)
    sa = s.astype(F32) / F32(127)
    sb = sW.astype(F32) / F32(127)
    with np.errstate(over="ignore"):        # fp16 overflow rounds to inf (IEEE)
        dq16 = ((acc.astype(F32) * sa[:, None]) * sb[None, :]).astype(F16)
    # step 7, FP16 part: each row over its own outlier columns, ascending, fp32 accumulation
    What = dequant_weight(Wq, sW)
    corr = np.zeros((n, N), dtype=F32)
    if routing == "record":
        groups = [(int(offsets[r]), int(offsets[r + 1]), np.flatnonzero(O[r]))
                  for r in range(len(offsets) - 1)]
    else:
        groups = [(0, n, np.flatnonzero(U))]
    for lo, hi, cols in groups:
        for j in cols:
            corr[lo:hi] = corr[lo:hi] + (R[lo:hi, j].astype(F32)[:, None] *
                                         What[:, j].astype(F32)[None, :])
    with np.errstate(over="ignore", invalid="ignore"):
        corr16 = corr.astype(F16)
        Y = (dq16.astype(F32) + corr16.astype(F32)).astype(F16)
    return {"M": M, "O": O, "U": U, "s": s, "Q": Q, "R": R, "acc": acc, "dq16": dq16,
            "corr16": corr16, "Y": Y}


def forward_one_record_at_a_time(A: np.ndarray, offsets, Wq, sW, tau: float) -> np.ndarray:
    """The reference semantics of Sec. 4.2: LLM.int8 run on all tokens of one record at a time
    (each record a batch of its own); the rows' outputs concatenated in order."""
    A = np.asarray(A, dtype=F16)
    outs = []
    for r in range(len(offsets) - 1):
        lo, hi = int(offsets[r]), int(offsets[r + 1])
        outs.append(forward(A[lo:hi], [0, hi - lo], Wq, sW, tau, "batch")["Y"])
    if not outs:
        return np.zeros((0, Wq.shape[0]), dtype=F16)
    return np.concatenate(outs, axis=0)
