"""Seeded synthetic inputs for the INT8 forward of a frozen layer (activations with outlier
columns, fp16 weights).  Holds none of the method's arithmetic.

Recipe (shaped after the natural-text traces of "Sensitivity Inflation from Cross-Record
Precision Routing in Private Quantized Fine-Tuning", Sec. 6.2: a few outlier columns per layer,
most of them shared by every record, a handful owned by a single record):
  - activations A[row, j] ~ N(0, 1), rounded to fp16;
  - n_shared systematic columns (the same for every record): each token row of every record
    takes a value of magnitude U[tau, 3 tau] with probability p_token, random sign;
  - with probability p_owned a record owns one private outlier column (not a shared one): 1 to 3
    of its rows take a magnitude U[tau, 2 tau] there;
  - weights W[o, j] ~ N(0, w_std), rounded to fp16.
Records are given by their row counts; offsets are the running sums.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Int8Layer:
    A: np.ndarray          # [n, K] fp16
    offsets: np.ndarray    # [n_rec + 1] int64
    W: np.ndarray          # [N, K] fp16
    shared: np.ndarray     # systematic outlier columns
    owned: dict            # record -> private column


def lengths_offsets(lens) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lens, dtype=np.int64))]).astype(np.int64)


def activations(seed: int, lens, K: int, tau: float = 6.0, n_shared: int = 3,
                p_token: float = 0.25, p_owned: float = 0.3):
    rng = np.random.default_rng(seed)
    offsets = lengths_offsets(lens)
    n = int(offsets[-1])
    A = rng.standard_normal((n, K), dtype=np.float32)
    n_shared = min(n_shared, K)
    shared = rng.choice(K, n_shared, replace=False) if n_shared else np.zeros(0, dtype=np.int64)
    if n_shared and n:
        hit = rng.random((n, n_shared)) < p_token
        mag = rng.uniform(tau, 3 * tau, (n, n_shared)) * rng.choice([-1.0, 1.0], (n, n_shared))
        cols = A[:, shared]
        cols[hit] = mag[hit]
        A[:, shared] = cols
    owned = {}
    free = np.setdiff1d(np.arange(K), shared)
    for r in range(len(offsets) - 1):
        lo, hi = int(offsets[r]), int(offsets[r + 1])
        if hi > lo and free.size and rng.random() < p_owned:
            j = int(rng.choice(free))
            rows = rng.choice(np.arange(lo, hi), min(hi - lo, int(rng.integers(1, 4))), replace=False)
            A[rows, j] = rng.uniform(tau, 2 * tau, rows.size) * rng.choice([-1.0, 1.0], rows.size)
            owned[r] = j
    return A.astype(np.float16), offsets, shared, owned


def weights(seed: int, N: int, K: int, w_std: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng(seed + 0x5EED)
    return (rng.standard_normal((N, K), dtype=np.float32) * w_std).astype(np.float16)


def layer(seed: int, lens, K: int, N: int, **kw) -> Int8Layer:
    A, offsets, shared, owned = activations(seed, lens, K, **kw)
    return Int8Layer(A=A, offsets=offsets, W=weights(seed, N, K), shared=shared, owned=owned)
