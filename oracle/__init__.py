"""CPU oracle of the DP-SGD private-gradient step (double precision).

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg
may import this package.  The product library never calls it, and it shares no code with the
GPU path.  The arithmetic lives in dpsgd_oracle.c; this module builds it and marshals numpy
arrays.  Every function states the definition it follows.

Pinned (see tests/test_oracle_pins.py): the clip formula and the worked clipping example of
"Privacy-Preserving Machine Learning"; the constructed witness of "Sensitivity Inflation from
Cross-Record Precision Routing in Private Quantized Fine-Tuning" App. A; the rank-one closed
form; integer brute force and the Gram identity; the no-clip case against a library GEMM;
the gradient convention against autograd; the sensitivity bounds; Philox4x32-10 against
rocRAND's implementation; the Gaussian moments and norm against the sigma*C*sqrt(d) RMS.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "liboracle.so")
F32, BF16, F64 = 0, 1, 2
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
_D = ctypes.c_double


def build() -> None:
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", LIB,
                           os.path.join(_HERE, "dpsgd_oracle.c"), "-lm"])
    global _lib
    _lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        sig = {
            "orc_record_grad": (None, [ctypes.c_int, _P, _P, _I64, _I64, _I64, _P]),
            "orc_layer_norm2": (ctypes.c_int, [ctypes.c_int, _P, _P, _I64, _I64, _I64, _I64, _P]),
            "orc_clip_factor": (_D, [_D, _D]),
            "orc_clip": (None, [_P, _I64, _D, _P, _P]),
            "orc_layer_clipped_sum": (ctypes.c_int,
                                      [ctypes.c_int, _P, _P, _I64, _I64, _I64, _I64, _P, _P]),
            "orc_philox4x32_10": (None, [_P, _P, _P]),
            "orc_philox_words": (None, [_U64, _U64, _U64, _U64, _P]),
            "orc_gauss": (None, [_U64, _U64, _U64, _I64, _P]),
            "orc_add_noise": (None, [_P, _I64, _U64, _D, _D, _U64, _U64]),
            "orc_num_threads": (ctypes.c_int, []),
            "orc_set_num_threads": (None, [ctypes.c_int]),
        }
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return _load().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads for the oracle's later OpenMP loops."""
    _load().orc_set_num_threads(n)


def _dtype_of(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    if x.dtype == np.float64:
        return F64
    raise TypeError(f"oracle inputs are float32, uint16 bf16 bit patterns or float64, got {x.dtype}")


def _c(x, dt):
    return np.ascontiguousarray(x, dtype=dt)


def record_grad(A_i: np.ndarray, G_i: np.ndarray) -> np.ndarray:
    """Per-record gradient P = A_i^T G_i, [d_in, d_out], for A_i [T, d_in], G_i [T, d_out]."""
    dt = _dtype_of(A_i)
    A_i = np.ascontiguousarray(A_i)
    G_i = np.ascontiguousarray(G_i)
    T, d_in = A_i.shape
    d_out = G_i.shape[1]
    P = np.empty((d_in, d_out), dtype=np.float64)
    _load().orc_record_grad(dt, A_i.ctypes.data, G_i.ctypes.data, T, d_in, d_out, P.ctypes.data)
    return P


def layer_norm2(A: np.ndarray, G: np.ndarray) -> np.ndarray:
    """Squared Frobenius norms of the per-record gradients of one layer (A [B,T,d_in],
    G [B,T,d_out]); each record's gradient is materialised first."""
    dt = _dtype_of(A)
    A = np.ascontiguousarray(A)
    G = np.ascontiguousarray(G)
    B, T, d_in = A.shape
    d_out = G.shape[2]
    out = np.zeros(B, dtype=np.float64)
    if B:
        rc = _load().orc_layer_norm2(dt, A.ctypes.data, G.ctypes.data, B, T, d_in, d_out,
                                     out.ctypes.data)
        assert rc == 0
    return out


def clip(norm2_total: np.ndarray, C: float):
    """(n, c): n_i = sqrt of the joint squared norm, c_i = 1 if n_i <= C else C / n_i."""
    norm2_total = _c(norm2_total, np.float64)
    B = norm2_total.size
    n = np.empty(B, dtype=np.float64)
    c = np.empty(B, dtype=np.float64)
    if B:
        _load().orc_clip(norm2_total.ctypes.data, B, float(C), n.ctypes.data, c.ctypes.data)
    return n, c


def clip_factor(norm2: float, C: float) -> float:
    return _load().orc_clip_factor(float(norm2), float(C))


def layer_clipped_sum(A: np.ndarray, G: np.ndarray, c: np.ndarray, S: np.ndarray = None):
    """S += sum_i c_i A_i^T G_i (records in ascending order), S [d_in, d_out] float64."""
    dt = _dtype_of(A)
    A = np.ascontiguousarray(A)
    G = np.ascontiguousarray(G)
    B, T, d_in = A.shape
    d_out = G.shape[2]
    if S is None:
        S = np.zeros((d_in, d_out), dtype=np.float64)
    assert S.dtype == np.float64 and S.flags.c_contiguous and S.size == d_in * d_out
    c = _c(c, np.float64)
    assert c.size >= B
    if B:
        rc = _load().orc_layer_clipped_sum(dt, A.ctypes.data, G.ctypes.data, B, T, d_in, d_out,
                                           c.ctypes.data, S.ctypes.data)
        assert rc == 0
    return S


def philox4x32_10(ctr, key) -> np.ndarray:
    ctr = _c(ctr, np.uint32)
    key = _c(key, np.uint32)
    out = np.empty(4, dtype=np.uint32)
    _load().orc_philox4x32_10(ctr.ctypes.data, key.ctypes.data, out.ctypes.data)
    return out


def philox_words(seed: int, step: int, first_block: int, n_blocks: int) -> np.ndarray:
    out = np.empty(4 * n_blocks, dtype=np.uint32)
    if n_blocks:
        _load().orc_philox_words(seed, step, first_block, n_blocks, out.ctypes.data)
    return out


def gauss(seed: int, step: int, first_e: int, n: int) -> np.ndarray:
    z = np.empty(n, dtype=np.float64)
    if n:
        _load().orc_gauss(seed, step, first_e, n, z.ctypes.data)
    return z


def add_noise(S_flat: np.ndarray, first_e: int, sigma: float, C: float, seed: int,
              step: int) -> np.ndarray:
    """In place: S_flat += sigma * C * Z[first_e : first_e + len]."""
    assert S_flat.dtype == np.float64 and S_flat.flags.c_contiguous
    if S_flat.size:
        _load().orc_add_noise(S_flat.ctypes.data, S_flat.size, first_e, float(sigma), float(C),
                              seed, step)
    return S_flat


def descent(theta, g_noised, lr: float, normalizer: float):
    """Phase 5 of the step ("Privacy-Preserving Machine Learning", section "Differentially
    private stochastic gradient descent", the descent step): the noised sum is divided by the
    fixed public normaliser L, scaled by the learning rate and subtracted from the parameters,
    theta' = theta - lr * (g_noised / L).  float64 in and out."""
    return np.asarray(theta, dtype=np.float64) - lr * (np.asarray(g_noised, dtype=np.float64) / normalizer)


def step(layers_A, layers_G, C: float, sigma: float, seed: int, step_idx: int,
         noise: bool = True, batches=None, descent_args=None):
    """Whole step for inputs given per layer (lists of [B,T,d] arrays).  `batches` optionally
    lists physical batches as (layers_A, layers_G) tuples for virtual batching: norms and clip
    factors are per physical batch (each record only ever sees its own data), the clipped sums
    accumulate across batches, and noise is drawn once.  `descent_args` = (thetas per layer, lr,
    L) adds the descent step on the noised sum (it is part of the release, so it needs the
    noise).  Returns dict with n, c (concatenated over batches in logical record order), S (list
    per layer, pre-noise), S_noised (list) and, with descent_args, theta (list)."""
    if batches is None:
        batches = [(layers_A, layers_G)]
    L = len(batches[0][0])
    shapes = [(batches[0][0][l].shape[2], batches[0][1][l].shape[2]) for l in range(L)]
    S = [np.zeros(s, dtype=np.float64) for s in shapes]
    ns, cs = [], []
    for As, Gs in batches:
        B = As[0].shape[0]
        norm2 = np.zeros(B, dtype=np.float64)
        for l in range(L):
            norm2 += layer_norm2(As[l], Gs[l])
        n, c = clip(norm2, C)
        ns.append(n)
        cs.append(c)
        for l in range(L):
            layer_clipped_sum(As[l], Gs[l], c, S[l])
    flat = np.concatenate([s.reshape(-1) for s in S]) if L else np.zeros(0)
    noised = flat.copy()
    if noise:
        add_noise(noised, 0, sigma, C, seed, step_idx)
    out, off = [], 0
    for s in shapes:
        out.append(noised[off:off + s[0] * s[1]].reshape(s))
        off += s[0] * s[1]
    res = {"n": np.concatenate(ns), "c": np.concatenate(cs), "S": S, "S_noised": out}
    if descent_args is not None:
        if not noise:
            raise ValueError("the descent step releases the noised sum: it needs the noise")
        thetas, lr, L = descent_args
        res["theta"] = [descent(t, o, lr, L) for t, o in zip(thetas, out)]
    return res
