"""Python binding of libdpsgd.so, the C ABI of include/dpsgd.h (the DP-SGD private-gradient step:
ghost per-record norms, clipping, clipped sum, Gaussian noise) on one MI355X GPU.

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
PyTorch is used for device memory (tensor data pointers) and the current stream.  Importing this
package fails loudly if the library has not been built (see __graft_entry__.build()).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdpsgd.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_NONFINITE = -3
ERR_HIP = -4

DTYPE_F32 = 0
DTYPE_BF16 = 1

PATH_AUTO, PATH_GRAM, PATH_DIRECT = 0, 1, 2
SUM_AUTO, SUM_GEMM, SUM_STORED = 0, 1, 2

ACCUMULATE = 1
NO_NOISE = 2
DESCENT = 4

PLAN_SEGMENTS = 1

EXPORTS = ("dpsgd_plan_create", "dpsgd_plan_destroy", "dpsgd_plan_layer_info",
           "dpsgd_plan_num_params", "dpsgd_ws_init", "dpsgd_ws_segments", "dpsgd_norms", "dpsgd_clip",
           "dpsgd_clipped_sum", "dpsgd_noise", "dpsgd_noise_descent", "dpsgd_step", "dpsgd_step_noalloc",
           "dpsgd_status",
           "dpsgd_layer_norm2",
           "dpsgd_philox_raw", "dpsgd_hbm_read", "dpsgd_poisson_ws_bytes", "dpsgd_poisson_sample",
           "dpsgd_rdp_sampled_gaussian", "dpsgd_rdp_to_epsilon", "dpsgd_gaussian_pair_delta",
           "dpsgd_gaussian_pair_epsilon", "dpsgd_i8_pitch", "dpsgd_i8_plan_create",
           "dpsgd_i8_plan_destroy", "dpsgd_i8_quantize_weight", "dpsgd_i8_set_records",
           "dpsgd_i8_forward", "dpsgd_i8_route", "dpsgd_i8_matmul", "dpsgd_i8_intermediates", "dpsgd_error_string", "dpsgd_last_error")


class DpsgdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (code {code})")
        self.code = code


class LayerShape(ctypes.Structure):
    _fields_ = [("d_in", ctypes.c_int64), ("d_out", ctypes.c_int64)]


class PlanDesc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("layers", ctypes.POINTER(LayerShape)),
                ("dtype", ctypes.c_int32), ("max_records", ctypes.c_int64),
                ("tokens", ctypes.c_int64), ("path_policy", ctypes.c_int32),
                ("sum_policy", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class StepArgs(ctypes.Structure):
    _fields_ = [("n_records", ctypes.c_int64), ("A", ctypes.POINTER(ctypes.c_void_p)),
                ("G", ctypes.POINTER(ctypes.c_void_p)), ("out", ctypes.POINTER(ctypes.c_void_p)),
                ("ws", ctypes.c_void_p), ("C", ctypes.c_double), ("sigma", ctypes.c_double),
                ("seed", ctypes.c_uint64), ("step", ctypes.c_uint64), ("flags", ctypes.c_uint32),
                ("norms_out", ctypes.c_void_p), ("clip_out", ctypes.c_void_p),
                ("params", ctypes.POINTER(ctypes.c_void_p)), ("lr", ctypes.c_double),
                ("normalizer", ctypes.c_double)]


_lib = None


def load():
    """Load libdpsgd.so (raises if it is missing: there is no fallback implementation)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, U32, U64, D = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                ctypes.c_uint64, ctypes.c_double)
    PP = ctypes.POINTER(ctypes.c_void_p)
    PD = ctypes.POINTER(ctypes.c_double)
    sigs = {
        "dpsgd_plan_create": (ctypes.c_int, [ctypes.POINTER(PlanDesc), ctypes.POINTER(P),
                                             ctypes.POINTER(ctypes.c_size_t)]),
        "dpsgd_plan_destroy": (None, [P]),
        "dpsgd_plan_layer_info": (ctypes.c_int, [P, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "dpsgd_plan_num_params": (I64, [P]),
        "dpsgd_ws_init": (ctypes.c_int, [P, P, P]),
        "dpsgd_ws_segments": (ctypes.c_int, [P, P, ctypes.POINTER(I64), I64, P]),
        "dpsgd_norms": (ctypes.c_int, [P, I64, I32, I32, PP, PP, P, P]),
        "dpsgd_clip": (ctypes.c_int, [P, I64, D, U32, P, P, P, P]),
        "dpsgd_clipped_sum": (ctypes.c_int, [P, I64, I32, I32, PP, PP, P, PP, U32, P, P]),
        "dpsgd_noise": (ctypes.c_int, [P, PP, D, D, U64, U64, P, P]),
        "dpsgd_noise_descent": (ctypes.c_int, [P, PP, PP, D, D, U64, U64, D, D, P, P]),
        "dpsgd_step": (ctypes.c_int, [P, ctypes.POINTER(StepArgs), P]),
        "dpsgd_step_noalloc": (ctypes.c_int, [P, ctypes.POINTER(StepArgs), P, P]),
        "dpsgd_status": (ctypes.c_int, [P, P, P]),
        "dpsgd_layer_norm2": (ctypes.c_int, [P, I64, I32, I32, P, P, P]),
        "dpsgd_philox_raw": (ctypes.c_int, [U64, U64, U64, U64, P, P]),
        "dpsgd_hbm_read": (ctypes.c_int, [P, ctypes.c_int64, P, P]),
        "dpsgd_poisson_ws_bytes": (I64, [I64]),
        "dpsgd_poisson_sample": (ctypes.c_int, [U64, U64, D, I64, P, P, P, P, P]),
        "dpsgd_rdp_sampled_gaussian": (ctypes.c_int, [D, D, PD, I32, PD]),
        "dpsgd_rdp_to_epsilon": (ctypes.c_int, [PD, PD, I32, D, I32, PD, PD]),
        "dpsgd_gaussian_pair_delta": (ctypes.c_int, [D, D, PD]),
        "dpsgd_gaussian_pair_epsilon": (ctypes.c_int, [D, D, PD]),
        "dpsgd_i8_pitch": (I64, [I64]),
        "dpsgd_i8_plan_create": (ctypes.c_int, [I64, I64, I64, ctypes.POINTER(P),
                                                ctypes.POINTER(ctypes.c_size_t)]),
        "dpsgd_i8_plan_destroy": (None, [P]),
        "dpsgd_i8_quantize_weight": (ctypes.c_int, [P, I64, I64, P, P, P]),
        "dpsgd_i8_set_records": (ctypes.c_int, [P, P, ctypes.POINTER(I64), I64, P]),
        "dpsgd_i8_forward": (ctypes.c_int, [P, P, I64, I64, P, I64, P, P, I64, ctypes.c_float, P, P]),
        "dpsgd_i8_route": (ctypes.c_int, [P, P, I64, I64, P, I64, ctypes.c_float, P]),
        "dpsgd_i8_matmul": (ctypes.c_int, [P, P, I64, I64, P, I64, P, P, I64, P, P]),
        "dpsgd_i8_intermediates": (ctypes.c_int, [P, P, I64, I64, I64, P, P, P, P, P]),
        "dpsgd_error_string": (ctypes.c_char_p, [ctypes.c_int]),
        "dpsgd_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(rc: int) -> int:
    if rc != OK:
        lib = load()
        raise DpsgdError(rc, f"{lib.dpsgd_error_string(rc).decode()}: "
                             f"{lib.dpsgd_last_error().decode()}")
    return rc


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _ptr_array(xs) -> Optional[ctypes.Array]:
    if xs is None:
        return None
    return (ctypes.c_void_p * max(1, len(xs)))(*[_ptr(x) for x in xs])


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """Host plan of dpsgd_plan_create: layer shapes, dtype, record capacity, tokens per record
    (with segments=True: records are variable-length segments of at most `tokens` rows whose
    offsets are set per workspace by ws_segments)."""

    def __init__(self, layers: Sequence[tuple], dtype: int, max_records: int, tokens: int,
                 path_policy: int = PATH_AUTO, sum_policy: int = SUM_AUTO, segments: bool = False):
        lib = load()
        self._layers = (LayerShape * len(layers))(*[LayerShape(int(a), int(b)) for a, b in layers]) \
            if len(layers) else None
        desc = PlanDesc(len(layers), self._layers, dtype, max_records, tokens, path_policy,
                        sum_policy, PLAN_SEGMENTS if segments else 0)
        h = ctypes.c_void_p()
        ws = ctypes.c_size_t()
        _check(lib.dpsgd_plan_create(ctypes.byref(desc), ctypes.byref(h), ctypes.byref(ws)))
        self.handle = h
        self.ws_bytes = ws.value
        self.layers = [tuple(x) for x in layers]
        self.dtype = dtype
        self.max_records = max_records
        self.tokens = tokens
        self.n_params = lib.dpsgd_plan_num_params(h)

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.dpsgd_plan_destroy(self.handle)
            self.handle = None

    def layer_info(self, layer: int):
        p, s = ctypes.c_int32(), ctypes.c_int32()
        _check(load().dpsgd_plan_layer_info(self.handle, layer, ctypes.byref(p), ctypes.byref(s)))
        return p.value, s.value

    def workspace(self, device="cuda"):
        import torch
        return torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)


def ws_segments(plan: Plan, ws, offsets, stream=None):
    """dpsgd_ws_segments: record r owns token rows [offsets[r], offsets[r + 1])."""
    arr = (ctypes.c_int64 * len(offsets))(*[int(v) for v in offsets])
    _check(load().dpsgd_ws_segments(plan.handle, _ptr(ws), arr, len(offsets) - 1, _stream(stream)))


def ws_init(plan: Plan, ws, stream=None):
    _check(load().dpsgd_ws_init(plan.handle, _ptr(ws), _stream(stream)))


def norms(plan: Plan, n_records: int, l0: int, l1: int, A, G, ws, stream=None):
    _check(load().dpsgd_norms(plan.handle, n_records, l0, l1, _ptr_array(A), _ptr_array(G),
                              _ptr(ws), _stream(stream)))


def clip(plan: Plan, n_records: int, C: float, ws, flags: int = 0, norms_out=None, clip_out=None,
         stream=None):
    _check(load().dpsgd_clip(plan.handle, n_records, C, flags, _ptr(ws), _ptr(norms_out),
                             _ptr(clip_out), _stream(stream)))


def clipped_sum(plan: Plan, n_records: int, l0: int, l1: int, A, G, clip_factors, out, ws,
                flags: int = 0, stream=None):
    _check(load().dpsgd_clipped_sum(plan.handle, n_records, l0, l1, _ptr_array(A), _ptr_array(G),
                                    _ptr(clip_factors), _ptr_array(out), flags, _ptr(ws),
                                    _stream(stream)))


def noise(plan: Plan, out, C: float, sigma: float, seed: int, step: int, ws=None, stream=None,
          params=None, lr: float = 0.0, normalizer: float = 1.0):
    """dpsgd_noise, or dpsgd_noise_descent when `params` (one fp32 buffer per layer) is given."""
    if params is None:
        _check(load().dpsgd_noise(plan.handle, _ptr_array(out), C, sigma, seed, step, _ptr(ws),
                                  _stream(stream)))
    else:
        _check(load().dpsgd_noise_descent(plan.handle, _ptr_array(out), _ptr_array(params), C,
                                          sigma, seed, step, lr, normalizer, _ptr(ws),
                                          _stream(stream)))


def step(plan: Plan, A, G, out, ws, C: float, sigma: float, seed: int, step_idx: int,
         n_records: Optional[int] = None, flags: int = 0, norms_out=None, clip_out=None,
         stream=None, params=None, lr: float = 0.0, normalizer: float = 1.0):
    """dpsgd_step; with `params` (one fp32 buffer per layer) the descent step is added
    (DESCENT flag set)."""
    n = plan.max_records if n_records is None else n_records
    a_arr, g_arr, o_arr = _ptr_array(A), _ptr_array(G), _ptr_array(out)
    p_arr = _ptr_array(params)
    if params is not None:
        flags |= DESCENT
    args = StepArgs(n, a_arr, g_arr, o_arr, _ptr(ws), C, sigma, seed, step_idx, flags,
                    _ptr(norms_out), _ptr(clip_out), p_arr, lr, normalizer)
    _check(load().dpsgd_step(plan.handle, ctypes.byref(args), _stream(stream)))


def step_noalloc(plan: Plan, A, G, out, C: float, sigma: float, seed: int, step_idx: int,
                 n_records: Optional[int] = None, flags: int = 0, norms_out=None, clip_out=None,
                 status_out=None, stream=None, params=None, lr: float = 0.0,
                 normalizer: float = 1.0):
    """dpsgd_step_noalloc: dpsgd_step on the library's per-device scratch (no workspace
    argument, no allocation); status_out: optional device uint32 receiving the status word."""
    n = plan.max_records if n_records is None else n_records
    a_arr, g_arr, o_arr = _ptr_array(A), _ptr_array(G), _ptr_array(out)
    p_arr = _ptr_array(params)
    if params is not None:
        flags |= DESCENT
    args = StepArgs(n, a_arr, g_arr, o_arr, None, C, sigma, seed, step_idx, flags,
                    _ptr(norms_out), _ptr(clip_out), p_arr, lr, normalizer)
    _check(load().dpsgd_step_noalloc(plan.handle, ctypes.byref(args), _ptr(status_out),
                                     _stream(stream)))


class StepCall:
    """A dpsgd_step call with its argument block marshalled once (for training loops that call
    the step repeatedly on the same buffers).  step_idx may be changed per call."""

    def __init__(self, plan: Plan, A, G, out, ws, C: float, sigma: float, seed: int,
                 step_idx: int = 0, n_records: Optional[int] = None, flags: int = 0,
                 norms_out=None, clip_out=None, stream=None, params=None, lr: float = 0.0,
                 normalizer: float = 1.0):
        self.plan = plan
        self._keep = (_ptr_array(A), _ptr_array(G), _ptr_array(out), _ptr_array(params))
        n = plan.max_records if n_records is None else n_records
        if params is not None:
            flags |= DESCENT
        self.args = StepArgs(n, self._keep[0], self._keep[1], self._keep[2], _ptr(ws), C, sigma,
                             seed, step_idx, flags, _ptr(norms_out), _ptr(clip_out),
                             self._keep[3], lr, normalizer)
        self.stream = _stream(stream)
        self._fn = load().dpsgd_step
        self._ref = ctypes.byref(self.args)

    def __call__(self, step_idx: Optional[int] = None):
        if step_idx is not None:
            self.args.step = step_idx
        rc = self._fn(self.plan.handle, self._ref, self.stream)
        if rc:
            _check(rc)


def status(plan: Plan, ws, stream=None) -> int:
    """Synchronise the stream and return OK or ERR_NONFINITE."""
    rc = load().dpsgd_status(plan.handle, _ptr(ws), _stream(stream))
    if rc not in (OK, ERR_NONFINITE):
        _check(rc)
    return rc


def layer_norm2(plan: Plan, n_records: int, l0: int, l1: int, ws, out, stream=None):
    _check(load().dpsgd_layer_norm2(plan.handle, n_records, l0, l1, _ptr(ws), _ptr(out),
                                    _stream(stream)))


HBM_READ_SINK_WORDS = 8192


def hbm_read(buf, nbytes: int, sink, stream=None):
    """dpsgd_hbm_read: streaming read of nbytes of buf; sink holds HBM_READ_SINK_WORDS uint32."""
    _check(load().dpsgd_hbm_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)))


def philox_raw(seed: int, step: int, first_block: int, n_blocks: int, out, stream=None):
    _check(load().dpsgd_philox_raw(seed, step, first_block, n_blocks, _ptr(out), _stream(stream)))


# ---------------------------------------------------------------- Poisson sampling

def poisson_ws_bytes(population: int) -> int:
    return load().dpsgd_poisson_ws_bytes(population)


def poisson_sample(seed: int, step: int, q: float, population: int, indices, count, ws, mask=None,
                   stream=None):
    """dpsgd_poisson_sample: the included records' indices (increasing) into `indices`, their
    number into `count` (device int64), the 0/1 inclusion bytes into `mask` if given."""
    _check(load().dpsgd_poisson_sample(seed, step, q, population, _ptr(mask), _ptr(indices),
                                       _ptr(count), _ptr(ws), _stream(stream)))


# ---------------------------------------------------------------- privacy accounting (host)

def _doubles(xs):
    return (ctypes.c_double * len(xs))(*[float(x) for x in xs])


def rdp_sampled_gaussian(q: float, sigma: float, orders) -> list:
    """Per-step RDP of the Poisson-subsampled Gaussian mechanism at each order."""
    o = _doubles(orders)
    out = (ctypes.c_double * len(orders))()
    _check(load().dpsgd_rdp_sampled_gaussian(q, sigma, o, len(orders), out))
    return list(out)


def rdp_to_epsilon(orders, rdp, delta: float, tight: bool = True):
    """(epsilon, minimising order) at delta from RDP values at `orders`."""
    e, a = ctypes.c_double(), ctypes.c_double()
    _check(load().dpsgd_rdp_to_epsilon(_doubles(orders), _doubles(rdp), len(orders), delta,
                                       1 if tight else 0, ctypes.byref(e), ctypes.byref(a)))
    return e.value, a.value


def gaussian_pair_delta(eps: float, mu: float) -> float:
    d = ctypes.c_double()
    _check(load().dpsgd_gaussian_pair_delta(eps, mu, ctypes.byref(d)))
    return d.value


def gaussian_pair_epsilon(delta: float, mu: float) -> float:
    e = ctypes.c_double()
    _check(load().dpsgd_gaussian_pair_epsilon(delta, mu, ctypes.byref(e)))
    return e.value


# ---------------------------------------------------------------- record-owned INT8 forward

def i8_pitch(k: int) -> int:
    """Bytes per INT8 code row (k rounded up to 64; 0 for k outside [1, 32768])."""
    return load().dpsgd_i8_pitch(k)


class I8Plan:
    """Host plan of dpsgd_i8_plan_create: capacities of the INT8 forward's workspace."""

    def __init__(self, max_rows: int, max_records: int, max_k: int):
        lib = load()
        h = ctypes.c_void_p()
        ws = ctypes.c_size_t()
        _check(lib.dpsgd_i8_plan_create(max_rows, max_records, max_k, ctypes.byref(h),
                                        ctypes.byref(ws)))
        self.handle = h
        self.ws_bytes = ws.value
        self.max_rows, self.max_records, self.max_k = max_rows, max_records, max_k

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.dpsgd_i8_plan_destroy(self.handle)
            self.handle = None

    def workspace(self, device="cuda"):
        import torch
        return torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)


def i8_quantize_weight(W, n_out: int, k: int, wq, w_scale, stream=None):
    """dpsgd_i8_quantize_weight: W fp16 [n_out, k] -> wq int8 [n_out, pitch(k)], w_scale fp32."""
    _check(load().dpsgd_i8_quantize_weight(_ptr(W), n_out, k, _ptr(wq), _ptr(w_scale),
                                           _stream(stream)))


def i8_set_records(plan: I8Plan, ws, offsets, stream=None):
    """dpsgd_i8_set_records: record r owns activation rows [offsets[r], offsets[r + 1])."""
    arr = (ctypes.c_int64 * len(offsets))(*[int(v) for v in offsets])
    _check(load().dpsgd_i8_set_records(plan.handle, _ptr(ws), arr, len(offsets) - 1,
                                       _stream(stream)))


def i8_forward(plan: I8Plan, ws, n_rows: int, n_records: int, A, k: int, wq, w_scale, n_out: int,
               tau: float, Y, stream=None):
    """dpsgd_i8_forward: Y [n_rows, n_out] fp16 = record-owned LLM.int8 forward of A."""
    _check(load().dpsgd_i8_forward(plan.handle, _ptr(ws), n_rows, n_records, _ptr(A), k,
                                   _ptr(wq), _ptr(w_scale), n_out, tau, _ptr(Y), _stream(stream)))


def i8_route(plan: I8Plan, ws, n_rows: int, n_records: int, A, k: int, tau: float, stream=None):
    """dpsgd_i8_route: Algorithm 1's steps 1-6 into the workspace."""
    _check(load().dpsgd_i8_route(plan.handle, _ptr(ws), n_rows, n_records, _ptr(A), k, tau,
                                 _stream(stream)))


def i8_matmul(plan: I8Plan, ws, n_rows: int, n_records: int, A, k: int, wq, w_scale, n_out: int, Y,
              stream=None):
    """dpsgd_i8_matmul: step 7 after a dpsgd_i8_route of the same activations."""
    _check(load().dpsgd_i8_matmul(plan.handle, _ptr(ws), n_rows, n_records, _ptr(A), k, _ptr(wq),
                                  _ptr(w_scale), n_out, _ptr(Y), _stream(stream)))


def i8_intermediates(plan: I8Plan, ws, n_rows: int, n_records: int, k: int, q=None,
                     row_scale=None, outlier_mask=None, owner=None, stream=None):
    _check(load().dpsgd_i8_intermediates(plan.handle, _ptr(ws), n_rows, n_records, k, _ptr(q),
                                         _ptr(row_scale), _ptr(outlier_mask), _ptr(owner),
                                         _stream(stream)))
