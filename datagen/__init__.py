"""Seeded synthetic inputs for the DP-SGD step (shared by the tests, the bench and the oracle's
inputs).  The value recipe is in dg.h; this module only builds and calls the two fills.

This module holds none of the method's arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

from .configs import BF16, F32, ELEM_BYTES, Workload, workload, reduced  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libdpgen_host.so")
DEV_LIB = os.path.join(_HERE, "libdpgen_dev.so")

_host = None
_dev = None


def build(device: bool = True) -> None:
    """Compile the host fill with gcc and (device=True) the device fill with hipcc for gfx950."""
    subprocess.check_call(
        ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-o", HOST_LIB,
         os.path.join(_HERE, "dg_host.c")])
    if device:
        subprocess.check_call(
            ["hipcc", "--offload-arch=gfx950", "-O3", "-ffp-contract=off", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-o", DEV_LIB, os.path.join(_HERE, "dg_device.hip")],
            stderr=subprocess.DEVNULL)
    global _host, _dev
    _host = _dev = None


def _load_host():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            build(device=False)
        lib = ctypes.CDLL(HOST_LIB)
        lib.dg_fill_host.restype = ctypes.c_int
        lib.dg_fill_host.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                     ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]
        lib.dg_gather_host.restype = ctypes.c_int
        lib.dg_gather_host.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64] + [ctypes.c_void_p] * 6
        _host = lib
    return _host


def _load_dev():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"device generator not built: {DEV_LIB} (run __graft_entry__.build())")
        lib = ctypes.CDLL(DEV_LIB)
        lib.dg_fill_device.restype = ctypes.c_int
        lib.dg_fill_device.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _dev = lib
    return _dev


def _np_dtype(dtype: int):
    return np.float32 if dtype == F32 else np.uint16


def record_params(w: Workload, layer: int, tensor: int, first: int, n: int):
    scale = np.array([w.record_scale(layer, tensor, first + r) for r in range(n)], dtype=np.float64)
    heavy = np.array([w.record_heavy(first + r) for r in range(n)], dtype=np.uint8)
    return scale, heavy


def tensor_dim(w: Workload, layer: int, tensor: int) -> int:
    return w.layers[layer][0] if tensor == 0 else w.layers[layer][1]


def host_tensor(w: Workload, layer: int, tensor: int, first: int = 0,
                n: Optional[int] = None) -> np.ndarray:
    """Records [first, first+n) of A (tensor=0) or G (tensor=1) of `layer`, shape [n, T, d];
    float32 values, or uint16 bf16 bit patterns for bf16 workloads."""
    n = w.B if n is None else n
    d = tensor_dim(w, layer, tensor)
    out = np.empty((n, w.T, d), dtype=_np_dtype(w.dtype))
    scale, heavy = record_params(w, layer, tensor, first, n)
    rc = _load_host().dg_fill_host(w.data_seed, layer, tensor, w.dtype, first, n, w.T, d,
                                   scale.ctypes.data, heavy.ctypes.data, out.ctypes.data)
    if rc != 0:
        raise RuntimeError("dg_fill_host failed")
    return out


def gather(w: Workload, layer: int, tensor: int, rec, tok, col) -> np.ndarray:
    """Single input values (as float32) at the given (record, token, column) index arrays."""
    rec = np.ascontiguousarray(rec, dtype=np.int64)
    tok = np.ascontiguousarray(tok, dtype=np.int64)
    col = np.ascontiguousarray(col, dtype=np.int64)
    n = rec.size
    uniq, inv = np.unique(rec, return_inverse=True)
    scale = np.array([w.record_scale(layer, tensor, int(r)) for r in uniq], dtype=np.float64)[inv]
    heavy = np.array([w.record_heavy(int(r)) for r in uniq], dtype=np.uint8)[inv]
    out = np.empty(n, dtype=np.float32)
    d = tensor_dim(w, layer, tensor)
    rc = _load_host().dg_gather_host(w.data_seed, layer, tensor, w.dtype, w.T, d, n,
                                     rec.ctypes.data, tok.ctypes.data, col.ctypes.data,
                                     scale.ctypes.data, heavy.ctypes.data, out.ctypes.data)
    if rc != 0:
        raise RuntimeError("dg_gather_host failed")
    return out


def device_fill(w: Workload, layer: int, tensor: int, out_ptr: int, first: int, n: int,
                scale_dev_ptr: int, heavy_dev_ptr: int, stream_ptr: int) -> None:
    """Fill device memory at out_ptr with records [first, first+n) of (layer, tensor).  The
    per-record scale (float64) and heavy (uint8) arrays must already be in device memory."""
    d = tensor_dim(w, layer, tensor)
    rc = _load_dev().dg_fill_device(w.data_seed, layer, tensor, w.dtype, first, n, w.T, d,
                                    scale_dev_ptr, heavy_dev_ptr, out_ptr, stream_ptr)
    if rc != 0:
        raise RuntimeError(f"dg_fill_device failed ({rc})")


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << 16).view(np.float32)
