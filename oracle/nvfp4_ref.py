"""ctypes front end of ``nvfp4_ref.c``: the oracle's NVFP4 quantizer and decoder in plain C.

TEST INFRASTRUCTURE ONLY (see ``nvfp4_oracle``): only ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg may import this module.

Same definition as ``nvfp4_oracle.quantize_nvfp4`` / ``dequantize_blocks`` (global scale
448*6/amax, E4M3 block scales and E2M1 codes by exact nearest-with-ties-to-even, the even element
in the low nibble), written element by element in C and run on row ranges in parallel threads, for
the full-size workloads where the NumPy form would take minutes.  The library is built by
``__graft_entry__.build()``; when it is missing or older than its source it is compiled here with
gcc (a test-time convenience: no product code depends on it).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "nvfp4_ref.c")
LIB = os.path.join(_HERE, "libnvfp4_ref.so")
GCC_FLAGS = ["-O2", "-std=c11", "-Wall", "-ffp-contract=off", "-fPIC", "-shared", "-pthread"]
_lib = None


def build(out: str = LIB) -> str:
    """Compile nvfp4_ref.c into ``out`` with gcc (no fast-math, no fp contraction)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *GCC_FLAGS, SRC, "-o", tmp, "-lm"], check=True, capture_output=True, text=True)
    os.replace(tmp, out)
    return out


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.nvfp4_ref_global_scale.argtypes = [ctypes.c_double]
        L.nvfp4_ref_global_scale.restype = ctypes.c_float
        L.nvfp4_ref_amax.argtypes = [p, i64, i64, p, i32]
        L.nvfp4_ref_amax.restype = ctypes.c_double
        L.nvfp4_ref_quantize.argtypes = [p, i64, i64, p, ctypes.c_float, p, p, i32]
        L.nvfp4_ref_quantize.restype = i32
        L.nvfp4_ref_dequantize.argtypes = [p, p, i64, i64, p, i32]
        L.nvfp4_ref_dequantize.restype = i32
        _lib = L
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def quantize_bits(bits: np.ndarray, valid_rows=None, gs=None, threads: Optional[int] = None):
    """NVFP4-quantize bf16 bit patterns ``bits`` (uint16 [rows, K]).

    ``gs`` None: the global scale comes from the amax of the valid rows (all rows when
    ``valid_rows`` is None); else it is the given float32 scale.  Invalid rows get zero codes and
    scales.  Returns (packed codes uint8 [rows, K/2], scale codes uint8 [rows, K/16], gs float32).
    """
    x = np.ascontiguousarray(bits, dtype=np.uint16)
    rows, K = x.shape
    th = threads or default_threads()
    valid = None if valid_rows is None else np.ascontiguousarray(valid_rows, dtype=np.uint8)
    if gs is None:
        gs = lib().nvfp4_ref_global_scale(lib().nvfp4_ref_amax(_ptr(x), rows, K, _ptr(valid), th))
    gs = np.float32(gs)
    codes = np.empty((rows, K // 2), np.uint8)
    scales = np.empty((rows, K // 16), np.uint8)
    rc = lib().nvfp4_ref_quantize(_ptr(x), rows, K, _ptr(valid), float(gs), _ptr(codes), _ptr(scales), th)
    if rc != 0:
        raise ValueError(f"nvfp4_ref_quantize: bad sizes {x.shape}")
    return codes, scales, gs


def dequantize(codes: np.ndarray, scales: np.ndarray, threads: Optional[int] = None) -> np.ndarray:
    """Exact float64 e2m1(code) * e4m3(scale) of every element ([rows, K])."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, K = c.shape[0], c.shape[1] * 2
    out = np.empty((rows, K), np.float64)
    rc = lib().nvfp4_ref_dequantize(_ptr(c), _ptr(s), rows, K, _ptr(out), threads or default_threads())
    if rc != 0:
        raise ValueError(f"nvfp4_ref_dequantize: bad sizes {c.shape}")
    return out
