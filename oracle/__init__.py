"""Test infrastructure only: the fp64 CPU oracle for attention.

Only ``tests/``, the smoke check and the CPU-baseline leg of ``bench.py`` may
import this package. It shares no code with the HIP library and never imports
it. The arithmetic lives in ``attn_oracle.c`` (plain C, double precision, one
explicit score row at a time); this module only compiles it with gcc, loads it
with ctypes and converts the fp16 inputs to double exactly.

Definition followed: the page "CuTe 详解：以 FlashAttention-2 拆解 Layout、
TiledCopy 与 TiledMMA", §"先看全局：FA2 中的数据究竟去了哪里" (S = Q Kᵀ,
P = softmax(S), O = P V) and §"教学配置：一块 CTA 做什么" (O_i = õ_i / ℓ_i), with
the softmax scale of §"沿 C fragment 做 Online Softmax" and the log-sum-exp
output named in §"与官方 FA2 比较时，先对齐契约".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "libattn_oracle.so")
_CFLAGS = ["-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99", "-Wall", "-Wextra"]

_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (IEEE double arithmetic: no -ffast-math)."""
    cmd = ["gcc", *_CFLAGS, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the compiled oracle; compile it first if it is missing or stale."""
    global _lib
    if path is None:
        if _lib is not None:
            return _lib
        if (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        path = _LIB
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.attn_oracle_f64.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_double, dp, dp,
                                    ctypes.c_int]
    lib.attn_oracle_f64.restype = ctypes.c_int
    lib.attn_oracle_rows_f64.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                         ctypes.POINTER(ctypes.c_longlong), ctypes.c_int, dp, dp,
                                         ctypes.c_int]
    lib.attn_oracle_rows_f64.restype = ctypes.c_int
    lib.attn_oracle_max_threads.argtypes = []
    lib.attn_oracle_max_threads.restype = ctypes.c_int
    if path == _LIB:
        _lib = lib
    return lib


def _as_f64(x) -> np.ndarray:
    # fp16 -> fp64 widening is exact; the oracle sees the very values the GPU reads.
    return np.ascontiguousarray(np.asarray(x), dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _check_shapes(q, k, v):
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v must be equal [B,H,S,D] arrays, got {q.shape} {k.shape} {v.shape}")


def attention(q, k, v, causal: bool, scale: float, nthreads: int = 0, lib=None):
    """O [B,H,S,D] and LSE [B,H,S] in float64 for [B,H,S,D] inputs.

    ``scale`` is used as given (a Python float is a double); callers that
    compare with a float32 kernel argument pass float(np.float32(scale)).
    """
    lib = lib or load()
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    _check_shapes(q, k, v)
    B, H, S, D = q.shape
    O = np.empty((B, H, S, D), dtype=np.float64)
    LSE = np.empty((B, H, S), dtype=np.float64)
    rc = lib.attn_oracle_f64(_ptr(q), _ptr(k), _ptr(v), B, H, S, D, int(bool(causal)),
                             float(scale), _ptr(O), _ptr(LSE), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"attn_oracle_f64 failed with code {rc}")
    return O, LSE


def attention_rows(q, k, v, causal: bool, scale: float, rows, nthreads: int = 0, lib=None):
    """The same definition for selected rows. ``rows`` are flat (b*H+h)*S+i
    indices; returns O [n, D] and LSE [n] in float64."""
    lib = lib or load()
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    _check_shapes(q, k, v)
    B, H, S, D = q.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = int(rows.size)
    O = np.empty((n, D), dtype=np.float64)
    LSE = np.empty((n,), dtype=np.float64)
    rc = lib.attn_oracle_rows_f64(_ptr(q), _ptr(k), _ptr(v), B, H, S, D, int(bool(causal)),
                                  float(scale),
                                  rows.ctypes.data_as(ctypes.POINTER(ctypes.c_longlong)), n,
                                  _ptr(O), _ptr(LSE), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"attn_oracle_rows_f64 failed with code {rc}")
    return O, LSE


def max_threads(lib=None) -> int:
    return int((lib or load()).attn_oracle_max_threads())


def timed_rows(q, k, v, causal: bool, scale: float, rows, nthreads: int = 0):
    """attention_rows plus its wall time in seconds (for the CPU baseline)."""
    lib = load()
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)  # widen outside the timed region
    t0 = time.perf_counter()
    O, LSE = attention_rows(q, k, v, causal, scale, rows, nthreads=nthreads, lib=lib)
    return O, LSE, time.perf_counter() - t0
