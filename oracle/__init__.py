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
output named in §"与官方 FA2 比较时，先对齐契约". The features that
§"哪些结论可以迁移，哪些只是本例特例" lists for a production kernel (local
masks, variable-length sequences, dropout, GQA/MQA) follow the readings stated
at the top of ``attn_oracle.c``: ``attention_ex`` and ``attention_varlen`` only
choose which rows form one (sequence, head) problem, and the C code evaluates
each problem.
"""
from __future__ import annotations

import ctypes
import math
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
    u32, ll_p = ctypes.c_uint32, ctypes.POINTER(ctypes.c_longlong)
    lib.attn_oracle_head_f64.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_double, ctypes.c_int, u32, u32, u32, u32, u32,
                                         ctypes.c_double, ll_p, ctypes.c_int, dp, dp, ctypes.c_int]
    lib.attn_oracle_head_f64.restype = ctypes.c_int
    lib.attn_oracle_philox4x32_10.argtypes = [ctypes.POINTER(u32), ctypes.POINTER(u32), ctypes.POINTER(u32)]
    lib.attn_oracle_philox4x32_10.restype = None
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


def philox4x32_10(counter, key, lib=None):
    """The four 32-bit output words of Philox4x32-10 for a 4-word counter and a
    2-word key (Salmon et al., SC 2011)."""
    lib = lib or load()
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in counter])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    out = (ctypes.c_uint32 * 4)()
    lib.attn_oracle_philox4x32_10(c, k, out)
    return [int(x) for x in out]


def dropout_threshold(p: float) -> int:
    """floor(p * 2^16), clamped to 2^16 - 1: a 16-bit draw >= it keeps the weight."""
    if not p > 0.0:
        return 0
    return min(int(math.floor(float(p) * 65536.0)), 0xFFFF)


def _head(lib, q2, k2, v2, scale, window, dropout_p, seed, offset, bh, rows, nthreads):
    """One (sequence, head) problem: q2 [S, D] against k2, v2 [S, D]."""
    S, D = q2.shape
    wl, wr = int(window[0]), int(window[1])
    drop = dropout_p > 0.0
    keep_scale = 1.0 / (1.0 - float(dropout_p)) if drop else 1.0
    if rows is None:
        n, rows_ptr = S, None
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n, rows_ptr = int(rows.size), rows.ctypes.data_as(ctypes.POINTER(ctypes.c_longlong))
    O = np.empty((n, D), dtype=np.float64)
    LSE = np.empty((n,), dtype=np.float64)
    rc = lib.attn_oracle_head_f64(_ptr(q2), _ptr(k2), _ptr(v2), S, D, wl, wr, float(scale), int(drop),
                                  dropout_threshold(dropout_p) if drop else 0, int(seed) & 0xFFFFFFFF,
                                  (int(seed) >> 32) & 0xFFFFFFFF, int(bh) & 0xFFFFFFFF,
                                  int(offset) & 0xFFFFFFFF, keep_scale, rows_ptr, n, _ptr(O), _ptr(LSE),
                                  int(nthreads))
    if rc != 0:
        raise RuntimeError(f"attn_oracle_head_f64 failed with code {rc}")
    return O, LSE


def attention_ex(q, k, v, scale: float, window=(-1, -1), dropout_p: float = 0.0, seed: int = 0,
                 offset: int = 0, rows=None, nthreads: int = 0, lib=None):
    """Dense [B,H,S,D] queries against [B,H_kv,S,D] keys/values (query head h
    reads K/V head h // (H // H_kv)), a local window (left, right) with -1 for
    an unbounded side, and dropout. Returns O [B,H,S,D] and LSE [B,H,S] in
    float64, or, with ``rows`` (flat (b*H+h)*S+i indices), O [n,D] and LSE [n].
    ``dropout_p`` and ``scale`` are used as given; pass float32-rounded values
    to match a float32 kernel argument."""
    lib = lib or load()
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:]:
        raise ValueError(f"q must be [B,H,S,D] and k, v [B,H_kv,S,D], got {q.shape} {k.shape} {v.shape}")
    B, H, S, D = q.shape
    H_kv = k.shape[1]
    if H % H_kv:
        raise ValueError("H must be a multiple of H_kv")
    group = H // H_kv
    if rows is None:
        O = np.empty((B, H, S, D))
        LSE = np.empty((B, H, S))
        for b in range(B):
            for h in range(H):
                O[b, h], LSE[b, h] = _head(lib, np.ascontiguousarray(q[b, h]), np.ascontiguousarray(k[b, h // group]),
                                           np.ascontiguousarray(v[b, h // group]), scale, window, dropout_p, seed,
                                           offset, b * H + h, None, nthreads)
        return O, LSE
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= B * H * S):
        raise RuntimeError("row index out of range")
    O = np.empty((rows.size, D))
    LSE = np.empty((rows.size,))
    heads = rows // S
    for bh in np.unique(heads):
        sel = np.nonzero(heads == bh)[0]
        b, h = divmod(int(bh), H)
        O[sel], LSE[sel] = _head(lib, np.ascontiguousarray(q[b, h]), np.ascontiguousarray(k[b, h // group]),
                                 np.ascontiguousarray(v[b, h // group]), scale, window, dropout_p, seed, offset,
                                 int(bh), rows[sel] % S, nthreads)
    return O, LSE


def attention_varlen(q, k, v, cu_seqlens, scale: float, window=(-1, -1), dropout_p: float = 0.0, seed: int = 0,
                     offset: int = 0, nthreads: int = 0, lib=None):
    """Packed sequences: q [total,H,D], k, v [total,H_kv,D]; sequence s is rows
    cu_seqlens[s] .. cu_seqlens[s+1]-1 and attends only within itself, with
    row indices counted from its start. Returns O [total,H,D] and LSE [H,total]
    in float64 (rows of empty sequences do not exist)."""
    lib = lib or load()
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    cu = [int(x) for x in np.asarray(cu_seqlens).tolist()]
    if q.ndim != 3 or k.ndim != 3 or k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2]:
        raise ValueError(f"q must be [total,H,D] and k, v [total,H_kv,D], got {q.shape} {k.shape} {v.shape}")
    total, H, D = q.shape
    H_kv = k.shape[1]
    if H % H_kv:
        raise ValueError("H must be a multiple of H_kv")
    if len(cu) < 2 or cu[0] != 0 or cu[-1] != total or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at total")
    group = H // H_kv
    O = np.full((total, H, D), np.nan)
    LSE = np.full((H, total), np.nan)
    for s_idx, (a, e) in enumerate(zip(cu, cu[1:])):
        if e == a:
            continue
        for h in range(H):
            O[a:e, h], LSE[h, a:e] = _head(lib, np.ascontiguousarray(q[a:e, h]),
                                           np.ascontiguousarray(k[a:e, h // group]),
                                           np.ascontiguousarray(v[a:e, h // group]), scale, window, dropout_p,
                                           seed, offset, s_idx * H + h, None, nthreads)
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
