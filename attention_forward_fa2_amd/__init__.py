"""MI355X-native FlashAttention-2 forward: Python binding of libfa2.so.

The binding only marshals arguments: every step of the forward pass runs in the
HIP kernels behind the C ABI of include/fa2.h. There is no CPU or PyTorch
fallback: if the library is missing, importing the binding's entry points
raises.

    fa2_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, S, D, causal, scale, stream)
        the C call itself (integers for pointers and the stream); returns the status.
    fa2_fwd_ex(q, k, v, o, lse, B, H, H_kv, S, D, window_left, window_right,
               dropout_p, seed, offset, scale, stream)
    fa2_fwd_varlen(q, k, v, o, lse, cu_seqlens, num_seqs, total, max_seqlen, H, H_kv, D,
                   window_left, window_right, dropout_p, seed, offset, scale, stream)
        the extended C calls (GQA/MQA, local window, dropout; packed sequences).
    fa2_strerror(status) -> str
    fa2_kernel_config(B, H, S, D, causal) -> dict
    forward(q, k, v, causal=False, scale=None, out=None, lse=None) -> (o, lse)
    forward_ex(q, k, v, causal=False, window=None, dropout_p=0.0, seed=0, offset=0, ...) -> (o, lse)
    forward_varlen(q, k, v, cu_seqlens, max_seqlen=None, causal=False, window=None, ...) -> (o, lse)
        torch conveniences: allocate outputs with torch, launch on the current stream.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa2.so")

FA2_OK = 0
STATUS_NAMES = {
    0: "FA2_OK", 1: "FA2_ERR_NULLPTR", 2: "FA2_ERR_SHAPE", 3: "FA2_ERR_SCALE", 4: "FA2_ERR_ALIGN",
    5: "FA2_ERR_OVERFLOW", 6: "FA2_ERR_DEVICE", 7: "FA2_ERR_LAUNCH", 8: "FA2_ERR_ALIAS",
    9: "FA2_ERR_ARG",
}
EXPORTED = ("fa2_fwd", "fa2_fwd_ex", "fa2_fwd_varlen", "fa2_strerror", "fa2_kernel_config")

_lib = None


class FA2Error(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {fa2_strerror(status)}")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa2.so. Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing; build it with `python -m attention_forward_fa2_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.fa2_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, ctypes.c_float, vp]
    lib.fa2_fwd.restype = i
    f, u64, u32 = ctypes.c_float, ctypes.c_ulonglong, ctypes.c_uint
    lib.fa2_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, u64, u32, f, vp]
    lib.fa2_fwd_ex.restype = i
    lib.fa2_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, u64, u32, f, vp]
    lib.fa2_fwd_varlen.restype = i
    lib.fa2_strerror.argtypes = [i]
    lib.fa2_strerror.restype = ctypes.c_char_p
    ip = ctypes.POINTER(ctypes.c_int)
    lib.fa2_kernel_config.argtypes = [i, i, i, i, i, ip, ip, ip, ctypes.POINTER(ctypes.c_longlong), ip]
    lib.fa2_kernel_config.restype = i
    if path == LIB_PATH:
        _lib = lib
    return lib


def fa2_fwd(q, k, v, o, lse, B, H, S, D, causal, scale, stream) -> int:
    """The C entry point: pointers and the stream as integers (0/None = NULL)."""
    return int(load_library().fa2_fwd(q, k, v, o, lse, int(B), int(H), int(S), int(D), int(causal),
                                      float(scale), stream))


def fa2_fwd_ex(q, k, v, o, lse, B, H, H_kv, S, D, window_left, window_right, dropout_p, seed, offset, scale,
               stream) -> int:
    return int(load_library().fa2_fwd_ex(q, k, v, o, lse, int(B), int(H), int(H_kv), int(S), int(D),
                                         int(window_left), int(window_right), float(dropout_p), int(seed),
                                         int(offset), float(scale), stream))


def fa2_fwd_varlen(q, k, v, o, lse, cu_seqlens, num_seqs, total, max_seqlen, H, H_kv, D, window_left,
                   window_right, dropout_p, seed, offset, scale, stream) -> int:
    return int(load_library().fa2_fwd_varlen(q, k, v, o, lse, cu_seqlens, int(num_seqs), int(total),
                                             int(max_seqlen), int(H), int(H_kv), int(D), int(window_left),
                                             int(window_right), float(dropout_p), int(seed), int(offset),
                                             float(scale), stream))


def fa2_strerror(status: int) -> str:
    return load_library().fa2_strerror(int(status)).decode()


def fa2_kernel_config(B, H, S, D, causal) -> dict:
    rows, keys, threads, lds = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    blocks = ctypes.c_longlong()
    st = load_library().fa2_kernel_config(int(B), int(H), int(S), int(D), int(causal), ctypes.byref(rows),
                                          ctypes.byref(keys), ctypes.byref(threads), ctypes.byref(blocks),
                                          ctypes.byref(lds))
    if st != FA2_OK:
        raise FA2Error(st)
    return {"rows_per_block": rows.value, "keys_per_tile": keys.value, "threads_per_block": threads.value,
            "blocks": blocks.value, "lds_bytes": lds.value}


def _check_inputs(q, k, v):
    import torch

    if q.dtype != torch.float16 or k.dtype != torch.float16 or v.dtype != torch.float16:
        raise TypeError("q, k, v must be torch.float16")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if k.device != q.device or v.device != q.device:
        raise ValueError(f"q, k, v must be on one device, got {q.device}, {k.device}, {v.device}")
    if k.shape != v.shape:
        raise ValueError(f"k and v must have the same shape, got {tuple(k.shape)} {tuple(v.shape)}")


def _output(t, shape, dtype, like, name):
    import torch

    if t is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or t.device != like.device:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {like.device}")
    return t


def _window(causal, window):
    wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    if causal:
        wr = 0
    return wl, wr


def forward(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None, stream=None):
    """O and LSE for contiguous fp16 [B,H,S,D] CUDA tensors (torch allocates;
    the library computes). ``scale`` defaults to 1/sqrt(D)."""
    _check_inputs(q, k, v)
    if q.dim() != 4 or q.shape != k.shape:
        raise ValueError(f"q, k, v must share a [B,H,S,D] shape, got {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    B, H, S, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = _output(out, q.shape, q.dtype, q, "out")
    import torch
    lse = _output(lse, (B, H, S), torch.float32, q, "lse")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):  # the library launches on the current device
        st = fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, S, D,
                     int(bool(causal)), scale, stream)
    if st != FA2_OK:
        raise FA2Error(st)
    return out, lse


def forward_ex(q, k, v, causal: bool = False, window=None, dropout_p: float = 0.0, seed: int = 0, offset: int = 0,
               scale: float | None = None, out=None, lse=None, stream=None):
    """GQA/MQA, local window and dropout. q: [B,H,S,D]; k, v: [B,H_kv,S,D]
    with H a multiple of H_kv. ``window=(left, right)`` admits keys
    i-left .. i+right (-1 = unbounded); ``causal=True`` sets right to 0."""
    import torch

    _check_inputs(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:]:
        raise ValueError(f"q must be [B,H,S,D] and k, v [B,H_kv,S,D], got {tuple(q.shape)} {tuple(k.shape)}")
    B, H, S, D = q.shape
    H_kv = k.shape[1]
    wl, wr = _window(causal, window)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = _output(out, q.shape, q.dtype, q, "out")
    lse = _output(lse, (B, H, S), torch.float32, q, "lse")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = fa2_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, H_kv, S,
                        D, wl, wr, dropout_p, seed, offset, scale, stream)
    if st != FA2_OK:
        raise FA2Error(st)
    return out, lse


def forward_varlen(q, k, v, cu_seqlens, max_seqlen: int | None = None, causal: bool = False, window=None,
                   dropout_p: float = 0.0, seed: int = 0, offset: int = 0, scale: float | None = None, out=None,
                   lse=None, stream=None):
    """Packed sequences. q: [total,H,D]; k, v: [total,H_kv,D]; cu_seqlens: int32
    GPU tensor [num_seqs+1] of start rows (0 first, total last). Returns o
    [total,H,D] and lse [H,total]. Without ``max_seqlen`` the table is copied to
    the host (a synchronisation), checked, and its longest sequence used."""
    import torch

    _check_inputs(q, k, v)
    if q.dim() != 3 or k.dim() != 3 or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2]:
        raise ValueError(f"q must be [total,H,D] and k, v [total,H_kv,D], got {tuple(q.shape)} {tuple(k.shape)}")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous() \
            or cu_seqlens.device != q.device or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be a contiguous int32 [num_seqs+1] tensor on the device of q")
    total, H, D = q.shape
    H_kv = k.shape[1]
    num_seqs = cu_seqlens.numel() - 1
    if max_seqlen is None:
        cu = cu_seqlens.cpu().tolist()
        if cu[0] != 0 or cu[-1] != total or any(b < a for a, b in zip(cu, cu[1:])):
            raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at total")
        max_seqlen = max(1, max(b - a for a, b in zip(cu, cu[1:])))
    wl, wr = _window(causal, window)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = _output(out, q.shape, q.dtype, q, "out")
    lse = _output(lse, (H, total), torch.float32, q, "lse")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = fa2_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            cu_seqlens.data_ptr(), num_seqs, total, max_seqlen, H, H_kv, D, wl, wr, dropout_p,
                            seed, offset, scale, stream)
    if st != FA2_OK:
        raise FA2Error(st)
    return out, lse
