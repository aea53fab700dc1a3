"""MI355X-native FlashAttention-2 forward: Python binding of libfa2.so.

The binding only marshals arguments: every step of the forward pass runs in the
HIP kernels behind the C ABI of include/fa2.h. There is no CPU or PyTorch
fallback: if the library is missing, importing the binding's entry points
raises.

    fa2_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, S, D, causal, scale, stream)
        the C call itself (integers for pointers and the stream); returns the status.
    fa2_strerror(status) -> str
    fa2_kernel_config(B, H, S, D, causal) -> dict
    forward(q, k, v, causal=False, scale=None, out=None, lse=None) -> (o, lse)
        torch convenience: allocates outputs with torch, launches on the current stream.
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
    5: "FA2_ERR_OVERFLOW", 6: "FA2_ERR_ALIAS", 7: "FA2_ERR_DEVICE", 8: "FA2_ERR_LAUNCH",
}
EXPORTED = ("fa2_fwd", "fa2_strerror", "fa2_kernel_config")

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


def forward(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None, stream=None):
    """O and LSE for contiguous fp16 [B,H,S,D] CUDA tensors (torch allocates;
    the library computes). ``scale`` defaults to 1/sqrt(D)."""
    import torch

    if q.dtype != torch.float16 or k.dtype != torch.float16 or v.dtype != torch.float16:
        raise TypeError("q, k, v must be torch.float16")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v must share a [B,H,S,D] shape, got {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    B, H, S, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, S, D,
                 int(bool(causal)), scale, stream)
    if st != FA2_OK:
        raise FA2Error(st)
    return out, lse
