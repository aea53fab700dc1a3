"""Race check of the K/V ring (GPU): the poisoned-LDS debug library.

There is no LDS race detector for this GPU. The debug build of the same
sources (libfa2_poison.so, FA2_POISON_LDS=1) writes NaN over every chunk of a
ring stage, on the lane that is about to load it, and waits for those writes,
immediately before the stage's direct-to-LDS loads are issued. Any LDS read
that the kernel's protocol (wait for the loads, then a workgroup barrier,
before a stage is read; a barrier after the last read of a stage before it is
refilled) fails to order would see NaN, and NaN reaches O or LSE. Each case
must match the oracle and be bit-identical to the normal library.

The cases cover every kernel instance family: full and half height, D = 64
and 128, unmasked, causal and windowed, dropout, GQA, packed sequences, ragged
ends, and grids of one round and several."""
import ctypes
import math
import os
import sys

import numpy as np
import pytest

import oracle
from fa2_inputs import make_packed, make_random

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
POISON_LIB = os.path.join(ROOT, "attention_forward_fa2_amd", "libfa2_poison.so")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _lib():
    import attention_forward_fa2_amd as fa2
    return fa2.load_library(POISON_LIB)


def _run_dense(lib, q, k, v, window, p, seed, offset, scale):
    import torch
    dev = torch.device("cuda:0")
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v))
    B, H, S, D = q.shape
    o = torch.empty_like(qt)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    st = lib.fa2_fwd_ex(qt.data_ptr(), kt.data_ptr(), vt.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                        k.shape[1], S, D, window[0], window[1], p, seed, offset, scale,
                        torch.cuda.current_stream().cuda_stream)
    assert st == 0, f"status {st}"
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def _run_varlen(lib, q, k, v, cu, window, p, seed, offset, scale):
    import torch
    dev = torch.device("cuda:0")
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v))
    cut = torch.from_numpy(np.asarray(cu, dtype=np.int32)).to(dev)
    total, H, D = q.shape
    o = torch.empty_like(qt)
    lse = torch.empty((H, total), dtype=torch.float32, device=dev)
    st = lib.fa2_fwd_varlen(qt.data_ptr(), kt.data_ptr(), vt.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            cut.data_ptr(), len(cu) - 1, total, int(np.max(np.diff(cu))), H, k.shape[1], D,
                            window[0], window[1], p, seed, offset, scale, torch.cuda.current_stream().cuda_stream)
    assert st == 0, f"status {st}"
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def _check(O, L, Oref, Lref, Onorm, Lnorm, what, dropout_p=0.0):
    O64, L64 = O.astype(np.float64), L.astype(np.float64)
    assert np.all(np.isfinite(O64)) and np.all(np.isfinite(L64)), f"{what}: NaN/inf reached the output"
    dO = np.abs(O64 - Oref)
    dL = np.abs(L64 - Lref)
    same = np.array_equal(O.view(np.uint16), Onorm.view(np.uint16)) and \
        np.array_equal(L.view(np.uint32), Lnorm.view(np.uint32))
    log(f"  {what}: max|dO|={dO.max():.3e} mean|dO|={dO.mean():.3e} max|dLSE|={dL.max():.3e} "
        f"bit-identical to the normal build: {same}")
    amp = 1.0 / (1.0 - dropout_p)      # with dropout, O and its errors scale by 1/(1-p)
    assert dO.max() <= 4e-3 * amp and dO.mean() <= 5e-4 * amp and dL.max() <= 1e-3, what
    assert same, f"{what}: differs from the normal build"


# (B, H, H_kv, S, D, window, p): window (-1, -1) plain, (-1, 0) causal
DENSE = [
    (4, 8, 8, 4096, 64, (-1, -1), 0.0),     # full height, one round (workload 2 non-causal)
    (4, 8, 8, 4096, 64, (-1, 0), 0.0),      # half height, one round, serpentine
    (4, 8, 8, 4100, 64, (-1, 0), 0.0),      # full height causal, several rounds, ragged
    (2, 5, 5, 1000, 64, (-1, -1), 0.0),     # half height plain (small grid), ragged
    (2, 16, 16, 1100, 128, (-1, 0), 0.0),   # D=128 full height causal, ragged
    (1, 16, 16, 2048, 128, (-1, -1), 0.0),  # D=128 one round
    (1, 8, 8, 3000, 128, (-1, -1), 0.0),    # D=128 half height plain
    (2, 8, 2, 2000, 64, (300, 40), 0.0),    # window, GQA
    (2, 4, 4, 1500, 64, (-1, -1), 0.2),     # dropout plain
    (2, 4, 4, 1500, 128, (-1, 0), 0.2),     # dropout causal D=128
    (1, 4, 1, 5000, 64, (700, 0), 0.1),     # window + dropout + MQA
]


@pytest.mark.parametrize("case", DENSE, ids=[f"B{c[0]}H{c[1]}kv{c[2]}S{c[3]}D{c[4]}w{c[5][0]}_{c[5][1]}p{c[6]}"
                                             for c in DENSE])
def test_poisoned_dense(case):
    import attention_forward_fa2_amd as fa2
    B, H, H_kv, S, D, window, p = case
    log(f"case poisoned LDS dense {case}")
    lib = _lib()
    q, _, _ = make_random(95_000 + S + D, B, H, S, D)
    _, k, v = make_random(96_000 + S + D, B, H_kv, S, D)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    p32 = float(np.float32(p))
    O, L = _run_dense(lib, q, k, v, window, p32, 77, 5, scale)
    On, Ln = _run_dense(fa2.load_library(), q, k, v, window, p32, 77, 5, scale)
    Oref, Lref = oracle.attention_ex(q, k, v, scale, window=window, dropout_p=p32, seed=77, offset=5)
    _check(O, L, Oref, Lref, On, Ln, f"poisoned dense {case}", p32)


PACKED = [([700, 0, 1200, 64, 333], 8, 2, 64, (-1, -1), 0.0),
          ([700, 0, 1200, 64, 333], 8, 2, 64, (-1, 0), 0.15),
          ([4100, 5001], 4, 4, 64, (-1, 0), 0.0),           # full-height packed causal
          ([900, 1300, 17], 4, 1, 128, (100, 20), 0.0)]


@pytest.mark.parametrize("case", PACKED, ids=[f"{'-'.join(map(str, c[0]))}H{c[1]}kv{c[2]}D{c[3]}"
                                              f"w{c[4][0]}_{c[4][1]}p{c[5]}" for c in PACKED])
def test_poisoned_packed(case):
    import attention_forward_fa2_amd as fa2
    lens, H, H_kv, D, window, p = case
    log(f"case poisoned LDS packed {case}")
    lib = _lib()
    q, k, v, cu = make_packed(97_000 + sum(lens) + D, lens, H, H_kv, D)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    p32 = float(np.float32(p))
    O, L = _run_varlen(lib, q, k, v, cu, window, p32, 9, 2, scale)
    On, Ln = _run_varlen(fa2.load_library(), q, k, v, cu, window, p32, 9, 2, scale)
    Oref, Lref = oracle.attention_varlen(q, k, v, cu, scale, window=window, dropout_p=p32, seed=9, offset=2)
    _check(O, L, Oref, Lref, On, Ln, f"poisoned packed {case}", p32)
