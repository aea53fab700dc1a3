"""GPU parity of the production features (GQA/MQA, local window, packed
variable-length sequences, dropout) through the C ABI, against the fp64
oracle, with the tolerances of the dense tests: max |dO| <= 4e-3,
mean |dO| <= 5e-4, max |dLSE| <= 1e-3. Dropout is compared with the oracle's
own Philox draws, so the same keys are dropped on both sides and the
comparison is element by element."""
import math
import sys

import numpy as np
import pytest

import oracle
from fa2_inputs import FEATURES, make_feature_inputs, make_packed, make_random, normal_f16

pytestmark = pytest.mark.gpu

TOL_MAX_O = 4e-3
TOL_MEAN_O = 5e-4
TOL_LSE = 1e-3
# With dropout every kept value of O is multiplied by 1/(1-p) (O_i = sum_j P_ij z_ij v_j / (1-p)), and
# so are the absolute rounding errors of O: the O bounds scale by that factor (the LSE, computed before
# dropout, keeps its bound). At p = 0.5 an fp16 O reaches |O| of 8 and more on peaked rows, where one
# fp16 step is 2^-7, and the unscaled bound would sit below the output format's own resolution.


def o_bounds(dropout_p: float = 0.0):
    """(max, mean) bounds of |O - O_ref| for a dropout probability."""
    amp = 1.0 / (1.0 - dropout_p)
    return TOL_MAX_O * amp, TOL_MEAN_O * amp


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(O, L, Oref, Lref, what, dropout_p: float = 0.0):
    O64, L64 = O.astype(np.float64), L.astype(np.float64)
    assert np.all(np.isfinite(O64)), f"{what}: non-finite O"
    assert np.all(np.isfinite(L64)), f"{what}: non-finite LSE"
    dO = np.abs(O64 - Oref)
    dL = np.abs(L64 - Lref)
    tol_max, tol_mean = o_bounds(dropout_p)
    log(f"  {what}: max|dO|={dO.max():.3e} mean|dO|={dO.mean():.3e} max|dLSE|={dL.max():.3e}")
    assert dO.max() <= tol_max, f"{what}: max|dO| {dO.max():.3e}"
    assert dO.mean() <= tol_mean, f"{what}: mean|dO| {dO.mean():.3e}"
    assert dL.max() <= TOL_LSE, f"{what}: max|dLSE| {dL.max():.3e}"


def gpu_ex(q, k, v, causal=False, window=None, dropout_p=0.0, seed=0, offset=0, scale=None):
    import torch
    import attention_forward_fa2_amd as fa2
    dev = torch.device("cuda:0")
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v))
    o, lse = fa2.forward_ex(qt, kt, vt, causal=causal, window=window, dropout_p=dropout_p, seed=seed,
                            offset=offset, scale=scale)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def gpu_varlen(q, k, v, cu, causal=False, window=None, dropout_p=0.0, seed=0, offset=0, scale=None,
               max_seqlen=None):
    import torch
    import attention_forward_fa2_amd as fa2
    dev = torch.device("cuda:0")
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v))
    cut = torch.from_numpy(np.asarray(cu, dtype=np.int32)).to(dev)
    o, lse = fa2.forward_varlen(qt, kt, vt, cut, max_seqlen=max_seqlen, causal=causal, window=window,
                                dropout_p=dropout_p, seed=seed, offset=offset, scale=scale)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def eff_window(causal, window):
    wl, wr = (-1, -1) if window is None else window
    return (wl, 0) if causal else (wl, wr)


def dense_case(q, k, v, causal=False, window=None, dropout_p=0.0, seed=0, offset=0, what=""):
    D = q.shape[-1]
    scale = 1.0 / math.sqrt(D)
    p32 = float(np.float32(dropout_p))
    log(f"case {what} q={q.shape} k={k.shape} causal={causal} window={window} p={dropout_p}")
    O, L = gpu_ex(q, k, v, causal, window, p32, seed, offset, scale)
    Oref, Lref = oracle.attention_ex(q, k, v, float(np.float32(scale)), window=eff_window(causal, window),
                                     dropout_p=p32, seed=seed, offset=offset)
    check(O, L, Oref, Lref, what, p32)
    return O, L


# ---- GQA / MQA ----

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H_kv", [1, 2, 8])
def test_gqa(D, H_kv):
    H = 8
    for S in (65, 300):
        q = normal_f16(70_000 + S + D + H_kv, (2, H, S, D))
        k = normal_f16(70_001 + S + D + H_kv, (2, H_kv, S, D))
        v = normal_f16(70_002 + S + D + H_kv, (2, H_kv, S, D))
        for causal in (False, True):
            dense_case(q, k, v, causal, what=f"GQA H={H} H_kv={H_kv} S={S} D={D}")


def test_gqa_equals_repeated_heads_bitwise():
    """GQA reads K/V head h // group: the result is bit-identical to the plain
    entry point on K/V repeated along the head axis."""
    import torch
    import attention_forward_fa2_amd as fa2
    q = normal_f16(71_000, (2, 6, 257, 64))
    k = normal_f16(71_001, (2, 2, 257, 64))
    v = normal_f16(71_002, (2, 2, 257, 64))
    for causal in (False, True):
        O1, L1 = gpu_ex(q, k, v, causal)
        dev = torch.device("cuda:0")
        kr = torch.from_numpy(np.ascontiguousarray(np.repeat(k, 3, axis=1))).to(dev)
        vr = torch.from_numpy(np.ascontiguousarray(np.repeat(v, 3, axis=1))).to(dev)
        o2, l2 = fa2.forward(torch.from_numpy(q).to(dev), kr, vr, causal=causal)
        torch.cuda.synchronize()
        assert np.array_equal(O1.view(np.uint16), o2.cpu().numpy().view(np.uint16))
        assert np.array_equal(L1.view(np.uint32), l2.cpu().numpy().view(np.uint32))


# ---- local window ----

WINDOWS = [(0, 0), (1, 0), (3, 7), (64, 0), (100, 100), (255, 1), (0, 300), (700, 5), (7, 2000), (63, 64)]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", [129, 513, 1000])
def test_window(D, S):
    q, k, v = make_random(72_000 + S + D, 1, 2, S, D)
    for window in WINDOWS:
        dense_case(q, k, v, window=window, what=f"window {window} S={S} D={D}")


def test_window_uniform_scores():
    """Q = 0: O_i is the mean of v over the window, LSE_i = ln(window size)."""
    S, D = 700, 64
    _, k, v = make_random(73_000, 1, 2, S, D)
    q = np.zeros_like(k)
    for wl, wr in ((5, 9), (0, 0), (300, 0)):
        O, L = gpu_ex(q, k, v, window=(wl, wr))
        i = np.arange(S)
        lo, hi = np.maximum(0, i - wl), np.minimum(S - 1, i + wr)
        csum = np.concatenate([np.zeros((1, 2, 1, D)), np.cumsum(v.astype(np.float64), axis=2)], axis=2)
        ref = (csum[:, :, hi + 1] - csum[:, :, lo]) / (hi - lo + 1)[None, None, :, None]
        assert np.max(np.abs(O.astype(np.float64) - ref)) <= TOL_MAX_O
        assert np.max(np.abs(L - np.log(hi - lo + 1)[None, None, :])) <= TOL_LSE


def test_window_special_cases_match_plain_entry():
    """(-1, -1) and (-1, 0), and windows wider than the sequence, take the plain
    kernels: bit-identical to fa2_fwd."""
    import torch
    import attention_forward_fa2_amd as fa2
    q, k, v = make_random(74_000, 2, 2, 300, 128)
    dev = torch.device("cuda:0")
    for window, causal in (((-1, -1), False), ((-1, 0), True), ((300, 300), False), ((5000, 0), True)):
        O1, L1 = gpu_ex(q, k, v, window=window)
        o2, l2 = fa2.forward(*(torch.from_numpy(x).to(dev) for x in (q, k, v)), causal=causal)
        torch.cuda.synchronize()
        assert np.array_equal(O1.view(np.uint16), o2.cpu().numpy().view(np.uint16)), window
        assert np.array_equal(L1.view(np.uint32), l2.cpu().numpy().view(np.uint32)), window


# ---- packed variable-length sequences ----

LENS = [[5, 0, 17, 1, 9], [256, 255, 257], [513, 64, 700, 1], [1000], [0, 3, 0]]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("lens", LENS, ids=["-".join(map(str, x)) for x in LENS])
def test_varlen(D, lens):
    for H, H_kv in ((4, 4), (4, 1)):
        q, k, v, cu = make_packed(75_000 + D + sum(lens), lens, H, H_kv, D)
        scale = 1.0 / math.sqrt(D)
        for causal, window in ((False, None), (True, None), (False, (30, 0)), (False, (2, 40))):
            log(f"case varlen lens={lens} H={H} H_kv={H_kv} D={D} causal={causal} window={window}")
            O, L = gpu_varlen(q, k, v, cu, causal, window, scale=scale)
            Oref, Lref = oracle.attention_varlen(q, k, v, cu, float(np.float32(scale)),
                                                 window=eff_window(causal, window))
            check(O, L, Oref, Lref, f"varlen {lens} H_kv={H_kv} causal={causal} window={window}")


def test_varlen_rows_are_independent_of_neighbours():
    """Changing one sequence's data leaves every other sequence's output
    bit-identical (no attention across sequence boundaries)."""
    lens = [300, 257, 129]
    q, k, v, cu = make_packed(76_000, lens, 2, 2, 64)
    O1, L1 = gpu_varlen(q, k, v, cu, causal=False)
    k2, v2 = k.copy(), v.copy()
    a, e = int(cu[1]), int(cu[2])
    k2[a:e] = normal_f16(76_010, k2[a:e].shape)
    v2[a:e] = normal_f16(76_011, v2[a:e].shape)
    O2, L2 = gpu_varlen(q, k2, v2, cu, causal=False)
    for s, (x, y) in enumerate(zip(cu, cu[1:])):
        same = np.array_equal(O1[x:y].view(np.uint16), O2[x:y].view(np.uint16))
        assert same == (s != 1), f"sequence {s}"


@pytest.mark.parametrize("nseq", [64, 65])
def test_varlen_many_sequences(nseq):
    """Up to 64 packed sequences are walked longest first (the kernel ranks
    the table), more in table order: both sides of that limit, with ties and
    empty sequences, against the oracle."""
    g = np.random.Generator(np.random.PCG64(79_000 + nseq))
    lens = g.integers(1, 300, size=nseq)
    lens[g.random(nseq) < 0.1] = 0
    lens[:4] = 150                                   # ties
    q, k, v, cu = make_packed(79_100 + nseq, lens.tolist(), 2, 1, 64)
    for causal in (False, True):
        log(f"case varlen {nseq} sequences causal={causal}")
        O, L = gpu_varlen(q, k, v, cu, causal, scale=0.125)
        Oref, Lref = oracle.attention_varlen(q, k, v, cu, 0.125, window=eff_window(causal, None))
        check(O, L, Oref, Lref, f"varlen {nseq} sequences causal={causal}")


def test_varlen_max_seqlen_given():
    lens = [100, 300, 50]
    q, k, v, cu = make_packed(77_000, lens, 2, 1, 128)
    O1, L1 = gpu_varlen(q, k, v, cu, causal=True)
    O2, L2 = gpu_varlen(q, k, v, cu, causal=True, max_seqlen=300)
    assert np.array_equal(O1.view(np.uint16), O2.view(np.uint16))
    assert np.array_equal(L1.view(np.uint32), L2.view(np.uint32))


# ---- dropout ----

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("p", [0.1, 0.5])
def test_dropout(D, p):
    for S in (200, 513):
        q, k, v = make_random(78_000 + S + D, 1, 2, S, D)
        for causal in (False, True):
            dense_case(q, k, v, causal, dropout_p=p, seed=0x0123_4567_89AB_CDEF, offset=S,
                       what=f"dropout p={p} S={S} D={D}")


def test_dropout_with_window_gqa_and_varlen():
    q = normal_f16(79_000, (1, 4, 300, 64))
    k = normal_f16(79_001, (1, 2, 300, 64))
    v = normal_f16(79_002, (1, 2, 300, 64))
    dense_case(q, k, v, window=(50, 10), dropout_p=0.25, seed=11, offset=3, what="dropout+window+GQA")
    lens = [77, 0, 200, 33]
    q, k, v, cu = make_packed(79_100, lens, 4, 2, 64)
    scale = 1.0 / math.sqrt(64)
    p32 = float(np.float32(0.3))
    for causal in (False, True):
        O, L = gpu_varlen(q, k, v, cu, causal, None, dropout_p=p32, seed=5, offset=9, scale=scale)
        Oref, Lref = oracle.attention_varlen(q, k, v, cu, float(np.float32(scale)),
                                             window=eff_window(causal, None), dropout_p=p32, seed=5, offset=9)
        check(O, L, Oref, Lref, f"dropout varlen causal={causal}", p32)


def test_dropout_is_reproducible_and_seeded():
    q, k, v = make_random(80_000, 2, 2, 257, 64)
    O1, L1 = gpu_ex(q, k, v, dropout_p=0.2, seed=42, offset=7)
    O2, L2 = gpu_ex(q, k, v, dropout_p=0.2, seed=42, offset=7)
    O3, L3 = gpu_ex(q, k, v, dropout_p=0.2, seed=42, offset=8)
    O4, _ = gpu_ex(q, k, v, dropout_p=0.2, seed=43, offset=7)
    assert np.array_equal(O1.view(np.uint16), O2.view(np.uint16))
    assert not np.array_equal(O1, O3) and not np.array_equal(O1, O4)
    assert np.array_equal(L1.view(np.uint32), L3.view(np.uint32))   # LSE is before dropout


def test_dropout_zero_is_plain():
    q, k, v = make_random(81_000, 1, 2, 300, 128)
    O1, L1 = gpu_ex(q, k, v, causal=True, dropout_p=0.0, seed=99)
    O2, L2 = gpu_ex(q, k, v, causal=True)
    assert np.array_equal(O1.view(np.uint16), O2.view(np.uint16))


# ---- the feature workloads at full size (every element) ----

@pytest.mark.parametrize("key", sorted(FEATURES))
def test_feature_workload_whole_tensor(key):
    f = FEATURES[key]
    log(f"case feature workload {key}: {f.name}")
    scale = float(np.float32(f.scale))
    if f.packed:
        q, k, v, cu = make_feature_inputs(key)
        O, L = gpu_varlen(q, k, v, cu, False, f.window, f.dropout_p, f.seed, 0, f.scale)
        Oref, Lref = oracle.attention_varlen(q, k, v, cu, scale, window=f.window, dropout_p=f.dropout_p,
                                             seed=f.seed, offset=0)
    else:
        q, k, v = make_feature_inputs(key)
        O, L = gpu_ex(q, k, v, False, f.window, f.dropout_p, f.seed, 0, f.scale)
        Oref, Lref = oracle.attention_ex(q, k, v, scale, window=f.window, dropout_p=f.dropout_p, seed=f.seed,
                                         offset=0)
    check(O, L, Oref, Lref, f"{key} whole tensor", f.dropout_p)


@pytest.mark.parametrize("key", ["dropout", "varlen", "window"])
def test_feature_workload_whole_tensor_causal(key):
    """The causal side of the feature workloads, as the bench runs them with
    --causal: the window's right edge at 0 (for an unbounded window, causal)."""
    f = FEATURES[key]
    win = (f.window[0], 0)
    log(f"case feature workload {key} causal: {f.name}, window {win}")
    scale = float(np.float32(f.scale))
    if f.packed:
        q, k, v, cu = make_feature_inputs(key)
        O, L = gpu_varlen(q, k, v, cu, False, win, f.dropout_p, f.seed, 0, f.scale)
        Oref, Lref = oracle.attention_varlen(q, k, v, cu, scale, window=win, dropout_p=f.dropout_p,
                                             seed=f.seed, offset=0)
    else:
        q, k, v = make_feature_inputs(key)
        O, L = gpu_ex(q, k, v, False, win, f.dropout_p, f.seed, 0, f.scale)
        Oref, Lref = oracle.attention_ex(q, k, v, scale, window=win, dropout_p=f.dropout_p, seed=f.seed,
                                         offset=0)
    check(O, L, Oref, Lref, f"{key} causal whole tensor", f.dropout_p)


def test_packed_causal_full_height():
    """Packed causal batch whose sequences average more than 4095 rows: it
    takes the full-height workgroups (shorter averages take half height), with
    ragged sequence ends; plain and with dropout, every element."""
    lens = [4100, 5001, 4500]
    assert sum(lens) / len(lens) > 4095
    q, k, v, cu = make_packed(83_000, lens, 8, 2, 64)
    scale = 0.125
    for p in (0.0, float(np.float32(0.2))):
        log(f"case packed causal full height lens={lens} p={p}")
        O, L = gpu_varlen(q, k, v, cu, True, None, dropout_p=p, seed=21, offset=4, scale=scale)
        Oref, Lref = oracle.attention_varlen(q, k, v, cu, scale, window=(-1, 0), dropout_p=p, seed=21, offset=4)
        check(O, L, Oref, Lref, f"packed causal full height p={p}", p)
