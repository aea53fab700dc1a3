"""Pins for the fp64 oracle: facts fixed by the pages and by mathematics.

Each ``pin_*`` takes a loaded oracle library (``oracle.load()`` or a copy of it
built with a planted mistake) and raises AssertionError when the library gets
the fact wrong. ``test_oracle.py`` runs them on the real oracle and
``test_oracle_mutants.py`` checks that every planted mistake breaks at least
one of them.

Definition pinned: the page "CuTe 详解：以 FlashAttention-2 拆解 Layout、
TiledCopy 与 TiledMMA", §"先看全局：FA2 中的数据究竟去了哪里" (S = Q Kᵀ scaled,
P = softmax(S), O = P V), §"教学配置：一块 CTA 做什么" (O_i = õ_i / ℓ_i with
ℓ_i the sum of e^{s_ij - m_i}), §"正确性、编译与计时方法" (the uniform-score
and concentrated-softmax inputs) and the log-sum-exp output of
§"与官方 FA2 比较时，先对齐契约" (natural log).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy.special import logsumexp, softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _rand(seed, shape, sigma=1.0):
    # fp16-representable values, as the kernel would receive them
    return (_rng(seed).standard_normal(shape) * sigma).astype(np.float16).astype(np.float64)


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert a.shape == b.shape and err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


def pin_worked_2x2(lib):
    g = json.load(open(os.path.join(GOLDEN, "worked_2x2.json")))
    q = np.array(g["q"], dtype=np.float64)[None, None]
    k = np.array(g["k"], dtype=np.float64)[None, None]
    v = np.array(g["v"], dtype=np.float64)[None, None]
    for mode, causal in (("noncausal", False), ("causal", True)):
        O, L = oracle.attention(q, k, v, causal, g["scale"], lib=lib)
        _close(O[0, 0], g[mode]["O"], 1e-14, f"2x2 {mode} O")
        _close(L[0, 0], g[mode]["LSE"], 1e-14, f"2x2 {mode} LSE")


def pin_worked_4x4(lib):
    g = json.load(open(os.path.join(GOLDEN, "worked_4x4.json")))
    q = np.array(g["q"], dtype=np.float64).reshape(1, 1, 4, 1)
    k = np.array(g["k"], dtype=np.float64).reshape(1, 1, 4, 1)
    v = np.array(g["v"], dtype=np.float64).reshape(1, 1, 4, 1)
    for mode, causal in (("noncausal", False), ("causal", True)):
        O, L = oracle.attention(q, k, v, causal, g["scale"], lib=lib)
        _close(O[0, 0, :, 0], g[mode]["O"], 1e-13, f"4x4 {mode} O")
        _close(L[0, 0], g[mode]["LSE"], 1e-13, f"4x4 {mode} LSE")


def pin_uniform_scores(lib):
    """Q = 0 makes every score equal: O_i is the mean of the admissible v_j and
    LSE_i = ln(number of admissible keys). The uniform-score input of the page."""
    B, H, S, D = 2, 3, 37, 8
    q = np.zeros((B, H, S, D))
    k = _rand(11, (B, H, S, D))
    v = _rand(12, (B, H, S, D))
    O, L = oracle.attention(q, k, v, False, 0.125, lib=lib)
    _close(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), 1e-13, "Q=0 non-causal O")
    _close(L, np.full((B, H, S), math.log(S)), 1e-13, "Q=0 non-causal LSE")
    O, L = oracle.attention(q, k, v, True, 0.125, lib=lib)
    prefix_mean = np.cumsum(v, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    _close(O, prefix_mean, 1e-13, "Q=0 causal O (prefix mean)")
    _close(L, np.broadcast_to(np.log(np.arange(1, S + 1)), (B, H, S)), 1e-13, "Q=0 causal LSE")


def pin_causal_first_row(lib):
    """Causal row 0 sees only key 0: O_0 = v_0 and LSE_0 = scale * q_0 . k_0."""
    B, H, S, D = 1, 2, 9, 16
    q, k, v = _rand(21, (B, H, S, D)), _rand(22, (B, H, S, D)), _rand(23, (B, H, S, D))
    O, L = oracle.attention(q, k, v, True, 0.25, lib=lib)
    _close(O[:, :, 0], v[:, :, 0], 1e-15, "causal row 0 O")
    _close(L[:, :, 0], 0.25 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), 1e-13,
           "causal row 0 LSE")


def pin_convexity(lib):
    """If every v_j is the same vector u, O_i = u (softmax weights sum to 1)."""
    B, H, S, D = 1, 2, 23, 8
    q, k = _rand(31, (B, H, S, D), 3.0), _rand(32, (B, H, S, D), 3.0)
    u = _rand(33, (B, H, 1, D))
    v = np.broadcast_to(u, (B, H, S, D)).copy()
    for causal in (False, True):
        O, _ = oracle.attention(q, k, v, causal, 0.125, lib=lib)
        _close(O, np.broadcast_to(u, O.shape), 1e-13, f"constant V (causal={causal})")


def pin_probabilities(lib):
    """With V = I (D = S), row i of O is row i of P: it is non-negative, sums to
    1, and equals exp(scale q_i.k_j - LSE_i), tying O and LSE together."""
    B, H, S = 1, 2, 12
    D = S
    q, k = _rand(41, (B, H, S, D)), _rand(42, (B, H, S, D))
    v = np.broadcast_to(np.eye(S), (B, H, S, D)).copy()
    scale = 0.3
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, causal, scale, lib=lib)
        assert np.all(O >= 0), "P has a negative entry"
        _close(O.sum(axis=-1), np.ones((B, H, S)), 1e-14, f"P rows sum to 1 (causal={causal})")
        s = scale * (q @ np.swapaxes(k, -1, -2))
        P = np.exp(s - L[..., None])
        if causal:
            P = P * np.tril(np.ones((S, S)))
        _close(O, P, 1e-14, f"P = exp(s - LSE) (causal={causal})")


def pin_key_shift(lib):
    """Adding one vector u to every key leaves P and O unchanged and adds
    scale*q_i.u to LSE_i (the shift factors out of the softmax)."""
    B, H, S, D = 1, 1, 19, 8
    q, k, v = _rand(51, (B, H, S, D)), _rand(52, (B, H, S, D)), _rand(53, (B, H, S, D))
    u = _rand(54, (D,))
    scale = 0.125
    for causal in (False, True):
        O1, L1 = oracle.attention(q, k, v, causal, scale, lib=lib)
        O2, L2 = oracle.attention(q, k + u, v, causal, scale, lib=lib)
        _close(O2, O1, 1e-12, f"key shift O (causal={causal})")
        _close(L2 - L1, scale * (q @ u), 1e-12, f"key shift LSE (causal={causal})")


def pin_permutations(lib):
    """Non-causal attention is invariant to a joint permutation of the (k_j, v_j)
    pairs and equivariant to a permutation of the queries."""
    B, H, S, D = 1, 2, 17, 8
    q, k, v = _rand(61, (B, H, S, D)), _rand(62, (B, H, S, D)), _rand(63, (B, H, S, D))
    perm = _rng(64).permutation(S)
    O1, L1 = oracle.attention(q, k, v, False, 0.125, lib=lib)
    O2, L2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], False, 0.125, lib=lib)
    _close(O2, O1, 1e-13, "joint K/V permutation O")
    _close(L2, L1, 1e-13, "joint K/V permutation LSE")
    O3, L3 = oracle.attention(q[:, :, perm], k, v, False, 0.125, lib=lib)
    _close(O3, O1[:, :, perm], 1e-15, "query permutation O")
    _close(L3, L1[:, :, perm], 1e-15, "query permutation LSE")


def pin_library_softmax(lib):
    """Against scipy.special.softmax / logsumexp applied to the explicit score
    matrix (a different route: whole-matrix numpy, masked with -inf)."""
    for seed, (B, H, S, D), sigma in ((71, (2, 2, 33, 16), 1.0), (72, (1, 3, 50, 8), 3.0)):
        q, k, v = _rand(seed, (B, H, S, D), sigma), _rand(seed + 1, (B, H, S, D), sigma), \
            _rand(seed + 2, (B, H, S, D))
        scale = 1.0 / math.sqrt(D)
        for causal in (False, True):
            s = scale * (q @ np.swapaxes(k, -1, -2))
            if causal:
                s = np.where(np.tril(np.ones((S, S), dtype=bool)), s, -np.inf)
            P = softmax(s, axis=-1)
            O, L = oracle.attention(q, k, v, causal, scale, lib=lib)
            _close(O, P @ v, 1e-12, f"scipy softmax O (causal={causal})")
            _close(L, logsumexp(s, axis=-1), 1e-12, f"scipy logsumexp (causal={causal})")


def pin_rectangular_head_dim(lib):
    """Scores contract q_i with k_j over D; a swapped operand or index shows up
    once D differs from S and Q differs from K."""
    B, H, S, D = 1, 1, 5, 3
    q = np.arange(S * D, dtype=np.float64).reshape(1, 1, S, D) / 10
    k = (np.arange(S * D, dtype=np.float64)[::-1].reshape(1, 1, S, D) - 7) / 10
    v = np.arange(S * D, dtype=np.float64).reshape(1, 1, S, D) ** 2 / 50
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, causal, 0.7, lib=lib)
        for i in range(S):
            keys = range(i + 1) if causal else range(S)
            sc = [0.7 * math.fsum(q[0, 0, i, d] * k[0, 0, j, d] for d in range(D)) for j in keys]
            M = max(sc)
            w = [math.exp(x - M) for x in sc]
            tot = math.fsum(w)
            for d in range(D):
                ref = math.fsum(wj * v[0, 0, j, d] for wj, j in zip(w, keys)) / tot
                assert abs(O[0, 0, i, d] - ref) <= 1e-13, f"row {i} col {d}: {O[0, 0, i, d]} vs {ref}"
            assert abs(L[0, 0, i] - (M + math.log(tot))) <= 1e-13, f"row {i} LSE"


def pin_dominant_key(lib):
    """The concentrated-softmax input taken to its limit: scores of -2000, 0 and
    2000 put all the weight on the largest admissible score, so O_i = v_j* and
    LSE_i = s_ij* to double precision. exp of an unshifted score overflows
    here, so this also pins the max subtraction."""
    q = np.full((1, 1, 3, 1), 40.0)
    k = np.array([-50.0, 0.0, 50.0]).reshape(1, 1, 3, 1)
    v = np.array([[1.0, -2.0], [3.0, 5.0], [-7.0, 11.0]]).reshape(1, 1, 3, 2)
    v1 = np.broadcast_to(v, (1, 1, 3, 2))
    O, L = oracle.attention(q, k, np.ascontiguousarray(v1[..., :1]), False, 1.0, lib=lib)
    _close(O[0, 0, :, 0], [-7.0, -7.0, -7.0], 0.0, "dominant key non-causal O")
    _close(L[0, 0], [2000.0] * 3, 1e-12, "dominant key non-causal LSE")
    O, L = oracle.attention(q, k, np.ascontiguousarray(v1[..., :1]), True, 1.0, lib=lib)
    _close(O[0, 0, :, 0], [1.0, 3.0, -7.0], 0.0, "dominant key causal O")
    _close(L[0, 0], [-2000.0, 0.0, 2000.0], 1e-12, "dominant key causal LSE")


ALL_PINS = [pin_dominant_key, pin_worked_2x2, pin_worked_4x4, pin_uniform_scores, pin_causal_first_row,
            pin_convexity, pin_probabilities, pin_key_shift, pin_permutations,
            pin_library_softmax, pin_rectangular_head_dim]


# ---- the production features of §"哪些结论可以迁移，哪些只是本例特例" ----
# GQA/MQA, local window, packed variable-length sequences and dropout, under the
# readings stated at the top of oracle/attn_oracle.c.

def pin_philox_known_answers(lib):
    """Philox4x32-10 reproduces the known-answer vectors its authors publish."""
    g = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    for vec in g["vectors"]:
        got = oracle.philox4x32_10([int(x, 16) for x in vec["counter"]], [int(x, 16) for x in vec["key"]], lib=lib)
        assert got == [int(x, 16) for x in vec["out"]], f"Philox KAT {vec['counter']}: got {[hex(x) for x in got]}"


def _band_mask(S, wl, wr):
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    ok = np.ones((S, S), dtype=bool)
    if wl >= 0:
        ok &= j >= i - wl
    if wr >= 0:
        ok &= j <= i + wr
    return ok


WINDOWS = [(-1, -1), (-1, 0), (0, 0), (3, 2), (0, 5), (7, -1), (-1, 4), (1, 0), (40, 40)]


def pin_window_uniform(lib):
    """Q = 0: O_i is the mean of v_j over the window and LSE_i = ln(window
    size), which fixes both window bounds to the key."""
    B, H, S, D = 1, 2, 29, 4
    q = np.zeros((B, H, S, D))
    k, v = _rand(81, (B, H, S, D)), _rand(82, (B, H, S, D))
    for wl, wr in WINDOWS:
        ok = _band_mask(S, wl, wr).astype(np.float64)
        cnt = ok.sum(axis=1)
        O, L = oracle.attention_ex(q, k, v, 0.125, window=(wl, wr), lib=lib)
        _close(O, (ok @ v) / cnt[:, None], 1e-13, f"window {wl},{wr} Q=0 O")
        _close(L, np.broadcast_to(np.log(cnt), (B, H, S)), 1e-13, f"window {wl},{wr} Q=0 LSE")


def pin_window_library_softmax(lib):
    """Against scipy's softmax / logsumexp of the full score matrix with -inf
    outside the band, for GQA heads (query head h reads K/V head h // group)."""
    B, H, H_kv, S, D = 2, 6, 2, 23, 8
    q, k, v = _rand(91, (B, H, S, D), 2.0), _rand(92, (B, H_kv, S, D), 2.0), _rand(93, (B, H_kv, S, D))
    kr = np.repeat(k, H // H_kv, axis=1)
    vr = np.repeat(v, H // H_kv, axis=1)
    scale = 0.3
    for wl, wr in WINDOWS:
        s = scale * (q @ np.swapaxes(kr, -1, -2))
        s = np.where(_band_mask(S, wl, wr), s, -np.inf)
        O, L = oracle.attention_ex(q, k, v, scale, window=(wl, wr), lib=lib)
        _close(O, softmax(s, axis=-1) @ vr, 1e-12, f"window {wl},{wr} scipy O")
        _close(L, logsumexp(s, axis=-1), 1e-12, f"window {wl},{wr} scipy LSE")


def pin_window_zero(lib):
    """Window (0, 0): each query sees only its own key, so O_i = v_i and
    LSE_i = scale * q_i . k_i."""
    B, H, S, D = 1, 3, 11, 8
    q, k, v = _rand(95, (B, H, S, D)), _rand(96, (B, H, S, D)), _rand(97, (B, H, S, D))
    O, L = oracle.attention_ex(q, k, v, 0.5, window=(0, 0), lib=lib)
    _close(O, v, 0.0, "window 0,0 O")
    _close(L, 0.5 * np.einsum("bhsd,bhsd->bhs", q, k), 1e-13, "window 0,0 LSE")


def pin_varlen_is_per_sequence(lib):
    """Packed sequences give, row for row, the dense result of each sequence on
    its own (empty sequences included), with GQA heads and a window."""
    H, H_kv, D = 4, 2, 8
    lens = [5, 0, 17, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    total = int(cu[-1])
    q, k, v = _rand(101, (total, H, D)), _rand(102, (total, H_kv, D)), _rand(103, (total, H_kv, D))
    for window in ((-1, -1), (-1, 0), (2, 1)):
        O, L = oracle.attention_varlen(q, k, v, cu, 0.25, window=window, lib=lib)
        for s, (a, e) in enumerate(zip(cu, cu[1:])):
            if e == a:
                continue
            qs = np.ascontiguousarray(q[a:e].transpose(1, 0, 2))[None]
            ks = np.ascontiguousarray(np.repeat(k[a:e], H // H_kv, axis=1).transpose(1, 0, 2))[None]
            vs = np.ascontiguousarray(np.repeat(v[a:e], H // H_kv, axis=1).transpose(1, 0, 2))[None]
            s_ = 0.25 * (qs @ np.swapaxes(ks, -1, -2))
            s_ = np.where(_band_mask(e - a, *window), s_, -np.inf)
            _close(O[a:e], (softmax(s_, axis=-1) @ vs)[0].transpose(1, 0, 2), 1e-12, f"varlen seq {s} O {window}")
            _close(L[:, a:e], logsumexp(s_, axis=-1)[0], 1e-12, f"varlen seq {s} LSE {window}")


def _keep_mask(S, bh, seed, offset, thr, lib):
    """z_ij from the generator: 16-bit draw (j mod 8) of Philox(j // 8, i, bh,
    offset), draw t being bits 16*(t % 2) of word t // 2, compared with thr."""
    z = np.zeros((S, S))
    for i in range(S):
        for j8 in range((S + 7) // 8):
            r = oracle.philox4x32_10([j8, i, bh, offset], [seed & 0xFFFFFFFF, seed >> 32], lib=lib)
            for t in range(8):
                if 8 * j8 + t < S:
                    draw = (r[t // 2] >> (16 * (t % 2))) & 0xFFFF
                    z[i, 8 * j8 + t] = 1.0 if draw >= thr else 0.0
    return z


def pin_dropout_mask(lib):
    """Q = 0 and V = I (D = S): O_ij = P_ij z_ij / (1 - p) with P_ij = 1/n_i,
    so O exposes every keep decision z_ij, which must be the generator's, with
    the counter (j // 8, i, b*H + h, offset), 16-bit draw j % 8 and the key
    from the seed. LSE is that of the softmax before dropout."""
    B, H, S = 1, 2, 10
    q = np.zeros((B, H, S, S))
    k = _rand(111, (B, H, S, S))
    v = np.broadcast_to(np.eye(S), (B, H, S, S)).copy()
    p = float(np.float32(0.3))
    seed, offset = 0x1234_5678_9ABC_DEF0, 77
    thr = oracle.dropout_threshold(p)
    for wl, wr in ((-1, -1), (-1, 0)):
        ok = _band_mask(S, wl, wr).astype(np.float64)
        n = ok.sum(axis=1)
        O, L = oracle.attention_ex(q, k, v, 0.125, window=(wl, wr), dropout_p=p, seed=seed, offset=offset, lib=lib)
        for h in range(H):
            z = _keep_mask(S, h, seed, offset, thr, lib)
            _close(O[0, h], ok * z / (n[:, None] * (1.0 - p)), 1e-14, f"dropout mask head {h} window {wl},{wr}")
        _close(L, np.broadcast_to(np.log(n), (B, H, S)), 1e-13, f"dropout LSE unchanged window {wl},{wr}")


def pin_dropout_statistics(lib):
    """Over many offsets the keep rate is 1 - p (binomial, 6 sigma) and the
    dropped output is an unbiased estimate of the plain one (mean within 6
    standard errors of its own spread)."""
    B, H, S, D = 1, 1, 24, 4
    q, k, v = _rand(121, (B, H, S, D)), _rand(122, (B, H, S, D)), _rand(123, (B, H, S, D))
    p = float(np.float32(0.25))
    O0, L0 = oracle.attention_ex(q, k, v, 0.5, lib=lib)
    draws = []
    for off in range(300):
        O, L = oracle.attention_ex(q, k, v, 0.5, dropout_p=p, seed=99, offset=off, lib=lib)
        _close(L, L0, 0.0, "dropout leaves LSE unchanged")
        draws.append(O)
    draws = np.array(draws)
    mean, se = draws.mean(axis=0), draws.std(axis=0) / math.sqrt(len(draws))
    z = np.abs(mean - O0) / np.maximum(se, 1e-12)
    assert np.max(z) < 6.0, f"dropout output biased: max z-score {np.max(z):.2f}"
    n = 0
    kept = 0
    thr = oracle.dropout_threshold(p)
    for off in range(40):
        for i in range(8):
            for j8 in range(3):
                r = oracle.philox4x32_10([j8, i, 0, off], [99, 0], lib=lib)
                kept += sum(1 for w in r for half in (w & 0xFFFF, w >> 16) if half >= thr)
                n += 8
    sigma = math.sqrt(n * p * (1 - p))
    assert abs(kept - n * (1 - p)) < 6 * sigma, f"keep rate {kept / n:.4f} vs {1 - p}"


def pin_dropout_off(lib):
    """p = 0 is the plain definition, whatever the seed."""
    B, H, S, D = 1, 2, 13, 8
    q, k, v = _rand(131, (B, H, S, D)), _rand(132, (B, H, S, D)), _rand(133, (B, H, S, D))
    for causal in (False, True):
        O0, L0 = oracle.attention(q, k, v, causal, 0.2, lib=lib)
        O1, L1 = oracle.attention_ex(q, k, v, 0.2, window=(-1, 0 if causal else -1), dropout_p=0.0, seed=5,
                                     offset=3, lib=lib)
        _close(O1, O0, 0.0, "p=0 O")
        _close(L1, L0, 0.0, "p=0 LSE")


ALL_PINS += [pin_philox_known_answers, pin_window_uniform, pin_window_library_softmax, pin_window_zero,
             pin_varlen_is_per_sequence, pin_dropout_mask, pin_dropout_statistics, pin_dropout_off]
