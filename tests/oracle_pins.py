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
