"""Test infrastructure only: an fp64 model of the tiled online softmax.

This is not the oracle (that is the plain definition in ``attn_oracle.c``); it
is the FlashAttention-2 recurrence written out step by step, so a test can show
that the recurrence reaches the plain definition for any key-tile width BN.
That is the algebra the GPU kernel relies on.

Steps, from the page "CuTe 详解：以 FlashAttention-2 拆解 Layout、TiledCopy 与
TiledMMA", §"沿 C fragment 做 Online Softmax" (its three update equations and
the closing paragraph), in that order, per query row and per key tile t:

    m_t   = max of the tile's raw scores q_i . k_j (masked keys count as -inf)
    m_new = max(m_old, m_t)
    alpha = e^{scale (m_old - m_new)}
    p_j   = e^{scale (s_j - m_new)}
    l_new = alpha l_old + sum_j p_j
    o_new = alpha o_old + sum_j p_j v_j

and after the last tile O = o / l (§"教学配置：一块 CTA 做什么"). The max is
taken on raw scores and the positive scale applied afterwards, as that section
allows for scale > 0. LSE = scale*m + ln l.

Where the page is silent (a tile in which a row has no admissible key), m_new
stays -inf and this model uses alpha = 1, p = 0 for that row, which is the
limit of the formulas; the kernel reaches the same result.
"""
from __future__ import annotations

import numpy as np


def online_attention(q, k, v, causal: bool, scale: float, BN: int):
    """O [B,H,S,D] and LSE [B,H,S] in float64 via the tiled recurrence."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, S, D = q.shape
    O = np.empty((B, H, S, D))
    LSE = np.empty((B, H, S))
    rows = np.arange(S)[:, None]
    for b in range(B):
        for h in range(H):
            m = np.full(S, -np.inf)
            l = np.zeros(S)
            o = np.zeros((S, D))
            for k0 in range(0, S, BN):
                kt, vt = k[b, h, k0:k0 + BN], v[b, h, k0:k0 + BN]
                raw = q[b, h] @ kt.T                      # [S, n] raw scores
                if causal:
                    cols = np.arange(k0, k0 + kt.shape[0])[None, :]
                    raw = np.where(cols <= rows, raw, -np.inf)
                m_t = raw.max(axis=1)
                m_new = np.maximum(m, m_t)
                live = np.isfinite(m_new)
                alpha = np.where(live, np.exp(scale * (m - np.where(live, m_new, 0.0))), 1.0)
                p = np.where(live[:, None],
                             np.exp(scale * (raw - np.where(live, m_new, 0.0)[:, None])), 0.0)
                l = alpha * l + p.sum(axis=1)
                o = alpha[:, None] * o + p @ vt
                m = m_new
            O[b, h] = o / l[:, None]
            LSE[b, h] = scale * m + np.log(l)
    return O, LSE
