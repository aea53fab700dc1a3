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

``lazy_reference_attention`` is the same recurrence with the reference moved
only when needed, the rule the GPU kernel follows (fp16 probabilities, a row
sum check against 2^15, rebase on failure); its docstring states the steps.
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


def lazy_reference_attention(q, k, v, causal: bool, scale: float, BN: int, rows_per_group: int = 32,
                             p_fp16: bool = True, check: bool = True, limit: float = 2.0 ** 15,
                             window=(-1, -1), headroom: float = 0.0):
    """The recurrence above with the reference kept lazily, as the GPU kernel
    runs it. Returns O [B,H,S,D], LSE [B,H,S] (float64) and the number of
    rebases per (b, h, row group).

    The page's update moves m to the new row maximum on every tile. Any common
    reference of o and l gives the same O = o / l and LSE = scale*m + ln l in
    exact arithmetic, so the only requirement on it is that every probability
    stays representable once rounded to fp16. Per key tile of BN keys and per
    group of ``rows_per_group`` query rows (a wave of the kernel owns 32 rows
    and takes one decision for all of them):

      1. the group's first tile always rebases (step 3);
      2. otherwise p = 2^(s*c - m*c) against the current reference, with
         c = scale*log2(e), each p rounded to fp16 (round to nearest even,
         overflow to +inf) when ``p_fp16``; the tile is accepted when every
         row's sum of those p is below ``limit`` (2^15), so that no single p
         overflowed fp16 (largest finite 65504);
      3. else (rebase): m_new = max(m, tile row max), o and l are scaled by
         alpha = 2^((m - m_new)*c), and p is recomputed against m_new;
      4. l += sum_j p_j and o += sum_j p_j v_j, over the same (rounded) p.

    The reference starts at the finite value -1e30 (base-2 units), so a row
    whose keys are all masked so far has alpha = 1 and p = 0. With
    ``check=False`` step 2 accepts every tile (used to show that the check is
    what keeps p finite). ``window`` is (left, right) with -1 unbounded;
    ``causal`` is the same as (-1, 0). ``headroom`` (base-2 units, >= 0) sets
    the reference that far above the tile maximum at each rebase, so that
    later tiles may rise 15 + headroom units before p overflows; the
    probabilities are then at most 2^-headroom."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, S, D = q.shape
    c = scale * np.log2(np.e)
    wl, wr = window
    if causal:
        wl, wr = -1, 0
    cols_all = np.arange(S)[None, :]
    rows_all = np.arange(S)[:, None]
    admissible = np.ones((S, S), dtype=bool)
    if wl >= 0:
        admissible &= cols_all >= rows_all - wl
    if wr >= 0:
        admissible &= cols_all <= rows_all + wr

    def expo(x):
        with np.errstate(over="ignore"):
            p = np.exp2(x)
            if p_fp16:
                p = p.astype(np.float16).astype(np.float64)
        return p

    O = np.empty((B, H, S, D))
    LSE = np.empty((B, H, S))
    ngroups = -(-S // rows_per_group)
    rebases = np.zeros((B, H, ngroups), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            raw_all = q[b, h] @ k[b, h].T
            for gi in range(ngroups):
                r0, r1 = gi * rows_per_group, min(S, (gi + 1) * rows_per_group)
                mc = np.full(r1 - r0, -1.0e30)     # reference times c
                l = np.zeros(r1 - r0)
                o = np.zeros((r1 - r0, D))
                fresh = True
                for k0 in range(0, S, BN):
                    k1 = min(S, k0 + BN)
                    adm = admissible[r0:r1, k0:k1]
                    if not adm.any():
                        continue                    # the kernel skips tiles outside every row's band
                    s = np.where(adm, raw_all[r0:r1, k0:k1], -np.inf)
                    accept = False
                    if not fresh:
                        p = expo(s * c - mc[:, None])
                        rs = p.sum(axis=1)
                        accept = (not check) or bool(np.all(rs < limit))
                    if not accept:
                        m_new = np.maximum(mc, s.max(axis=1) * c + headroom)
                        alpha = np.exp2(mc - m_new)
                        o *= alpha[:, None]
                        l *= alpha
                        mc = m_new
                        p = expo(s * c - mc[:, None])
                        rebases[b, h, gi] += 1
                    fresh = False
                    l += p.sum(axis=1)
                    o += p @ v[b, h, k0:k1]
                with np.errstate(invalid="ignore", divide="ignore"):
                    O[b, h, r0:r1] = o / l[:, None]
                    LSE[b, h, r0:r1] = (mc + np.log2(l)) * np.log(2.0)
    return O, LSE, rebases
