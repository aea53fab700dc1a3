"""The FlashAttention-2 online-softmax recurrence reaches the plain definition
for every key-tile width: the algebra the kernel relies on (the update
equations of §"沿 C fragment 做 Online Softmax" on the page "CuTe 详解：以
FlashAttention-2 拆解 Layout、TiledCopy 与 TiledMMA", including the rescale of
the old output that the page warns must not be skipped)."""
import numpy as np
import pytest

import oracle
from fa2_inputs import make_random
from oracle.online_model import online_attention


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("BN", [1, 3, 16, 64, 77])
def test_online_equals_definition(causal, BN):
    q, k, v = make_random(900, 2, 2, 77, 16, sigma_qk=3.0)
    O, L = oracle.attention(q, k, v, causal, 0.125)
    Om, Lm = online_attention(q, k, v, causal, 0.125, BN)
    assert np.max(np.abs(Om - O)) <= 1e-12
    assert np.max(np.abs(Lm - L)) <= 1e-12


def test_skipping_the_rescale_breaks_it():
    """Without alpha * o_old the result depends on the tile boundaries, as the
    page states; the tests above would catch a kernel that forgot it."""
    q, k, v = make_random(901, 1, 1, 64, 8, sigma_qk=3.0)
    O, _ = oracle.attention(q, k, v, False, 0.125)
    qd, kd, vd = (x.astype(np.float64)[0, 0] for x in (q, k, v))
    raw = qd @ kd.T
    m = np.full(64, -np.inf)
    l = np.zeros(64)
    o = np.zeros((64, 8))
    for k0 in range(0, 64, 16):
        r = raw[:, k0:k0 + 16]
        m_new = np.maximum(m, r.max(axis=1))
        alpha = np.exp(0.125 * (m - m_new))
        p = np.exp(0.125 * (r - m_new[:, None]))
        l = alpha * l + p.sum(axis=1)
        o = o + p @ vd[k0:k0 + 16]          # the rescale of the old output is skipped
        m = m_new
    assert np.max(np.abs(o / l[:, None] - O[0, 0])) > 1e-3


# ---- the kernel's lazy reference (oracle.online_model.lazy_reference_attention) ----

from oracle.online_model import lazy_reference_attention  # noqa: E402

# The kernel sets the reference 8 base-2 units above the tile maximum at each
# rebase (so probabilities are at most 2^-8 right after it).
KERNEL_HEADROOM = 8.0


def _ramp(direction, S=515, D=64, H=2, seed=902):
    """Scores that rise (or fall) by about 180 base-2 units per 64 keys at
    scale 1: rising keys raise every row's maximum on every tile, falling ones
    never after the first."""
    q = np.zeros((1, H, S, D), np.float16)
    k = np.zeros((1, H, S, D), np.float16)
    q[..., 0] = 4.0
    ramp = (np.arange(S) * 0.5).astype(np.float16)
    k[0, :, :, 0] = ramp if direction == "rising" else ramp[::-1]
    _, _, v = make_random(seed, 1, H, S, D)
    return q, k, v


def _cases():
    yield "sigma3", make_random(903, 1, 2, 300, 64, sigma_qk=3.0), 0.125
    yield "sigma1", make_random(904, 2, 1, 257, 64), 0.125
    yield "rising", _ramp("rising"), 1.0
    yield "falling", _ramp("falling"), 1.0


LAZY_CASES = list(_cases())


@pytest.mark.parametrize("headroom", [0.0, KERNEL_HEADROOM])
@pytest.mark.parametrize("window", [(-1, -1), (-1, 0), (40, 7)], ids=["plain", "causal", "window"])
@pytest.mark.parametrize("BN,group", [(64, 32), (64, 1), (16, 32), (77, 16)])
@pytest.mark.parametrize("name,qkv,scale", LAZY_CASES, ids=[c[0] for c in LAZY_CASES])
def test_lazy_reference_is_exact_algebra(name, qkv, scale, BN, group, window, headroom):
    """Without fp16 rounding of p, keeping the reference lazily reaches the
    plain definition to rounding (the common reference of o and l cancels):
    the algebra the kernel's rule relies on, for several tile widths and row
    groupings."""
    q, k, v = qkv
    O, L = oracle.attention_ex(q, k, v, scale, window=window)
    Om, Lm, _ = lazy_reference_attention(q, k, v, False, scale, BN, group, p_fp16=False, window=window,
                                         headroom=headroom)
    assert np.max(np.abs(Om - O)) <= 1e-12
    assert np.max(np.abs(Lm - L) / np.maximum(1.0, np.abs(L))) <= 1e-12


@pytest.mark.parametrize("window", [(-1, -1), (-1, 0), (40, 7)], ids=["plain", "causal", "window"])
@pytest.mark.parametrize("name,qkv,scale", LAZY_CASES, ids=[c[0] for c in LAZY_CASES])
def test_lazy_reference_with_fp16_p_meets_the_tolerances(name, qkv, scale, window):
    """With p rounded to fp16 (the operand of the PV product, and what l sums),
    the kernel's rule at its tiling (64-key tiles, 32-row waves) stays within
    the parity tolerances of the GPU tests: max |dO| <= 4e-3,
    mean |dO| <= 5e-4, max |dLSE| <= 1e-3."""
    q, k, v = qkv
    O, L = oracle.attention_ex(q, k, v, scale, window=window)
    Om, Lm, _ = lazy_reference_attention(q, k, v, False, scale, 64, 32, p_fp16=True, window=window,
                                         headroom=KERNEL_HEADROOM)
    dO = np.abs(Om - O)
    assert np.all(np.isfinite(Om)) and np.all(np.isfinite(Lm))
    assert dO.max() <= 4e-3 and dO.mean() <= 5e-4
    assert np.max(np.abs(Lm - L)) <= 1e-3


def test_lazy_reference_moves_only_when_needed():
    """Falling keys: only the first tile of each row group rebases. Rising
    keys: every tile does (each raises the maximum by about 180 base-2 units,
    far past 2^15). iid N(0,1) inputs at scale 1/8: almost never after the
    first tile."""
    S = 576
    tiles = S // 64
    _, _, reb = lazy_reference_attention(*_ramp("falling", S=S), False, 1.0, 64, 32)
    assert np.all(reb == 1)
    _, _, reb = lazy_reference_attention(*_ramp("rising", S=S), False, 1.0, 64, 32)
    assert np.all(reb == tiles)
    # a ragged last tile of 3 keys raises the maximum by only 3 keys' worth
    # (about 8.7 base-2 units), which fp16 holds: it is accepted without a rebase
    _, _, reb = lazy_reference_attention(*_ramp("rising", S=515), False, 1.0, 64, 32)
    assert np.all(reb == 8)
    q, k, v = make_random(905, 1, 2, 1024, 64)
    _, _, reb = lazy_reference_attention(q, k, v, False, 0.125, 64, 32)
    assert reb.mean() < 1.5


def test_lazy_reference_check_is_what_keeps_p_finite():
    """Accepting every tile after the first (no row-sum check) lets p overflow
    fp16 on rising keys, and the output is no longer finite: the check is
    load-bearing. With the check the same inputs match the definition."""
    q, k, v = _ramp("rising")
    Om, _, _ = lazy_reference_attention(q, k, v, False, 1.0, 64, 32, check=False)
    assert not np.all(np.isfinite(Om))
    O, _ = oracle.attention(q, k, v, False, 1.0)
    Om, _, _ = lazy_reference_attention(q, k, v, False, 1.0, 64, 32, check=True)
    assert np.max(np.abs(Om - O)) <= 4e-3


def test_lazy_reference_check_catches_an_infinite_p():
    """A p that overflows fp16 becomes +inf and so does its row sum, which
    fails the check whatever the limit: 2^15 (the kernel's, which also keeps
    every accepted p below 2^15) and even an infinite limit give results
    within the tolerances on rising keys; only dropping the check fails."""
    q, k, v = _ramp("rising")
    O, L = oracle.attention(q, k, v, False, 1.0)
    for limit in (2.0 ** 15, float("inf")):
        Om, Lm, _ = lazy_reference_attention(q, k, v, False, 1.0, 64, 32, limit=limit)
        assert np.max(np.abs(Om - O)) <= 4e-3
        assert np.max(np.abs(Lm - L)) <= 1e-3


def test_reference_headroom_halves_rebases_of_peaked_rows():
    """Scores with a standard deviation of about 13 base-2 units (Q, K ~ N(0, 3^2),
    D = 64, scale 1/8) keep raising the row maximum over 1000 keys: with the
    reference at the tile maximum each 32-row group rebases about 4.4 times,
    with it 8 units above about 2.0 times, and the result stays within the
    parity tolerances; with 12 or more units the fp16 subnormal range starts
    to cost accuracy, which is why the kernel stops at 8."""
    q, k, v = make_random(906, 1, 4, 1000, 64, sigma_qk=3.0)
    O, L = oracle.attention(q, k, v, False, 0.125)
    res = {}
    for hr in (0.0, KERNEL_HEADROOM, 14.0):
        Om, Lm, reb = lazy_reference_attention(q, k, v, False, 0.125, 64, 32, headroom=hr)
        res[hr] = (reb.mean(), np.abs(Om - O).max(), np.abs(Lm - L).max())
    assert res[KERNEL_HEADROOM][0] < 0.6 * res[0.0][0]
    assert res[KERNEL_HEADROOM][1] <= 4e-3 and res[KERNEL_HEADROOM][2] <= 1e-3
    assert res[14.0][1] > 2 * res[KERNEL_HEADROOM][1]
