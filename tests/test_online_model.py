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
