"""The fp64 oracle against its pins (closed forms, worked examples, invariants,
a library route and brute force). See tests/oracle_pins.py for each fact's
source on the FlashAttention-2 page."""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(lib, pin):
    pin(lib)


def _brute(q, k, v, causal, scale):
    """Pure-Python attention with math.fsum, for shapes of a few elements."""
    S, D = len(q), len(q[0])
    O, L = [], []
    for i in range(S):
        keys = range(i + 1) if causal else range(S)
        s = [scale * math.fsum(q[i][d] * k[j][d] for d in range(D)) for j in keys]
        M = max(s)
        w = [math.exp(x - M) for x in s]
        tot = math.fsum(w)
        O.append([math.fsum(wj * v[j][d] for wj, j in zip(w, keys)) / tot for d in range(D)])
        L.append(M + math.log(tot))
    return O, L


@settings(max_examples=60, deadline=None)
@given(S=st.integers(1, 6), D=st.integers(1, 4), causal=st.booleans(),
       seed=st.integers(0, 2**31 - 1), scale=st.floats(0.01, 4.0))
def test_bruteforce_tiny(S, D, causal, seed, scale):
    g = np.random.Generator(np.random.PCG64(seed))
    q, k, v = (g.standard_normal((1, 1, S, D)) * 2 for _ in range(3))
    O, L = oracle.attention(q, k, v, causal, scale)
    Ob, Lb = _brute(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), causal, scale)
    assert np.max(np.abs(O[0, 0] - np.array(Ob))) <= 1e-12
    assert np.max(np.abs(L[0, 0] - np.array(Lb))) <= 1e-12


def test_rows_equal_full(lib):
    """The sampled-row entry point evaluates the same definition bit for bit."""
    g = np.random.Generator(np.random.PCG64(5))
    q, k, v = ((g.standard_normal((2, 3, 41, 16))).astype(np.float16) for _ in range(3))
    rows = np.array([0, 1, 40, 41, 100, 245, 2 * 3 * 41 - 1])
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, causal, 0.125)
        Or, Lr = oracle.attention_rows(q, k, v, causal, 0.125, rows)
        assert np.array_equal(Or, O.reshape(-1, 16)[rows])
        assert np.array_equal(Lr, L.reshape(-1)[rows])


def test_rejects_bad_arguments(lib):
    q = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        oracle.attention(q, q[:, :, :3], q, False, 1.0)
    with pytest.raises(RuntimeError):
        oracle.attention_rows(q, q, q, False, 1.0, [4])
