"""GPU parity over a seeded random sweep of valid arguments, through both
extended entry points (dense fa2_fwd_ex and packed fa2_fwd_varlen), against
the fp64 oracle with the tolerances of the other parity tests.

Each case draws, from its own seed: the head dimension, the numbers of query
and K/V heads (GQA group 1-4), dense [B,H,S,D] or packed sequences (some of
them empty), the mask (none, causal, or a local window with either side
possibly unbounded), dropout (off, or p in (0, 0.6) with a random seed and
offset) and the softmax scale. The sweep covers combinations the targeted
tests do not enumerate one by one."""
import numpy as np
import pytest

import oracle
from fa2_inputs import make_packed, make_random
from test_parity_features import check, eff_window, gpu_ex, gpu_varlen, log

pytestmark = pytest.mark.gpu

N_CASES = 400
# Seeds beyond the sweep whose outputs (D = 128, p = 0.48-0.59, |O| up to 8.9) exceed the unscaled
# O bound and meet the dropout-scaled one: kept to hold that bound to the cases that need it.
HIGH_DROPOUT = [939, 1589, 1646, 1825, 1893]


def sweep_case(i: int) -> dict:
    g = np.random.Generator(np.random.PCG64(90_000 + i))
    D = int(g.choice([64, 128]))
    H_kv = int(g.integers(1, 4))
    H = H_kv * int(g.integers(1, 5))
    mask = str(g.choice(["none", "causal", "window"]))
    window = None
    if mask == "window":
        wl = -1 if g.random() < 0.25 else int(g.integers(0, 600))
        wr = -1 if g.random() < 0.25 else (0 if g.random() < 0.2 else int(g.integers(0, 600)))
        window = (wl, wr)
    p = 0.0 if g.random() < 0.6 else float(np.float32(g.uniform(0.01, 0.6)))
    case = {"i": i, "D": D, "H": H, "H_kv": H_kv, "causal": mask == "causal", "window": window, "p": p,
            "seed": int(g.integers(0, 2**63)), "offset": int(g.integers(0, 2**32)),
            "scale": float(np.float32(g.uniform(0.04, 0.3))), "packed": bool(g.random() < 0.35)}
    if case["packed"]:
        n = int(g.integers(1, 6))
        lens = np.where(g.random(n) < 0.15, 0, g.integers(1, 700, size=n))
        if lens.sum() == 0:
            lens[0] = 1
        case["lens"] = [int(x) for x in lens]
    else:
        case["B"] = int(g.integers(1, 4))
        case["S"] = int(g.integers(1, 800))
    return case


def case_id(i: int) -> str:
    c = sweep_case(i)
    shape = f"lens{c['lens']}" if c["packed"] else f"B{c['B']}S{c['S']}"
    mask = "causal" if c["causal"] else (f"win{c['window'][0]}_{c['window'][1]}" if c["window"] else "plain")
    return f"{i}-D{c['D']}-H{c['H']}kv{c['H_kv']}-{shape}-{mask}-p{c['p']:.2f}".replace(" ", "")


CASES = list(range(N_CASES)) + HIGH_DROPOUT


@pytest.mark.parametrize("i", CASES, ids=[case_id(i) for i in CASES])
def test_sweep(i):
    c = sweep_case(i)
    log(f"case sweep {case_id(i)} scale={c['scale']} seed={c['seed']} offset={c['offset']}")
    win = eff_window(c["causal"], c["window"])
    if c["packed"]:
        q, k, v, cu = make_packed(91_000 + 7 * i, c["lens"], c["H"], c["H_kv"], c["D"])
        O, L = gpu_varlen(q, k, v, cu, c["causal"], c["window"], c["p"], c["seed"], c["offset"], c["scale"])
        Oref, Lref = oracle.attention_varlen(q, k, v, cu, c["scale"], window=win, dropout_p=c["p"],
                                             seed=c["seed"], offset=c["offset"])
    else:
        q, _, _ = make_random(92_000 + 7 * i, c["B"], c["H"], c["S"], c["D"])
        _, k, v = make_random(93_000 + 7 * i, c["B"], c["H_kv"], c["S"], c["D"])
        O, L = gpu_ex(q, k, v, c["causal"], c["window"], c["p"], c["seed"], c["offset"], c["scale"])
        Oref, Lref = oracle.attention_ex(q, k, v, c["scale"], window=win, dropout_p=c["p"], seed=c["seed"],
                                         offset=c["offset"])
    check(O, L, Oref, Lref, f"sweep {i}", c["p"])
