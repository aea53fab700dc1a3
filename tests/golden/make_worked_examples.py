"""Writes the worked attention examples in this folder from their closed forms.

The FlashAttention-2 page ("CuTe 详解：以 FlashAttention-2 拆解 Layout、TiledCopy
与 TiledMMA", §"先看全局：FA2 中的数据究竟去了哪里") defines the computation as
S = Q Kᵀ (times the softmax scale), P = row softmax of S, O = P V, and names a
log-sum-exp output (§"与官方 FA2 比较时，先对齐契约"); it prints no numerical
example. The two cases below are small enough to solve by hand. This script
evaluates those hand derivations (exact fractions, e and ln) and calls neither
the oracle nor the GPU library.

Run from the repository root:  python tests/golden/make_worked_examples.py
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))


def worked_2x2():
    # Q = K = I2, V = [[1,2],[3,4]], scale 1. Row 0 scores are (1, 0), row 1 (0, 1).
    # Row 0: weights e/(e+1), 1/(e+1)  -> O = v0 + (v1 - v0)/(e+1) = [1 + 2/(e+1), 2 + 2/(e+1)]
    # Row 1: weights 1/(e+1), e/(e+1)  -> O = v1 - (v1 - v0)/(e+1) = [3 - 2/(e+1), 4 - 2/(e+1)]
    # LSE of both rows: ln(e^1 + e^0) = ln(e + 1).
    # Causal: row 0 sees key 0 only -> O = v0 = [1, 2], LSE = s00 = 1; row 1 sees both keys.
    e = math.e
    t = 2.0 / (e + 1.0)
    nc_O = [[1.0 + t, 2.0 + t], [3.0 - t, 4.0 - t]]
    nc_L = [math.log(e + 1.0)] * 2
    c_O = [[1.0, 2.0], [3.0 - t, 4.0 - t]]
    c_L = [1.0, math.log(e + 1.0)]
    return {
        "citation": "definition S=QK^T*scale, P=softmax(S), O=PV and the LSE output: "
                    "CuTe 详解：以 FlashAttention-2 拆解 Layout、TiledCopy 与 TiledMMA, "
                    "§先看全局 and §与官方 FA2 比较时，先对齐契约; values derived by hand",
        "closed_form": {
            "noncausal_O": "[[1+2/(e+1), 2+2/(e+1)], [3-2/(e+1), 4-2/(e+1)]]",
            "noncausal_LSE": "[ln(e+1), ln(e+1)]",
            "causal_O": "[[1, 2], [3-2/(e+1), 4-2/(e+1)]]",
            "causal_LSE": "[1, ln(e+1)]",
        },
        "scale": 1.0,
        "q": [[1.0, 0.0], [0.0, 1.0]],
        "k": [[1.0, 0.0], [0.0, 1.0]],
        "v": [[1.0, 2.0], [3.0, 4.0]],
        "noncausal": {"O": nc_O, "LSE": nc_L},
        "causal": {"O": c_O, "LSE": c_L},
    }


def worked_4x4():
    # D = 1, scale = ln 2, so each weight e^{scale*q_i*k_j} is 2^{q_i*k_j}.
    # q = [0,1,1,2], k = [0,1,2,3], v = [1,2,3,4].
    q, k, v = [0, 1, 1, 2], [0, 1, 2, 3], [1, 2, 3, 4]
    out = {}
    for causal in (False, True):
        Os, Ls = [], []
        for i in range(4):
            keys = range(i + 1) if causal else range(4)
            w = [Fraction(2) ** (q[i] * k[j]) for j in keys]
            total = sum(w)
            o = sum(wj * v[j] for wj, j in zip(w, keys)) / total
            Os.append(o)
            Ls.append(total)  # LSE = ln(total)
        out["causal" if causal else "noncausal"] = {
            "O_exact": [f"{x.numerator}/{x.denominator}" for x in Os],
            "O": [float(x) for x in Os],
            "LSE_is_ln_of": [f"{x.numerator}/{x.denominator}" for x in Ls],
            "LSE": [math.log(float(x)) for x in Ls],
        }
    return {
        "citation": "definition S=QK^T*scale, P=softmax(S), O=PV and the LSE output: "
                    "CuTe 详解：以 FlashAttention-2 拆解 Layout、TiledCopy 与 TiledMMA, "
                    "§先看全局 and §与官方 FA2 比较时，先对齐契约; values derived by hand",
        "note": "weights are 2^(q_i k_j) because scale = ln 2; every input is exact in fp16",
        "scale": math.log(2.0),
        "q": q, "k": k, "v": v,
        **out,
    }


def main():
    for name, data in (("worked_2x2.json", worked_2x2()), ("worked_4x4.json", worked_4x4())):
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(data, f, indent=1, ensure_ascii=False)
            f.write("\n")


if __name__ == "__main__":
    main()
