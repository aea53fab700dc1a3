"""Every plausible mistake planted in a copy of the oracle's C source breaks at
least one pin, so the pins are strong enough to trust the oracle.

Each mutant is a text substitution applied to a temporary copy of
oracle/attn_oracle.c, compiled with the oracle's own flags and loaded in place
of the real library. All of this runs on the CPU."""
import os
import shutil
import subprocess

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

MUTANTS = {
    "scale dropped": ("s[t] = scale * dot;", "s[t] = dot;"),
    "scale applied twice": ("s[t] = scale * dot;", "s[t] = scale * scale * dot;"),
    "window right bound one short (causal admits one key fewer)": ("*hi = i + wr;", "*hi = i + wr - 1;"),
    "window right bound one long (causal admits one key more)": ("*hi = i + wr;", "*hi = i + wr + 1;"),
    "window left bound one short": ("*lo = i - wl;", "*lo = i - wl + 1;"),
    "window left bound one long": ("if (wl >= 0 && i - wl > 0)\n        *lo = i - wl;",
                                   "if (wl >= 0 && i - wl > 1)\n        *lo = i - wl - 1;"),
    "window sides swapped": ("key_range(S, i, wl, wr, &lo, &hi);", "key_range(S, i, wr, wl, &lo, &hi);"),
    "mask ignored": ("causal ? 0 : -1", "-1"),
    "query/key swapped in score": ("attend_row(q + base + i * D, k + base", "attend_row(k + base + i * D, k + base"),
    "key index is the query index": ("const double *kj = k + (lo + t) * D;", "const double *kj = k + i * D;"),
    "value from the query row": ("acc += p[t] * v[(lo + t) * D + d];", "acc += p[t] * v[i * D + d];"),
    "value transposed": ("acc += p[t] * v[(lo + t) * D + d];",
                         "acc += p[t] * v[(d * D + lo + t) % ((hi + 1) * D)];"),
    "no normalisation": ("p[t] = exp(s[t] - M) / l;", "p[t] = exp(s[t] - M);"),
    "max not subtracted in P": ("p[t] = exp(s[t] - M) / l;", "p[t] = exp(s[t]) / l;"),
    "LSE without max": ("*lse_out = M + log(l);", "*lse_out = log(l);"),
    "LSE in base 2": ("*lse_out = M + log(l);", "*lse_out = M + log2(l);"),
    "LSE of the max only": ("*lse_out = M + log(l);", "*lse_out = M;"),
    "min instead of max": ("if (s[t] > M)", "if (s[t] < M)"),
    "first key dropped from the sum": ("for (long long t = 0; t < n_keys; ++t)\n        l += exp",
                                       "for (long long t = 1; t < n_keys; ++t)\n        l += exp"),
    "last head dim dropped": ("for (long long d = 0; d < D; ++d)\n            dot +=",
                              "for (long long d = 0; d + 1 < D; ++d)\n            dot +="),
    "wrong head base": ("const long long base = head * (long long)S * D;",
                        "const long long base = (head / 2) * (long long)S * D;"),
    "dropout ignored": ("if (dc && dc->on)", "if (0)"),
    "dropout not rescaled": ("p[t] * dc->keep_scale : 0.0", "p[t] : 0.0"),
    "dropout keeps the draws below the threshold": ("return draw >= dc->thr;", "return draw < dc->thr;"),
    "dropout reads the wrong word": ("r[t / 2] >> (16 * (t % 2))", "r[(t / 2 + 1) % 4] >> (16 * (t % 2))"),
    "dropout reads the wrong half of a word": ("r[t / 2] >> (16 * (t % 2))", "r[t / 2] >> (16 * (1 - t % 2))"),
    "dropout draws 32-bit": ("& 0xFFFFu;", "& 0xFFFFFFFFu;"),
    "dropout counter with query and key swapped": ("{(uint32_t)(j / 8), (uint32_t)i,", "{(uint32_t)(i / 8), (uint32_t)j,"),
    "dropout counter groups of four keys": ("{(uint32_t)(j / 8), (uint32_t)i,", "{(uint32_t)(j / 4), (uint32_t)i,"),
    "dropout counter without the head": ("(uint32_t)i, dc->bh, dc->offset}", "(uint32_t)i, 0u, dc->offset}"),
    "dropout counter without the offset": ("(uint32_t)i, dc->bh, dc->offset}", "(uint32_t)i, dc->bh, 0u}"),
    "dropout removes dropped weight from the normaliser": (
        "p[t] = kept(dc, i, lo + t) ? p[t] * dc->keep_scale : 0.0;",
        "{ if (!kept(dc, i, lo + t)) l -= p[t] * l; p[t] = kept(dc, i, lo + t) ? p[t] * dc->keep_scale : 0.0; }"),
    "Philox with one round fewer": ("round < 10", "round < 9"),
    "Philox key schedule constants swapped": ("k0 += weyl0;", "k0 += weyl1;"),
    "Philox key bumped before the first round": ("if (round > 0) {", "if (round >= 0) {"),
    "Philox products swapped": ("(uint32_t)(prod1 >> 32) ^ x[1] ^ k0", "(uint32_t)(prod0 >> 32) ^ x[1] ^ k0"),
    "Philox output words reordered": ("(uint32_t)prod1,\n", "(uint32_t)prod0 ^ 1u,\n"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation site not found: {old!r}"
    mutated = text.replace(old, new)
    src = tmp_path / "mutant.c"
    src.write_text(mutated)
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build(str(src), lib_path)
    lib = oracle.load(lib_path)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError) as e:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the mutant '{name}'"
