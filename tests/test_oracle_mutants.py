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
    "scale dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "scale applied twice": ("s[j] = scale * dot;", "s[j] = scale * scale * dot;"),
    "causal admits one key fewer": ("causal ? i + 1 : S", "causal ? i : S"),
    "causal admits one key more": ("causal ? i + 1 : S", "causal ? (i + 2 < S ? i + 2 : S) : S"),
    "mask ignored": ("causal ? i + 1 : S", "S"),
    "query/key swapped in score": ("const double *qi = q + i * D;", "const double *qi = k + i * D;"),
    "key index is the query index": ("const double *kj = k + j * D;", "const double *kj = k + i * D;"),
    "value from the query row": ("acc += p[j] * v[j * D + d];", "acc += p[j] * v[i * D + d];"),
    "value transposed": ("acc += p[j] * v[j * D + d];", "acc += p[j] * v[(d * D + j) % (S * D)];"),
    "no normalisation": ("p[j] = exp(s[j] - M) / l;", "p[j] = exp(s[j] - M);"),
    "max not subtracted in P": ("p[j] = exp(s[j] - M) / l;", "p[j] = exp(s[j]) / l;"),
    "LSE without max": ("*lse_out = M + log(l);", "*lse_out = log(l);"),
    "LSE in base 2": ("*lse_out = M + log(l);", "*lse_out = M + log2(l);"),
    "LSE of the max only": ("*lse_out = M + log(l);", "*lse_out = M;"),
    "min instead of max": ("if (s[j] > M)", "if (s[j] < M)"),
    "first key dropped from the sum": ("for (long long j = 0; j < n_keys; ++j)\n        l += exp",
                                       "for (long long j = 1; j < n_keys; ++j)\n        l += exp"),
    "last head dim dropped": ("for (long long d = 0; d < D; ++d)\n            dot +=",
                              "for (long long d = 0; d + 1 < D; ++d)\n            dot +="),
    "wrong head base": ("const long long base = head * (long long)S * D;",
                        "const long long base = (head / 2) * (long long)S * D;"),
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
