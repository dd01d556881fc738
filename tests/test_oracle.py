"""The fp64 oracle against its pins, and a mutation test of the pins.

CPU only. See ``oracle_pins.py`` for what each pin checks and why it is
independent of the oracle's own code.
"""
import os
import shutil

import pytest

import oracle
from tests import oracle_pins

pytestmark = pytest.mark.cpu


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# Plausible mistakes planted in a copy of the oracle's C source. Each one must
# make at least one pin fail; a mutant no pin catches would mean a hole in the
# pins.
MUTANTS = {
    "exp_sign_flipped": ("e[j] = exp(s[j] - m);", "e[j] = exp(m - s[j]);"),
    "no_normalisation": ("const double p = e[j] / L;", "const double p = e[j];"),
    "causal_off_by_one": ("n = i + (Skv - Sq) + 1;", "n = i + (Skv - Sq);"),
    "causal_top_left": ("n = i + (Skv - Sq) + 1;", "n = i + 1;"),
    "gqa_modulo_mapping": ("const int g = (int)((long)h * Hkv / Hq);\n      const double* kb",
                           "const int g = (int)(h % Hkv);\n      const double* kb"),
    "scale_dropped": ("s[j] = scale * dot(qi, kb + (size_t)j * d, d);", "s[j] = dot(qi, kb + (size_t)j * d, d);"),
    "keys_reversed": ("s[j] = scale * dot(qi, kb + (size_t)j * d, d);",
                      "s[j] = scale * dot(qi, kb + (size_t)(n - 1 - j) * d, d);"),
    "dot_transposed": ("acc += a[c] * b[c];", "acc += a[c] * b[d - 1 - c];"),
    "lse_missing_log": ("return m + log(L);", "return m + L;"),
    "page_slot_wrong": ("* page + (size_t)(t % page);", "* page + (size_t)(t / page % page);"),
    "merge_unweighted": ("const double w = exp(ls[s] - M);", "const double w = 1.0;"),
    "merge_plain_sum": ("for (int c = 0; c < d; ++c) orow[c] /= W;", ""),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found for {name}"
    mutated = src.replace(old, new, 1)
    csrc = os.path.join(tmp_path, f"mut_{name}.c")
    with open(csrc, "w") as f:
        f.write(mutated)
    lib = oracle.build(force=True, src=csrc, out=os.path.join(tmp_path, f"libmut_{name}.so"))
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib=lib)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
