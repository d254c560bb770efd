"""The oracle pins must fail when a plausible mistake is planted in the
oracle.  Each case compiles a mutated copy of moe_oracle.c into a temporary
directory (the committed oracle is untouched), points the pins at it through
ORACLE_LIB and expects the pin suite to fail."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTATIONS = {
    "nibble order swapped": ("(byte & 0x0F) : (byte >> 4)", "(byte >> 4) : (byte & 0x0F)"),
    "scale block of 16": ("s_row[j / 32]", "s_row[j / 16]"),
    "activation not rounded": ("a[i] = mid ? oracle_bf16_round(v) : v;", "a[i] = v;"),
    "output not rounded": ("fin ? oracle_bf16_round(v) : v", "v"),
    "intermediates rounded under the output policy": (
        "const int mid = rounding == ORACLE_ROUND_BF16_ALL;",
        "const int mid = rounding != ORACLE_ROUND_NONE;"),
    "silu on the up half": ("double v = g * sigmoid(g) * u; /* silu",
                            "double v = u * sigmoid(u) * g; /* silu"),
    "routing weight dropped": ("ylat[l] += wsel[j] * ye[l]", "ylat[l] += ye[l]"),
    "bias sign flipped": ("s[e] + (bias ? (double)bias[e]", "s[e] - (bias ? (double)bias[e]"),
    "keys rounded to binary32": ("kb[e] = s[e] + (bias ? (double)bias[e] : 0.0);",
                                 "kb[e] = (float)(s[e] + (bias ? (double)bias[e] : 0.0));"),
    "shared expert dropped": ("double v = u + sh[h];", "double v = u;"),
    "ties to higher id": ("return (a->id > b->id) - (a->id < b->id);",
                          "return (a->id < b->id) - (a->id > b->id);"),
    "up-projection of z": ("dot_bf16(lat_up + h * L, ylat, L)", "dot_bf16(lat_up + h * L, z, L)"),
    "weights from keys": ("total += s[sel[j]];", "total += kb[sel[j]];"),
    "gate/up rows swapped": ("q13 + (I + i) * (L / 2), s13 + (I + i) * (L / 32)",
                             "q13 + i * (L / 2), s13 + i * (L / 32)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor missing: {old!r}"
    mutated = tmp_path / "moe_oracle.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                    str(mutated), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins passed with mutation {name!r}:\n{r.stdout[-2000:]}"


# Mistakes planted in the near-tie helper of the oracle's Python front end
# (which decides the GPU selections the parity tests accept): the mutated
# function replaces the real one while the near-tie pins run in this process.
PY_MUTATIONS = {
    "must-keep set from the k-th key": ("key64_row > v_k1 + tau", "key64_row > v_k + tau"),
    "gap between the wrong ranks": ("if v_k - v_k1 > tau:", "if v_k - key64_row[order[min(k + 1, E - 1)]] > tau:"),
    "candidates not reaching below the k-th": ("(key64_row >= v_k - tau)", "(key64_row >= v_k)"),
    "no final filter": ("if _is_valid_selection(key64_row, sel, tau):", "if True:"),
    "candidates not reaching above the (k+1)-th": ("(key64_row <= v_k1 + tau)",
                                                   "(key64_row <= v_k1)"),
}


@pytest.mark.parametrize("name", sorted(PY_MUTATIONS))
def test_near_tie_pins_catch_planted_mistake(name, monkeypatch):
    import itertools
    import types

    import oracle
    import test_oracle_pins as pins
    old, new = PY_MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    assert src.count(old) == 1, f"mutation anchor missing: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__file__"] = os.path.join(ROOT, "oracle", "__init__.py")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    monkeypatch.setattr(oracle, "near_tie_alternatives", mod.near_tie_alternatives)
    cases = ["exact tie", "gap just below tau", "gap just above tau",
             "key within tau above the k-th", "many within tau", "all equal", "random"]
    caught = False
    for case, (E, k) in itertools.product(cases, [(6, 1), (8, 3), (10, 4), (12, 2), (9, 9)]):
        try:
            pins.test_near_tie_alternatives_match_bruteforce(case, E, k)
        except AssertionError:
            caught = True
            break
    if not caught:
        try:
            pins.test_near_tie_gap_above_tau_accepts_only_the_oracle_selection()
        except AssertionError:
            caught = True
    assert caught, f"near-tie pins passed with mutation {name!r}"
