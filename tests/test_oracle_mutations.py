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
    "bias sign flipped": ("(float)(s[e] + (bias", "(float)(s[e] - (bias"),
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
