"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a temporary copy of the oracle's C source
(CPU only), builds it, and runs the pin suite (tests/test_oracle.py) against
it in a subprocess; the suite must fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "trellis_oracle.c")

MUTANTS = {
    "palette-index-bit-order": ("int palette = p0 | (p1 << 1);", "int palette = p1 | (p0 << 1);"),
    "entry-permutation-bit-order": ("int entry = b ^ (q0 | (q1 << 1));", "int entry = b ^ (q1 | (q0 << 1));"),
    "mask-typo": ("MASK_P0 = 0x1089u", "MASK_P0 = 0x1088u"),
    "msb-first-symbols": ("row_words[k / 16] >> (2 * (k % 16))", "row_words[k / 16] >> (30 - 2 * (k % 16))"),
    "state-shift-direction": ("s = ((s << 2) | (uint32_t)row_symbol(w, k)) & 0xFFFFu;",
                              "s = ((s >> 2) | ((uint32_t)row_symbol(w, k) << 14)) & 0xFFFFu;"),
    "no-row-reset": ("uint32_t s = 0;                                   /* reset per row (R2) */",
                     "static uint32_t s = 0;"),
    "p3-zero-positive": ("{-2.0, -0.0, 1.5, 6.0}", "{-2.0, 0.0, 1.5, 6.0}"),
    "scale-bias": ("return ldexp(1.0, e - 127);", "return ldexp(1.0, e - 128);"),
    "gemv-drops-last-column": ("for (int64_t k = 0; k < cols; ++k) {\n        s = ((s << 2) | (uint32_t)row_symbol(words, k)) & 0xFFFFu;\n        double w",
                               "for (int64_t k = 0; k < cols - 1; ++k) {\n        s = ((s << 2) | (uint32_t)row_symbol(words, k)) & 0xFFFFu;\n        double w"),
    "swiglu-gate-up-swapped": ("double g = y_gu[s * 2 * inter + i];\n            double u = y_gu[s * 2 * inter + inter + i];",
                               "double u = y_gu[s * 2 * inter + i];\n            double g = y_gu[s * 2 * inter + inter + i];"),
    "gate-weight-transposed": ("double g = gate_w ? gate_w[t * k + j] : 1.0;", "double g = gate_w ? gate_w[j * T + t] : 1.0;"),
    "expand-nibble-order": ("(codes[2 * j] | (codes[2 * j + 1] << 4))", "(codes[2 * j + 1] | (codes[2 * j] << 4))"),
    "viterbi-drops-curvature": ("double c = cost[prev] + d[k] * err * err;", "double c = cost[prev] + err * err;"),
    "window-too-short": ("int64_t first = k - 7 < 0 ? 0 : k - 7;", "int64_t first = k - 5 < 0 ? 0 : k - 5;"),
    "e5m3-bias": ("return ldexp(1.0 + (double)m / 8.0, E - 15);", "return ldexp(1.0 + (double)m / 8.0, E - 16);"),
    "e5m3-no-subnormals": ("if (E == 0) return ldexp((double)m / 8.0, -14);",
                           "if (E == 0) return ldexp(1.0 + (double)m / 8.0, -15);"),
    "e5m3-mantissa-weight": ("return ldexp(1.0 + (double)m / 8.0, E - 15);", "return ldexp(1.0 + (double)m / 16.0, E - 15);"),
    "e5m3-read-as-ue8m0": ("return fmt == SCALE_E5M3 ? oracle_e5m3_scale(byte) : oracle_ue8m0_scale(byte);",
                           "return oracle_ue8m0_scale(byte);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = tmp_path / "trellis_oracle.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                           "-o", str(lib), str(mutated), "-lm"])
    env = dict(os.environ, TRELLIS_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
