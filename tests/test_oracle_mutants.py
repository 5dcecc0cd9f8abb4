"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a copy of oracle.c (on the CPU only),
builds it, and runs the oracle pin tests against that build; every run must
fail.  The mistakes cover each part of the oracle: the binary16 conversions, both
block decodes, the q8 quantizer, the integer dots and the result's terms.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "f16 tie direction": ("r = (lo & 1) ? hi : lo;", "r = (lo & 1) ? lo : hi;"),
    "f16 subnormal exponent": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    "q6k ql half select": ("ql[64 * h + 32 * (m % 2) + l]", "ql[64 * h + 32 * (m / 2) + l]"),
    "q6k nibble select": ("(m < 2) ? (lowbyte & 15) : (lowbyte >> 4)",
                          "(m < 2) ? (lowbyte >> 4) : (lowbyte & 15)"),
    "q6k centring": ("(low | (high << 4)) - 32", "(low | (high << 4)) - 31"),
    "q6k qh index": ("qh[32 * h + l]", "qh[32 * h + l % 16]"),
    "q4k min high bits": ("| ((P[c] >> 6) << 4));", "| ((P[c - 4] >> 6) << 4));"),
    "q4k code index": ("qs[32 * (e / 64) + e % 32]", "qs[32 * (e / 64) + e % 16]"),
    "q8 divisor": ("amax / 127.0f", "amax / 128.0f"),
    "q8 quantizes with the unrounded scale": ("const float r = xc[k] / dhf;",
                                              "const float r = xc[k] / d32;"),
    "q8 ties away from zero": ("float n = rintf(r);", "float n = roundf(r);"),
    "q8 sum scale": ("oracle_f32_to_f16(dhf * (float)S)", "oracle_f32_to_f16(d32 * (float)S)"),
    "q4k min sign": ("const double tau2 = -(", "const double tau2 = +("),
    "q4k min uses d": ("(double)r->dmin[b] * (double)r->mn4[c]", "(double)r->d[b] * (double)r->mn4[c]"),
    "q6k scale index": ("(double)r->sc6[g] * dh", "(double)r->sc6[c] * dh"),
    "activation scale index": ("oracle_f16_to_f64(dhrow[c])", "oracle_f16_to_f64(dhrow[b])"),
    "q6k group operand swap": ("idot(r->w6 + 16 * g, qrow + 16 * g, 16)",
                               "idot(r->w6 + 16 * g, qrow + 16 * (g ^ 1), 16)"),
    "q4k chunk super-scale": ("(double)r->d[b] * (double)r->sc4[c] * dh",
                              "(double)r->d[c % 2] * (double)r->sc4[c] * dh"),
    "q6k J scale index": ("(int32_t)(sc[2 * c] * d0 + sc[2 * c + 1] * d1)",
                          "(int32_t)(sc[c] * d0 + sc[c + 1] * d1)"),
    "q6k J halves' scales swapped": ("(int32_t)(sc[2 * c] * d0 + sc[2 * c + 1] * d1)",
                                     "(int32_t)(sc[2 * c + 1] * d0 + sc[2 * c] * d1)"),
}

PIN_TESTS = ["tests/test_oracle_f16.py", "tests/test_oracle_decode.py",
             "tests/test_oracle_quantize.py", "tests/test_oracle_mmq.py"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                    "-I", os.path.join(ROOT, "oracle"), str(mut), "-o", str(lib), "-lm"],
                   check=True)
    env = dict(os.environ, QMM_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_TESTS], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0, f"pins did not catch: {name}\n{r.stdout[-2000:]}"
