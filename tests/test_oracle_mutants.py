"""Plant plausible mistakes in copies of the oracle's C source and check that
every one of them fails at least one pin.  CPU only (gcc)."""
import os
import subprocess
import tempfile

import pytest

from oracle import pnref
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "pnref.c")

MUTANTS = [
    ("halves swapped", "16 * (j & 1) + b * (j >> 1);", "16 * (1 - (j & 1)) + b * (j >> 1);"),
    ("pair offsets permuted", "16 * (j & 1) + b * (j >> 1);", "16 * (j & 1) + b * ((j >> 1) ^ 1);"),
    ("zero point off by one", "    const int z = 1 << (b - 1);\n    const uint32_t mask",
     "    const int z = (1 << (b - 1)) - 1;\n    const uint32_t mask"),
    ("word order reversed", "load_le32(blk + 2 + 4 * i)", "load_le32(blk + 2 + 4 * (7 - i))"),
    ("scale big-endian", "(uint16_t)(blk[0] | (blk[1] << 8))", "(uint16_t)(blk[1] | (blk[0] << 8))"),
    ("half exponent bias", "e - 25);", "e - 24);"),
    ("half subnormal scale", "ldexp((double)f, -24);", "ldexp((double)f, -23);"),
    ("negative zero lost", "out[i * c + j] = d * (float)(n - z);", "out[i * c + j] = d * (float)(n - z) + 0.0f;"),
    ("unused bit read", "const uint32_t mask = (1u << b) - 1u;", "const uint32_t mask = (1u << (b == 3 ? 4 : b)) - 1u;"),
    ("first product dropped", "for (int64_t i = 0; i < k; ++i) {\n        const double p",
     "for (int64_t i = 1; i < k; ++i) {\n        const double p"),
    ("abs sum signed", "t += fabs(p);", "t += p;"),
    ("fp32 accumulation", "double s = 0.0, t = 0.0;", "float s = 0.0f; double t = 0.0;"),
    ("batch rows share output", "ym + mi * ldy + r", "ym + r"),
    ("quantizer scale sign", "-(double)src[istar] / (double)z", "(double)src[istar] / (double)z"),
    ("quantizer argmax ties to last", "if (fabsf(src[i]) > fabsf(src[istar])) istar = i;",
     "if (fabsf(src[i]) >= fabsf(src[istar])) istar = i;"),
    ("quantizer rounds half up", "nearbyint((double)src[i] / d)", "floor((double)src[i] / d + 0.5)"),
    ("quantizer without clamp", "if (v > (double)((1 << b) - 1)) v = (double)((1 << b) - 1);", ""),
    ("half rounding truncates", "double q = nearbyint(ldexp(a, 10 - e));", "double q = floor(ldexp(a, 10 - e));"),
    ("rotation sign flipped", "& 1) ? -v : v;", "& 1) ? v : -v;"),
    ("rotation transposed index", "popcountll((uint64_t)(i & j))", "popcountll((uint64_t)(i | j))"),
    ("rotation scale off", "ldexp(1.0, -lg / 2)", "ldexp(1.0, -lg / 2 + 1)"),
    ("rotation block offset lost", "pnref_half_to_float(x[b0 + j])", "pnref_half_to_float(x[j])"),
    ("rotation first term dropped", "for (int64_t j = 0; j < block; ++j) {\n                const double v",
     "for (int64_t j = 1; j < block; ++j) {\n                const double v"),
    ("rotation accumulates in fp32", "            double s = 0.0;\n            for (int64_t j = 0",
     "            float s = 0.0f;\n            for (int64_t j = 0"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    src = open(SRC).read()
    assert old in src, "mutation site not found: %s" % name
    mutated = src.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "pnref.c")
        so = os.path.join(d, "libpnref_mut.so")
        open(c, "w").write(mutated)
        subprocess.run(["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                        "-fPIC", "-shared", "-I" + os.path.dirname(SRC), "-o", so, c, "-lm"],
                       check=True, capture_output=True)
        o = pnref.Oracle(so)
        failed = []
        for pin in ALL_PINS:
            try:
                pin(o)
            except (AssertionError, ValueError):
                failed.append(pin.__name__)
                break
        assert failed, "mutant '%s' passed every pin" % name
