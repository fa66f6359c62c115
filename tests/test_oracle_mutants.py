"""The pins must catch plausible mistakes in the oracle.

Each case copies tq_oracle.c to a temporary directory, plants one mistake by a
textual edit (a dropped term, a wrong index, a wrong rounding rule ...),
compiles the copy with gcc and runs the pins against it.  At least one pin must
fail for every planted mistake.  Everything here runs on the CPU.
"""
import os
import shutil
import subprocess

import pytest

import oracle
from test_oracle_pins import CHECKS

MUTANTS = {
    "dx_index_per_group": ("dx[t * B + g / 2]", "dx[t * B + g / 2 + (g & 1) * (g + 1 < G)]"),
    "pq2_fields_high_first": ("(qs[k >> 2] >> (2 * (k & 3))) & 3", "(qs[k >> 2] >> (6 - 2 * (k & 3))) & 3"),
    "pq2_no_offset": ("w[k] = (int8_t)(u - 1);", "w[k] = (int8_t)(u);"),
    "ptq1_trit_order": ("const int j = k % 5;", "const int j = 4 - k % 5;"),
    "ptq1_divisor": ("(3 * v) / 256", "(3 * v) / 255"),
    "q8k_scale_128": ("amax / 127.0f", "amax / 128.0f"),
    "q8k_round_half_away": ("float r = rintf(ratio);", "float r = roundf(ratio);"),
    "q8k_bsum_span": ("s += qb[16 * j + i];", "s += qb[16 * j + (i & 7)];"),
    "dot_drops_last": ("for (int k = 0; k < TQO_GROUP; ++k)\n                    s += (int64_t)w[k] * (int64_t)qt[k];\n                if (s > INT32_MAX",
                       "for (int k = 0; k < TQO_GROUP - 1; ++k)\n                    s += (int64_t)w[k] * (int64_t)qt[k];\n                if (s > INT32_MAX"),
    "matmul_scale_swapped": ("((double)dw * (double)dx[t * B + g / 2])", "((double)dw * (double)dx[t * B + (g % B)])"),
    "half_bias": ("expo - 25", "expo - 24"),
    "matmul_transposed_q": ("const int8_t *qt = q + t * cols + g * TQO_GROUP;\n                int64_t s = 0;\n                for (int k = 0; k < TQO_GROUP; ++k)\n                    s += (int64_t)w[k] * (int64_t)qt[k];\n                const double",
                             "const int8_t *qt = q + t * cols + g * TQO_GROUP;\n                int64_t s = 0;\n                for (int k = 0; k < TQO_GROUP; ++k)\n                    s += (int64_t)w[k] * (int64_t)qt[127 - k];\n                const double"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    path = tmp_path / "m.c"
    path.write_text(mutated)
    so = str(tmp_path / "libm.so")
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(path), "-o", so, "-lm"])
    saved = oracle._lib
    oracle._lib = oracle.load(so)
    failed = []
    try:
        for check in CHECKS:
            try:
                check(oracle)
            except (AssertionError, OverflowError, ValueError, IndexError):
                failed.append(check.__name__)
    finally:
        oracle._lib = saved
    assert failed, f"no pin caught the planted mistake {name}"
