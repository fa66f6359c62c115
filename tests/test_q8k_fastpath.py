"""The q8_K block scale d = fl(max|x| / 127) is formed on the GPU without a
division (q8k_div127 in csrc/q8k_block.h): a product with fl(1/127) and one
FMA correction.  That this equals the IEEE quotient is a property of fp32
arithmetic, checked here on the host for every significand at exponents
spanning the range the kernels use it on (maxima from 2^-93 up to the largest
finite float; smaller maxima take the IEEE division), with the C library's
correctly rounded fmaf.  The GPU parity tests then check the kernels'
quantized blocks bit for bit against the oracle."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("div127") / "div127_check")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                           os.path.join(HERE, "host", "div127_check.c"), "-o", exe, "-lm"])
    return exe


def test_div127_matches_ieee_quotient(checker):
    # biased exponents: 34 is 2^-93 (the smallest maximum on the fast path),
    # 254 the top binade; the others sample the range between
    exps = [34, 35, 60, 100, 126, 127, 128, 160, 200, 253, 254]
    out = subprocess.check_output([checker, *map(str, exps)], text=True).split()
    n, bad = int(out[0]), int(out[1])
    assert n == len(exps) << 23
    assert bad == 0, f"{bad} of {n} significands differ from the IEEE quotient"
