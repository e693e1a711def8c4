"""The NVFP4 kernels compute the block value b = fp32(a / 6) without a
division for a >= 2^-125: q = a * RN(1/6), then one FMA-based correction
with the exact residual a - 6q. This test proves that equal to the correctly
rounded division for every fp32 value in that range, by exhaustion on the
host's IEEE arithmetic (gcc, no contraction, fmaf correctly rounded), and
shows the threshold is needed: the shortcut differs from the division for
some subnormal quotients. (CPU only; about 20 s.)"""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("div6") / "div6_exhaustive")
    subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
                    os.path.join(ROOT, "tests", "div6_exhaustive.c"), "-o", exe, "-lm"], check=True)
    return exe


def test_div6_shortcut_is_exact_above_threshold(checker):
    r = subprocess.run([checker], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checked 2122317824 values, 0 disagree" in r.stdout, r.stdout


def shortcut(a):
    a = np.float32(a)
    zh = np.float32(1.0) / np.float32(6.0)
    q = np.float32(a * zh)
    t = np.float32(np.float64(-q) * 6.0 + np.float64(a))        # exact residual here: |t| is tiny
    return np.float32(np.float64(t) * np.float64(zh) + np.float64(q))


def test_div6_threshold_is_needed():
    # a = 9 * 2^-149: a / 6 = 1.5 * 2^-149 rounds to 2 * 2^-149 (tie to even),
    # the shortcut gives 1 * 2^-149; the kernels divide below 2^-125
    a = np.uint32(9).view(np.float32)
    assert (a / np.float32(6.0)).view(np.uint32) == 2
    assert shortcut(a).view(np.uint32) == 1
