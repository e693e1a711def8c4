"""Pins of the oracle's stochastic rounding (CPU only).

The pages name stochastic rounding for FP4 gradients ([MP] "NVFP4"; [LP]
section 2.4 item 5) without fixing its arithmetic; the oracle's reading is
"add 16 random bits below the last kept bit and truncate", so a value goes up
with probability equal to its distance to the lower neighbour in 2^-16
steps; the bits come from Philox4x32-10. These tests pin
  - the generator against PyTorch's independent Philox4x32-10 engine,
  - the element mapping against one continuous stream of that engine,
  - the rounding against its defining properties: only the two neighbours,
    the exact up-count over all 65536 random values, unbiasedness,
    saturation and sign,
  - the NVFP4 recipe with SR against the round-to-nearest recipe.
"""
import math
import os
import subprocess

import numpy as np
import pytest

from conftest import ROOT, golden

M32 = (1 << 32) - 1
M64 = (1 << 64) - 1


@pytest.fixture(scope="module")
def torch_philox(tmp_path_factory):
    """PyTorch's CPU Philox4x32-10 engine, compiled from its header: an
    implementation of the generator independent of the oracle. Returns
    f(seed, subsequence, offset, count) -> the engine's first `count` words
    (counter = (offset, subsequence) as 4 x 32-bit words, key = seed)."""
    import torch
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_ref")
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", inc, os.path.join(ROOT, "tests", "philox_ref.cpp"),
                    "-o", exe], check=True)

    def run(queries):
        text = "".join(f"{s} {q} {o} {n}\n" for s, q, o, n in queries)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return [[int(v) for v in line.split()] for line in out.splitlines()]
    return run


def test_philox_matches_torch_engine(orc, torch_philox):
    rng = np.random.default_rng(11)
    cases = [(0, 0, 0), (M64, M64, M64), (1, 2, 3), (0x0123456789ABCDEF, 5, 9), (7, 0, M32), (7, M32, M64 - 1)]
    for _ in range(200):
        cases.append(tuple(int(v) for v in rng.integers(0, 1 << 64, 3, dtype=np.uint64)))
    ref = torch_philox([(s, q, o, 4) for s, q, o in cases])
    for (seed, sub, off), want in zip(cases, ref):
        ctr = [off & M32, off >> 32, sub & M32, sub >> 32]
        key = [seed & M32, seed >> 32]
        assert list(orc.philox4x32_10(ctr, key)) == want, (seed, sub, off)


@pytest.mark.parametrize("seed,offset,plane", [(0, 0, 0), (1234567, 9, 0), (2**64 - 5, 2**40, 1),
                                               (3, 2**63 + 4, 1)])
def test_sr_bits_follow_one_torch_stream(orc, torch_philox, seed, offset, plane):
    # groups h0, h0+1, ... are consecutive counters of one engine stream
    h0, n = (1 << 32) - 5, 32            # crosses the carry into counter word 1
    stream = (2 * offset + plane) & M64
    words = torch_philox([(seed, stream, h0, 4 * n)])[0]
    for e in range(8 * h0, 8 * (h0 + n), 3):
        h, j = divmod(e, 8)
        want = words[4 * (h - h0) + j // 2] >> (16 * (j % 2)) & 0xFFFF
        assert orc.sr_bits(seed, offset, plane, e) == want, e


E2M1 = golden("e2m1_values.json")["values"]
GRID = sorted(set(abs(v) for v in E2M1))  # 0, .5, 1, 1.5, 2, 3, 4, 6


def neighbours(v):
    lo = max(g for g in GRID if g <= v)
    hi = min(g for g in GRID if g > v)
    return lo, hi


def test_e2m1_sr_neighbours_and_exact_up_count(orc):
    rng = np.random.default_rng(12)
    ys = list(rng.uniform(-6, 6, 120).astype(np.float32))
    ys += [np.float32(v) for v in (0.25, 1.25, 2.5, 5.0, 5.999999, 1e-30, -3.75, 0.49999997, 4.0000005)]
    u = np.arange(65536, dtype=np.uint16)
    for y in ys:
        codes = orc.encode_e2m1_sr(np.full(65536, y, np.float32), u)
        vals = np.array([E2M1[c] for c in codes], np.float64)
        v = abs(float(y))
        lo, hi = neighbours(v)
        mags = np.abs(vals)
        assert set(np.unique(mags)) <= {lo, hi}, y
        # exact count: round up iff u + g * 2^16 >= 2^16, so floor(g * 2^16) values go up,
        # and they are the largest u
        g = (v - lo) / (hi - lo)
        up = mags == hi
        ups = int(up.sum())
        assert ups == math.floor(g * 65536), (y, ups, g)
        assert np.all(up[65536 - ups:]) and not np.any(up[:65536 - ups])
        # unbiased to within one 2^-16 step of the spacing
        assert abs(mags.mean() - v) <= (hi - lo) / 65536 + 1e-12, y
        # sign kept
        assert np.all((codes >> 3) == (1 if np.signbit(y) else 0))


def sr_add_truncate_bits(v, u):
    """Stochastic rounding of a non-negative fp32 v < 6 to the E2M1 grid as
    integer work on its bit pattern: the grid spacing h at v is 2^k (0.5 below
    2, 1 below 4, 2 below 6); v/h in fixed point with 16 fraction bits is the
    24-bit significand shifted (bits below those 16 are dropped); u is added
    to that integer and the sum truncated to whole units of h. Returns the
    grid values (float64) for an array of u."""
    bits = int(np.float32(v).view(np.uint32))
    e, m = (bits >> 23) & 0xFF, bits & 0x7FFFFF
    sig, exp = (m | 0x800000, e - 150) if e else (m, -149)    # v = sig * 2^exp
    k = -1 if v < 2 else (0 if v < 4 else 1)                  # h = 2^k
    shift = exp - k + 16                                      # v/h * 2^16 = sig * 2^shift
    t = sig << shift if shift >= 0 else sig >> -shift
    s = t + u.astype(np.int64)
    return (s >> 16).astype(np.float64) * 2.0 ** k


def test_e2m1_sr_equals_bit_level_add_and_truncate(orc):
    """The oracle's rule (up iff u + g*2^16 >= 2^16, compared in fp32) against
    the add-and-truncate form of stochastic rounding done on the integer
    significand: every one of the 65536 random values, for fp32 inputs
    spread over every binade from 2^-140 to 6 and the E2M1 midpoints +-1 ulp."""
    rng = np.random.default_rng(13)
    u = np.arange(65536, dtype=np.uint16)
    vs = list(np.exp2(rng.uniform(-140, np.log2(6.0), 160)).astype(np.float32))
    for mid in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0):
        m = np.float32(mid)
        vs += [np.nextafter(m, np.float32(0)), m, np.nextafter(m, np.float32(7))]
    vs += [np.float32(v) for v in (0.5, 1.0, 2.0, 4.0, 5.9999995, 2.0 ** -149)]
    for v in vs:
        if not v < 6:
            continue
        want = sr_add_truncate_bits(v, u)
        codes = orc.encode_e2m1_sr(np.full(65536, v, np.float32), u)
        got = np.array([E2M1[c] for c in codes], np.float64)
        assert np.array_equal(got, want), v


def test_e2m1_sr_grid_values_are_fixed(orc):
    u = np.arange(0, 65536, 97, dtype=np.uint16)
    for code, val in enumerate(E2M1):
        q = orc.encode_e2m1_sr(np.full(u.size, val, np.float32), u)
        assert np.all(q == code), (code, val)


def test_e2m1_sr_saturation_and_signed_zero(orc):
    u = np.arange(65536, dtype=np.uint16)
    for y, want in ((6.0, 0x7), (7.5, 0x7), (1e30, 0x7), (-6.0, 0xF), (-300.0, 0xF)):
        assert np.all(orc.encode_e2m1_sr(np.full(65536, y, np.float32), u) == want), y
    assert np.all(orc.encode_e2m1_sr(np.full(65536, -0.0, np.float32), u) == 0x8)
    # a negative value far below 2^-17 never reaches -0.5; one of 2^-16 does for u = 65535 only
    assert np.all(orc.encode_e2m1_sr(np.full(65536, -1e-30, np.float32), u) == 0x8)
    q = orc.encode_e2m1_sr(np.full(65536, -2.0**-17, np.float32), u)
    assert q[-1] == 0x9 and np.all(q[:-1] == 0x8)


def grid_index(val):
    return GRID.index(abs(val))


def test_nvfp4_sr_changes_only_element_rounding(orc):
    rng = np.random.default_rng(13)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    rt = orc.quantize_nvfp4(x, (1, 16), 3)
    sr = orc.quantize_nvfp4(x, (1, 16), 3, sr=(99, 5))
    assert np.array_equal(rt["c_row"], sr["c_row"]) and np.array_equal(rt["c_col"], sr["c_col"])
    assert rt["S"] == sr["S"]
    for key in ("p_row", "p_col"):
        a = np.stack([rt[key] & 15, rt[key] >> 4], -1).ravel()
        b = np.stack([sr[key] & 15, sr[key] >> 4], -1).ravel()
        va = np.array([E2M1[c] for c in a])
        vb = np.array([E2M1[c] for c in b])
        ia = np.array([grid_index(v) for v in va])
        ib = np.array([grid_index(v) for v in vb])
        assert np.all(np.abs(ia - ib) <= 1), key            # a neighbour of the nearest value, or it
        nz = (va != 0) & (vb != 0)
        assert np.all(np.sign(va[nz]) == np.sign(vb[nz]))
        assert 0.05 < np.mean(a != b) < 0.6, key            # it does round differently


def test_nvfp4_sr_is_unbiased_where_nearest_is_not(orc):
    # every element 1/4 of the way from 1.0 to 1.5 after scaling: nearest always
    # gives 1.0, the stochastic mean must approach 1.125 (not 1.375, which a
    # flipped comparison would give)
    R, C = 16, 1024
    x = np.full((R, C), 1.125, np.float32)
    x[:, ::16] = 6.0            # each block's max maps to 6 exactly, so r_B = 1
    means = []
    for off in range(4):
        sr = orc.quantize_nvfp4(x, (1, 16), 1, amax=6.0 * 448, sr=(2024, off))
        assert np.all(sr["c_row"] == sr["c_row"].flat[0])
        nib = np.stack([sr["p_row"] & 15, sr["p_row"] >> 4], -1).reshape(R, C)
        v = np.array([E2M1[c] for c in nib.ravel()]).reshape(R, C)
        mask = np.ones((R, C), bool)
        mask[:, ::16] = False
        assert set(np.unique(v[mask])) <= {1.0, 1.5}
        means.append(v[mask].mean())
    m = float(np.mean(means))
    n = 4 * mask.sum()
    assert abs(m - 1.125) < 6 * 0.5 * math.sqrt(0.25 * 0.75 / n), m


def test_nvfp4_sr_streams(orc):
    rng = np.random.default_rng(14)
    a = rng.standard_normal((64, 64)).astype(np.float32)
    x = ((a + a.T) / 2).astype(np.float32)  # X^T == X: both planes see the same blocks
    s1 = orc.quantize_nvfp4(x, (1, 16), 3, sr=(5, 0))
    s2 = orc.quantize_nvfp4(x, (1, 16), 3, sr=(5, 0))
    s3 = orc.quantize_nvfp4(x, (1, 16), 3, sr=(5, 1))
    s4 = orc.quantize_nvfp4(x, (1, 16), 3, sr=(6, 0))
    assert np.array_equal(s1["p_row"], s2["p_row"]) and np.array_equal(s1["p_col"], s2["p_col"])
    assert np.array_equal(s1["c_row"], s1["c_col"])
    assert not np.array_equal(s1["p_row"], s1["p_col"])      # planes 0 and 1 draw different bits
    assert not np.array_equal(s1["p_row"], s3["p_row"])      # offset is part of the counter
    assert not np.array_equal(s1["p_row"], s4["p_row"])      # seed is the key
