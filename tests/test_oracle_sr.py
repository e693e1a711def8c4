"""Pins of the oracle's stochastic rounding (CPU only).

The pages name stochastic rounding for FP4 gradients ([MP] "NVFP4"; [LP]
section 2.4 item 5) without fixing its arithmetic; the oracle's reading is
"round up with probability equal to the distance to the lower neighbour,
measured in 2^-16 steps", driven by Philox4x64-10. These tests pin
  - the generator against numpy's independent Philox4x64-10,
  - the element mapping against one continuous numpy Philox stream,
  - the rounding against its defining properties: only the two neighbours,
    the exact up-count over all 65536 random values, unbiasedness,
    saturation and sign,
  - the NVFP4 recipe with SR against the round-to-nearest recipe.
"""
import math

import numpy as np
import pytest

from conftest import golden

M64 = (1 << 64) - 1


def numpy_philox(counter_words, key_words, n_blocks=1):
    """numpy's Philox4x64-10 blocks for counters c, c+1, ... (numpy bumps the
    counter before each block, hence the -1)."""
    c = sum(int(v) << (64 * i) for i, v in enumerate(counter_words))
    k = int(key_words[0]) | (int(key_words[1]) << 64)
    g = np.random.Philox(counter=(c - 1) % (1 << 256), key=k)
    return g.random_raw(4 * n_blocks).reshape(n_blocks, 4)


def test_philox_matches_numpy(orc):
    rng = np.random.default_rng(11)
    cases = [([0, 0, 0, 0], [0, 0]), ([M64] * 4, [M64, M64]), ([M64, 0, 0, 0], [1, 0]),
             ([1, 2, 3, 4], [5, 6])]
    for _ in range(200):
        cases.append(([int(v) for v in rng.integers(0, 1 << 64, 4, dtype=np.uint64)],
                      [int(v) for v in rng.integers(0, 1 << 64, 2, dtype=np.uint64)]))
    for c, k in cases:
        assert np.array_equal(orc.philox4x64_10(c, k), numpy_philox(c, k)[0]), (c, k)


@pytest.mark.parametrize("seed,offset,plane", [(0, 0, 0), (1234567, 9, 0), (2**64 - 5, 2**40, 1)])
def test_sr_bits_follow_one_numpy_stream(orc, seed, offset, plane):
    # groups g0, g0+1, ... are consecutive counters of one stream
    g0, n = 1000, 64
    blocks = numpy_philox([g0, offset, plane, 0], [seed, 0], n)
    for e in range(16 * g0, 16 * (g0 + n), 7):
        g, j = divmod(e, 16)
        want = int(blocks[g - g0][j // 4]) >> (16 * (j % 4)) & 0xFFFF
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
        # exact count: round up iff u / 2^16 < g, so ceil(g * 2^16) values go up
        g = (v - lo) / (hi - lo)
        ups = int((mags == hi).sum())
        assert ups == math.ceil(g * 65536), (y, ups, g)
        # unbiased to within one 2^-16 step of the spacing
        assert abs(mags.mean() - v) <= (hi - lo) / 65536 + 1e-12, y
        # sign kept
        assert np.all((codes >> 3) == (1 if np.signbit(y) else 0))


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
    # a negative value far below 0.5 rounds up (to -0.5) for u = 0 only
    q = orc.encode_e2m1_sr(np.full(65536, -1e-30, np.float32), u)
    assert q[0] == 0x9 and np.all(q[1:] == 0x8)


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
