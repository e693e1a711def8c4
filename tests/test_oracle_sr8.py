"""Pins of the oracle's stochastic rounding to the 8-bit formats (CPU only).

The pages list stochastic rounding beside round-to-nearest-even as a way to
round FP8 values ([MP] "FP8 数据格式", rounding) and put it on gradients ([LP]
section 2.4 item 5). The oracle carries its FP4 reading to E4M3 and E5M2: 16
random bits added below the last kept bit, then truncation, with the bits of
each element from the Philox4x32-10 mapping pinned in test_oracle_sr.py.
These tests pin
  - orc_encode_sr against the add-and-truncate form done on the integer fp32
    significand (an implementation that shares nothing with the oracle's
    table search), with codes decoded by torch's float8 types,
  - its defining properties: only the two neighbours, the exact up-count over
    all 65536 random values (the largest u go up), unbiasedness, grid values
    fixed, saturation at the largest finite value, the sign,
  - the E2M1 case of the generic function against orc_encode_e2m1_sr,
  - the per-tensor, blockwise 1x128 and MX recipes with stochastic rounding:
    scales as with round-to-nearest, every element recomputed by the test
    from its scaled value and its plane's random bits, unbiased where
    round-to-nearest is not, and the random streams separated by plane,
    offset and seed.
"""
import math

import numpy as np
import pytest
import torch

E4M3, E5M2, E2M1 = 0, 1, 2
FMAX = {E4M3: 448.0, E5M2: 57344.0}
MIN_NORMAL_EXP = {E4M3: -6, E5M2: -14}
MBITS = {E4M3: 3, E5M2: 2}
TORCH_T = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def decode(fmt, codes):
    """Values of 8-bit codes by torch's float8 types (independent of the oracle)."""
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8).ravel())
    return c.view(TORCH_T[fmt]).to(torch.float64).numpy().reshape(np.shape(codes))


def sr_add_truncate(fmt, v, u):
    """Stochastic rounding of a non-negative fp32 v below Fmax done on bits:
    the grid spacing h = 2^k at v (2^(E - mbits) in the normal binade 2^E,
    the subnormal spacing below the smallest normal); v/h with 16 fraction
    bits is the 24-bit significand shifted (bits below those 16 dropped);
    u is added and the sum truncated to whole units of h. Returns the grid
    values (float64) for an array of u."""
    bits = int(np.float32(v).view(np.uint32))
    e, m = (bits >> 23) & 0xFF, bits & 0x7FFFFF
    sig, exp = (m | 0x800000, e - 150) if e else (m, -149)      # v = sig * 2^exp
    E = max(math.floor(math.log2(v)), MIN_NORMAL_EXP[fmt]) if v > 0 else MIN_NORMAL_EXP[fmt]
    k = E - MBITS[fmt]
    shift = exp - k + 16
    t = sig << shift if shift >= 0 else sig >> -shift
    s = t + u.astype(np.int64)
    return (s >> 16).astype(np.float64) * 2.0 ** k


def sample_inputs(fmt, rng):
    vs = list(np.exp2(rng.uniform(-149, math.log2(FMAX[fmt]), 150)).astype(np.float32))
    # midpoints between neighbours and their fp32 neighbours, in every binade
    grid = np.unique(np.abs(decode(fmt, np.arange(256))))
    grid = grid[np.isfinite(grid) & (grid <= FMAX[fmt])]
    for a, b in zip(grid[:-1:3], grid[1::3]):
        mid = np.float32((a + b) / 2)
        vs += [np.nextafter(mid, np.float32(0)), mid, np.nextafter(mid, np.float32(1e9))]
    vs += [np.float32(FMAX[fmt]) * np.float32(1 - 2.0 ** -20), np.float32(2.0 ** -149)]
    return [v for v in vs if v < FMAX[fmt]]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_fp8_sr_equals_bit_level_add_and_truncate(orc, fmt):
    u = np.arange(65536, dtype=np.uint16)
    for v in sample_inputs(fmt, np.random.default_rng(30 + fmt)):
        want = sr_add_truncate(fmt, v, u)
        got = decode(fmt, orc.encode_sr(fmt, np.full(65536, v, np.float32), u))
        assert np.array_equal(got, want), (fmt, float(v))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_fp8_sr_neighbours_exact_up_count_and_unbiased(orc, fmt):
    rng = np.random.default_rng(40 + fmt)
    u = np.arange(65536, dtype=np.uint16)
    grid = np.unique(np.abs(decode(fmt, np.arange(256))))
    grid = grid[np.isfinite(grid) & (grid <= FMAX[fmt])]
    ys = list((rng.choice([-1, 1], 80) * np.exp2(rng.uniform(-24, math.log2(FMAX[fmt]), 80))).astype(np.float32))
    for y in ys:
        v = abs(float(y))
        lo = grid[grid <= v].max()
        hi = grid[grid > v].min()
        codes = orc.encode_sr(fmt, np.full(65536, y, np.float32), u)
        vals = decode(fmt, codes)
        mags = np.abs(vals)
        assert set(np.unique(mags)) <= {lo, hi}, y
        g = (v - lo) / (hi - lo)
        up = mags == hi
        ups = int(up.sum())
        assert ups == math.floor(g * 65536), (y, ups, g)
        assert np.all(up[65536 - ups:]) and not np.any(up[:65536 - ups])
        assert abs(mags.mean() - v) <= (hi - lo) / 65536 + 1e-15 * v, y
        assert np.all((codes >> 7) == (1 if np.signbit(y) else 0))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_fp8_sr_grid_values_fixed_saturation_and_sign(orc, fmt):
    u = np.arange(0, 65536, 61, dtype=np.uint16)
    for c in range(256):
        val = decode(fmt, np.array([c]))[0]
        if not np.isfinite(val) or (c & 0x7F) == 0:
            continue
        assert np.all(orc.encode_sr(fmt, np.full(u.size, val, np.float32), u) == c), c
    top = {E4M3: 0x7E, E5M2: 0x7B}[fmt]
    for y in (FMAX[fmt], FMAX[fmt] * 1.01, 3e38):
        assert np.all(orc.encode_sr(fmt, np.full(u.size, y, np.float32), u) == top)
        assert np.all(orc.encode_sr(fmt, np.full(u.size, -y, np.float32), u) == top | 0x80)
    assert np.all(orc.encode_sr(fmt, np.full(u.size, -0.0, np.float32), u) == 0x80)
    assert np.all(orc.encode_sr(fmt, np.full(u.size, 0.0, np.float32), u) == 0x00)


def test_generic_sr_equals_e2m1_sr(orc):
    rng = np.random.default_rng(50)
    y = rng.uniform(-7, 7, 65536).astype(np.float32)
    u = rng.integers(0, 65536, 65536).astype(np.uint16)
    assert np.array_equal(orc.encode_sr(E2M1, y, u), orc.encode_e2m1_sr(y, u))


# ---------------------------------------------------------------- recipes
def to_f32(x):
    return (x.astype(np.uint32) << 16).view(np.float32) if x.dtype == np.uint16 else x


def bits_of(orc, seed, offset, plane, n):
    return np.array([orc.sr_bits(seed, offset, plane, e) for e in range(n)], np.uint16)


def expect_codes(orc, fmt, y, seed, offset, plane):
    """The test's own stochastic codes of a plane of scaled fp32 values y
    (row-major), from the bit-level rounding and the plane's random bits."""
    flat = y.ravel()
    u = bits_of(orc, seed, offset, plane, flat.size)
    out = np.empty(flat.size, np.float64)
    for i, (v, ui) in enumerate(zip(flat, u)):
        a = min(abs(float(v)), FMAX[fmt])
        out[i] = (FMAX[fmt] if a >= FMAX[fmt] else
                  sr_add_truncate(fmt, np.float32(a), np.array([ui]))[0]) * (-1 if np.signbit(v) else 1)
    return out.reshape(y.shape)


def same_values(got_codes, fmt, want):
    g = decode(fmt, got_codes)
    assert np.array_equal(np.abs(g), np.abs(want))
    nz = want != 0
    assert np.array_equal(np.signbit(g[nz]), np.signbit(want[nz]))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_per_tensor_sr_recomputed(orc, fmt, dtype):
    rng = np.random.default_rng(60 + fmt)
    x = (rng.standard_normal((24, 40)) * 3).astype(np.float32)
    if dtype == "bf16":
        x = (x.view(np.uint32) >> 16).astype(np.uint16)
    xf = to_f32(x)
    seed, off = 12345, 6
    sr = orc.quantize_current(x, fmt, outputs=3, sr=(seed, off))
    rn = orc.quantize_current(x, fmt, outputs=3)
    assert sr["s"] == rn["s"] and sr["amax"] == rn["amax"]
    alpha = np.float32(FMAX[fmt]) / np.float32(rn["amax"])
    y = (xf * alpha).astype(np.float32)
    same_values(sr["q_row"], fmt, expect_codes(orc, fmt, y, seed, off, 0))
    same_values(sr["q_col"], fmt, expect_codes(orc, fmt, np.ascontiguousarray(y.T), seed, off, 1))


@pytest.mark.parametrize("pow2", [False, True])
def test_block_1x128_sr_recomputed(orc, pow2):
    rng = np.random.default_rng(70 + pow2)
    x = (rng.standard_normal((128, 256)) * np.exp2(rng.integers(-8, 8, (128, 1)))).astype(np.float32)
    seed, off = 99, 3
    sr = orc.quantize_block(x, (1, 128), outputs=3, pow2=pow2, sr=(seed, off))
    rn = orc.quantize_block(x, (1, 128), outputs=3, pow2=pow2)
    assert np.array_equal(sr["s_row"], rn["s_row"]) and np.array_equal(sr["s_col"], rn["s_col"])
    for plane, (xx, s) in enumerate(((x, rn["s_row"]), (np.ascontiguousarray(x.T), rn["s_col"]))):
        R, C = xx.shape
        a = np.abs(xx).reshape(R, C // 128, 128).max(-1)
        if pow2:
            mult = np.exp2(-np.log2(s.astype(np.float64))).astype(np.float32)   # s is a power of two
        else:
            mult = np.where(a == 0, np.float32(1), np.float32(448.0) / np.where(a == 0, 1, a)).astype(np.float32)
        y = (xx.reshape(R, C // 128, 128) * mult[..., None]).astype(np.float32).reshape(R, C)
        same_values(sr["q_row" if plane == 0 else "q_col"], E4M3, expect_codes(orc, E4M3, y, seed, off, plane))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_mx_sr_recomputed(orc, fmt):
    rng = np.random.default_rng(80 + fmt)
    x = (rng.standard_t(3, (64, 96)) * 0.01).astype(np.float32)
    seed, off = 7, 2 ** 40 + 1
    sr = orc.quantize_mx(x, outputs=3, fmt=fmt, sr=(seed, off))
    rn = orc.quantize_mx(x, outputs=3, fmt=fmt)
    assert np.array_equal(sr["e_row"], rn["e_row"]) and np.array_equal(sr["e_col"], rn["e_col"])
    for plane, (xx, e) in enumerate(((x, rn["e_row"]), (np.ascontiguousarray(x.T), rn["e_col"]))):
        R, C = xx.shape
        mult = np.exp2(127.0 - e.astype(np.float64))                            # 2^-(code - 127), exact
        y = (xx.reshape(R, C // 32, 32).astype(np.float64) * mult[..., None]).astype(np.float32).reshape(R, C)
        same_values(sr["q_row" if plane == 0 else "q_col"], fmt, expect_codes(orc, fmt, y, seed, off, plane))


def test_per_tensor_sr_is_unbiased_where_nearest_is_not(orc):
    # 1 + 1/32 is a quarter of the E4M3 spacing (1/8) above 1: nearest gives 1
    # every time, stochastic rounding 1.125 a quarter of the time
    R, C = 32, 1024
    x = np.full((R, C), 1 + 1 / 32, np.float32)
    x[0, 0] = 448.0                     # amax 448, so alpha = 1
    means = []
    for off in range(4):
        q = orc.quantize_current(x, E4M3, outputs=1, sr=(2025, off))["q_row"]
        v = decode(E4M3, q).ravel()[1:]
        assert set(np.unique(v)) <= {1.0, 1.125}
        means.append(v.mean())
    rn = decode(E4M3, orc.quantize_current(x, E4M3)["q_row"]).ravel()[1:]
    assert np.all(rn == 1.0)
    n = 4 * (R * C - 1)
    assert abs(np.mean(means) - (1 + 1 / 32)) < 6 * 0.125 * math.sqrt(0.25 * 0.75 / n)


def test_sr_streams_by_plane_offset_and_seed(orc):
    rng = np.random.default_rng(90)
    a = rng.standard_normal((128, 128)).astype(np.float32)
    x = ((a + a.T) / 2).astype(np.float32)   # X^T == X: both planes see the same values
    for q in (lambda sr: orc.quantize_current(x, E5M2, outputs=3, sr=sr),
              lambda sr: orc.quantize_block(x, (1, 128), outputs=3, sr=sr),
              lambda sr: orc.quantize_mx(x, outputs=3, sr=sr)):
        s1, s2, s3, s4 = q((5, 0)), q((5, 0)), q((5, 1)), q((6, 0))
        assert np.array_equal(s1["q_row"], s2["q_row"]) and np.array_equal(s1["q_col"], s2["q_col"])
        assert not np.array_equal(s1["q_row"], s1["q_col"])      # planes 0 and 1 draw different bits
        assert not np.array_equal(s1["q_row"], s3["q_row"])      # offset is part of the counter
        assert not np.array_equal(s1["q_row"], s4["q_row"])      # seed is the key


def test_sr_refused_where_not_offered(orc):
    x = np.ones((128, 128), np.float32)
    with pytest.raises((orc.OracleError, ValueError)):
        orc.quantize_block(x, (128, 128), sr=(1, 0))
    with pytest.raises(orc.OracleError):
        orc.quantize_mx(x, fmt=E2M1, sr=(1, 0))
