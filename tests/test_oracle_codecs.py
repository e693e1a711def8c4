"""Pins for the oracle's element codecs (CPU only).

Each test ties the oracle to something other than itself: the format facts
the pages print (tests/golden), torch's own float8 casts and decodes, and a
brute-force nearest-value search written independently here.
"""
import math

import numpy as np
import pytest
import torch

from conftest import golden

E4M3, E5M2, E2M1 = 0, 1, 2
TORCH_DT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def all_finite_bf16_as_f32():
    b = np.arange(65536, dtype=np.uint32)
    f = (b << 16).view(np.float32)
    return f[np.isfinite(f)]


def brute_force_encode(values_pos, y):
    """Nearest positive value by exhaustive search over every code, ties to
    the even code, magnitude clamped to the largest value, sign kept."""
    vals = np.asarray(values_pos, dtype=np.float64)
    a = np.minimum(np.abs(y.astype(np.float64)), vals[-1])
    d = np.abs(a[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    codes = np.arange(len(vals))
    # among the tied candidates pick the even code (there are at most two)
    even = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    signbit = np.signbit(y).astype(np.uint32)
    return pick.astype(np.uint32), signbit


def positive_values(orc, fmt):
    return [orc.decode(fmt, c) for c in range(orc.max_code(fmt) + 1)]


# ---------------------------------------------------------------- decode
def test_format_maxima_and_specials(orc):
    facts = golden("format_facts.json")["formats"]
    assert orc.fmax(E4M3) == facts["e4m3"]["max_finite"]
    assert orc.fmax(E5M2) == facts["e5m2"]["max_finite"]
    # E4M3: NaN exists (all-ones exponent and mantissa), no infinity anywhere
    assert math.isnan(orc.decode(E4M3, 0x7F)) and math.isnan(orc.decode(E4M3, 0xFF))
    assert not any(math.isinf(orc.decode(E4M3, c)) for c in range(256))
    # E5M2: +-Inf and NaN encodings
    assert orc.decode(E5M2, 0x7C) == math.inf and orc.decode(E5M2, 0xFC) == -math.inf
    assert all(math.isnan(orc.decode(E5M2, c)) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    # bit budget from the table: 1 + e + m = 8
    for k in ("e4m3", "e5m2"):
        f = facts[k]
        assert f["sign_bits"] + f["exponent_bits"] + f["mantissa_bits"] == 8


def test_e4m3_grid_between_32_and_64(orc):
    facts = golden("format_facts.json")
    vals = sorted(v for v in (orc.decode(E4M3, c) for c in range(0x7F)) if 32 <= v < 64)
    # three mantissa bits: eight evenly spaced values in the binade [32, 64)
    assert vals == [32.0 + 4.0 * i for i in range(8)]
    for v in facts["e4m3_grid_32_64_listed"]:
        assert v in vals
    for v in facts["e4m3_not_representable"]:
        assert v not in vals


def test_e2m1_values_and_layout(orc):
    g = golden("e2m1_values.json")
    got = [orc.decode(E2M1, c) for c in range(16)]
    assert got == g["values"]
    # signed zero in code 8
    assert math.copysign(1.0, got[8]) == -1.0
    # field layout: sign bit 3, exponent bits 2-1, mantissa bit 0, bias 1
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = (m / 2.0) if e == 0 else (1 + m / 2.0) * 2.0 ** (e - 1)
        assert got[c] == (-mag if s else mag)


def test_decode_matches_torch_all_codes(orc):
    codes = torch.arange(256, dtype=torch.uint8)
    for fmt, dt in TORCH_DT.items():
        ref = codes.view(dt).float().numpy().astype(np.float64)
        got = np.array([orc.decode(fmt, c) for c in range(256)])
        assert np.array_equal(np.isnan(ref), np.isnan(got))
        ok = ~np.isnan(ref)
        assert np.array_equal(ref[ok], got[ok])
        assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_e8m0_decode_matches_torch(orc):
    g = golden("e8m0_facts.json")
    assert g["bits"] == 8 and g["mantissa_bits"] == 0 and not g["signed"]
    codes = torch.arange(256, dtype=torch.uint8)
    with np.errstate(invalid="ignore"):                 # code 0xFF is NaN
        ref = codes.view(torch.float8_e8m0fnu).float().numpy().astype(np.float64)
    got = np.array([orc.decode_e8m0(c) for c in range(256)])
    assert math.isnan(got[255]) and math.isnan(ref[255])
    assert np.array_equal(ref[:255], got[:255])
    # the code is the fp32 exponent field of the power of two it stands for
    for c in range(1, 255):
        bits = np.array([got[c]], np.float32).view(np.uint32)[0]
        assert (bits >> 23) & 0xFF == c and bits & 0x7FFFFF == 0


# ---------------------------------------------------------------- encode
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("scale", [1.0, 0.448, 2.0 ** -10, 2.0 ** 7, 3.7, 57344.0 / 3.0])
def test_encode_matches_torch_cast_on_all_bf16(orc, fmt, scale):
    """torch's fp32->float8 cast is round-to-nearest-even without saturation,
    so the saturating encode must equal torch's cast of the clamped value."""
    x = all_finite_bf16_as_f32()
    with np.errstate(over="ignore"):                    # products past fp32's range are dropped next
        y = (x * np.float32(scale)).astype(np.float32)
    y = y[np.isfinite(y)]
    fm = np.float32(orc.fmax(fmt))
    ref = torch.from_numpy(np.clip(y, -fm, fm)).to(TORCH_DT[fmt]).view(torch.uint8).numpy()
    got = orc.encode_array(fmt, y)
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, f"first mismatch y={y[bad[0]]!r} torch={ref[bad[0]]:#x} oracle={got[bad[0]]:#x}"


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_matches_torch_cast_random_fp32(orc, fmt):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    y = bits.view(np.float32)
    y = y[np.isfinite(y)]
    fm = np.float32(orc.fmax(fmt))
    ref = torch.from_numpy(np.clip(y, -fm, fm)).to(TORCH_DT[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(orc.encode_array(fmt, y), ref)


@pytest.mark.parametrize("fmt", [E4M3, E5M2, E2M1])
def test_encode_brute_force_at_ties_and_neighbours(orc, fmt):
    """Every midpoint between adjacent codes, one fp32 ulp either side, each
    code value itself and values past the top, both signs."""
    v = np.array(positive_values(orc, fmt), dtype=np.float64)
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    pts = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf)),
                          v.astype(np.float32), np.float32(v[-1]) * np.array([1.0001, 1.5, 2.0, 1e6], np.float32),
                          np.array([0.0, 1e-30, 1e-45], np.float32)]).astype(np.float32)
    pts = np.concatenate([pts, -pts])
    mag, sign = brute_force_encode(v, pts)
    sign_bit = 0x8 if fmt == E2M1 else 0x80
    want = (mag | (sign * sign_bit)).astype(np.uint8)
    got = orc.encode_array(fmt, pts)
    bad = np.nonzero(want != got)[0]
    assert bad.size == 0, f"y={pts[bad[0]]!r} want={want[bad[0]]:#x} got={got[bad[0]]:#x}"


def test_encode_brute_force_random(orc):
    rng = np.random.default_rng(11)
    for fmt, hi in ((E4M3, 500.0), (E5M2, 60000.0), (E2M1, 7.0)):
        v = np.array(positive_values(orc, fmt))
        y = (rng.uniform(-hi, hi, 20000) * np.exp2(rng.integers(-12, 1, 20000))).astype(np.float32)
        mag, sign = brute_force_encode(v, y)
        want = (mag | (sign * (0x8 if fmt == E2M1 else 0x80))).astype(np.uint8)
        assert np.array_equal(orc.encode_array(fmt, y), want)


def test_e2m1_ties_to_even(orc):
    # midpoints of the FP4 grid go to the neighbour with an even code
    cases = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for y, want in cases.items():
        c = orc.encode(E2M1, y)
        assert orc.decode(E2M1, c) == want and c % 2 == 0
        assert orc.decode(E2M1, orc.encode(E2M1, -y)) == -want


def test_saturation_and_signed_zero(orc):
    assert orc.encode(E4M3, 1e30) == 0x7E and orc.encode(E4M3, -1e30) == 0xFE
    assert orc.encode(E4M3, 465.0) == 0x7E       # torch would give NaN here
    assert orc.encode(E5M2, 61440.0) == 0x7B     # torch would give Inf here
    assert orc.encode(E2M1, 100.0) == 0x7 and orc.encode(E2M1, -100.0) == 0xF
    assert orc.encode(E4M3, -1e-9) == 0x80
    assert orc.encode(E5M2, -1e-9) == 0x80
    assert orc.encode(E2M1, -0.1) == 0x8
    assert orc.encode(E4M3, 0.0) == 0x00 and orc.encode(E4M3, -0.0) == 0x80


def test_e4m3_subnormals(orc):
    # smallest subnormal 2^-9, smallest normal 2^-6 (bias 7)
    assert orc.decode(E4M3, 0x01) == 2.0 ** -9
    assert orc.decode(E4M3, 0x08) == 2.0 ** -6
    assert orc.encode(E4M3, 2.0 ** -10) == 0x00                 # tie between 0 and 2^-9 -> even (0)
    assert orc.encode(E4M3, np.nextafter(np.float32(2.0 ** -10), np.float32(1))) == 0x01
    assert orc.decode(E5M2, 0x01) == 2.0 ** -16
