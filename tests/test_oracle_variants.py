"""Pins of the oracle's format variants (CPU only):
  - MX with E5M2 elements and MXFP4 (E2M1 elements packed two per byte),
    with the scale rule 2^(floor(log2 a) - floor(log2 Fmax));
  - blockwise E4M3 with power-of-two tile scales (the MX rule on the tile).
Each is checked against closed forms computed here from the floating-point
fields, brute-force nearest codes over the whole code table, the formats'
error bounds, and the equivalence of a pow2 tile with MX blocks sharing its
exponent ([MP] "Blockwise scaling": blockwise run as MXFP8 blocks sharing one
scaling factor per tile)."""
import numpy as np
import pytest

from fp8_fp4_tensor_amd import workloads as W
from test_oracle_recipes import dec, nearest_positive

E4M3, E5M2, E2M1 = 0, 1, 2
ROW, COL = 1, 2
EMAX = {E4M3: 8, E5M2: 15, E2M1: 2}        # floor(log2 448), floor(log2 57344), floor(log2 6)
FMAX = {E4M3: 448.0, E5M2: 57344.0, E2M1: 6.0}


def unpack(p):
    out = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
    out[:, 0::2], out[:, 1::2] = p & 0xF, p >> 4
    return out


def codes_of(q, fmt):
    return unpack(q) if fmt == E2M1 else q


@pytest.mark.parametrize("fmt", [E4M3, E5M2, E2M1])
def test_mx_code_closed_form_all_bf16(orc, fmt):
    """code = max(E - emax, 0), E the biased exponent field of the fp32 amax."""
    b = np.arange(0x0000, 0x7F80, dtype=np.uint32)
    a = (b << 16).view(np.float32)
    E = (a.view(np.uint32) >> 23) & 0xFF
    want = np.maximum(E.astype(np.int64) - EMAX[fmt], 0)
    want[a == 0] = 0
    got = np.array([orc.mx_code(v, fmt) for v in a])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", [E5M2, E2M1])
def test_mx_variant_invariants(orc, fmt):
    R, C = 64, 96
    x = W.student_t((R, C), 3.0, 51 + fmt, W.BF16)
    r = orc.quantize_mx(x, fmt=fmt)
    xf = W.bf16_bits_to_f32(x).reshape(R, C)
    for mat, q, codes in ((xf, r["q_row"], r["e_row"]), (xf.T.copy(), r["q_col"], r["e_col"])):
        rr, cc = mat.shape
        blocks = mat.reshape(rr, cc // 32, 32)
        a = np.abs(blocks).max(axis=2)
        e = np.floor(np.log2(a.astype(np.float64))) - EMAX[fmt]
        assert np.array_equal(codes, (e + 127).astype(np.uint8))
        scale = np.exp2(codes.astype(np.float64) - 127)
        y = a / scale
        assert ((y >= 2.0 ** EMAX[fmt]) & (y < 2.0 ** (EMAX[fmt] + 1))).all()
        qc = codes_of(q, fmt).reshape(rr, cc // 32, 32)
        for i in range(rr):
            for j in range(cc // 32):
                m = np.abs(blocks[i, j]) == a[i, j]
                vals = np.abs(dec(orc, fmt, qc[i, j][m]))
                assert ((vals >= 2.0 ** EMAX[fmt]) & (vals <= FMAX[fmt])).all()
        xhat = orc.dequant_mx(q, codes, fmt)
        ys = np.abs(mat) / np.repeat(scale, 32, axis=1)
        if fmt == E5M2:
            ok = (ys >= 2.0 ** -14) & (ys <= FMAX[fmt])
            bound = 2.0 ** -3
        else:
            ok = (ys >= 1.0) & (ys <= FMAX[fmt])
            bound = 2.0 ** -2
        assert ok.sum() > 100
        assert (np.abs(xhat - mat)[ok] / np.abs(mat)[ok]).max() <= bound * (1 + 1e-6)
    rt = orc.quantize_mx(np.ascontiguousarray(x.T), outputs=ROW, fmt=fmt)
    assert np.array_equal(r["q_col"], rt["q_row"]) and np.array_equal(r["e_col"], rt["e_row"])


@pytest.mark.parametrize("fmt", [E5M2, E2M1])
def test_mx_variant_brute_force_tiny(orc, fmt):
    rng = np.random.default_rng(29 + fmt)
    x = (rng.standard_t(3, (2, 64)) * 10.0 ** rng.integers(-3, 3)).astype(np.float32)
    x[1, 40] = -0.0
    r = orc.quantize_mx(x, outputs=ROW, fmt=fmt)
    q = codes_of(r["q_row"], fmt)
    sign = 0x8 if fmt == E2M1 else 0x80
    for i in range(2):
        for j in range(2):
            blk = x[i, j * 32:(j + 1) * 32]
            a = float(np.abs(blk).max())
            e = int(np.floor(np.log2(a))) - EMAX[fmt]
            assert r["e_row"][i, j] == e + 127
            for k in range(32):
                y = np.float32(blk[k] * np.float32(2.0 ** -e))
                want = nearest_positive(orc, fmt, y) | (sign if np.signbit(y) else 0)
                assert q[i, j * 32 + k] == want, (i, j, k, y)


def test_mxfp4_nibble_order_and_zero(orc):
    # element 2k in bits 3..0, 2k+1 in bits 7..4 (the pages' float4_e2m1fn_x2 layout)
    x = np.zeros((1, 32), np.float32)
    x[0, 0], x[0, 1], x[0, 2] = 6.0, -1.0, 0.5
    r = orc.quantize_mx(x, outputs=ROW, fmt=E2M1)
    assert r["e_row"][0, 0] == 127                   # amax 6: 2^(2 - 2)
    assert r["q_row"][0, 0] == (0x7 | (0xA << 4))    # 6 -> 0x7, -1 -> 0xA
    assert r["q_row"][0, 1] == 0x1                   # 0.5 -> 0x1
    z = orc.quantize_mx(np.zeros((32, 32), np.float32), fmt=E2M1)
    assert not z["q_row"].any() and not z["e_row"].any() and not z["e_col"].any()


@pytest.mark.parametrize("block", [(1, 128), (128, 128)])
def test_block_pow2_invariants(orc, block):
    br, bc = block
    R, C = (256, 256) if br == 128 else (128, 256)
    x = W.normal((R, C), 0.02, 61 + br, W.BF16)
    xf = W.bf16_bits_to_f32(x).reshape(R, C)
    r = orc.quantize_block(x, block, outputs=ROW | COL, pow2=True)
    tiles = xf.reshape(R // br, br, C // bc, bc)
    a = np.abs(tiles).max(axis=(1, 3)).astype(np.float64)
    s_want = np.exp2(np.floor(np.log2(a)) - 8).astype(np.float32)
    assert np.array_equal(r["s_row"], s_want)
    qt = r["q_row"].reshape(R // br, br, C // bc, bc)
    for i in range(R // br):
        for j in range(C // bc):
            m = np.abs(tiles[i, :, j, :]) == a[i, j]
            v = np.abs(dec(orc, E4M3, qt[i, :, j, :][m]))
            assert ((v >= 256) & (v <= 448)).all()
    xhat = orc.dequant_block(r["q_row"], r["s_row"], block)
    ys = np.abs(xf) / np.repeat(np.repeat(s_want, br, axis=0), bc, axis=1)
    ok = (ys >= 2.0 ** -6) & (ys <= 448)
    assert (np.abs(xhat - xf)[ok] / np.abs(xf)[ok]).max() <= 2.0 ** -4 * (1 + 1e-6)
    rt = orc.quantize_block(np.ascontiguousarray(x.T), block, pow2=True)
    if br == 128:
        assert np.array_equal(r["q_col"], r["q_row"].T)
    assert np.array_equal(r["q_col"], rt["q_row"]) and np.array_equal(r["s_col"], rt["s_row"])


def test_block_pow2_equals_mx_when_subblocks_share_the_exponent(orc):
    # each 1x128 tile = four MX blocks; when their amaxes share floor(log2), the
    # tile's pow2 scale is their common E8M0 scale and the codes coincide
    rng = np.random.default_rng(71)
    R, C = 8, 256
    x = rng.uniform(-1, 1, (R, C)).astype(np.float32)
    for r in range(R):
        for b in range(C // 32):
            x[r, b * 32 + rng.integers(0, 32)] = np.float32(rng.uniform(4.0, 8.0) * (1 if b % 2 else -1))
    blk = orc.quantize_block(x, (1, 128), pow2=True)
    mx = orc.quantize_mx(x, outputs=ROW)
    assert np.array_equal(blk["q_row"], mx["q_row"])
    assert np.array_equal(np.repeat(blk["s_row"], 4, axis=1), np.exp2(mx["e_row"].astype(np.float64) - 127))


def test_block_pow2_brute_force_tiny(orc):
    rng = np.random.default_rng(73)
    x = (rng.standard_normal((2, 256)) * np.exp2(rng.integers(-8, 8, (2, 256)))).astype(np.float32)
    r = orc.quantize_block(x, (1, 128), pow2=True)
    for i in range(2):
        for j in range(2):
            blk = x[i, j * 128:(j + 1) * 128]
            e = int(np.floor(np.log2(float(np.abs(blk).max())))) - 8
            assert r["s_row"][i, j] == np.float32(2.0 ** e)
            for k in range(128):
                y = np.float32(blk[k] * np.float32(2.0 ** -e))
                want = nearest_positive(orc, E4M3, y) | (0x80 if np.signbit(y) else 0)
                assert r["q_row"][i, j * 128 + k] == want
    z = orc.quantize_block(np.zeros((1, 128), np.float32), (1, 128), pow2=True)
    assert z["s_row"][0, 0] == np.float32(2.0 ** -127) and not z["q_row"].any()


# ------------------------------------------------------------ blockwise 1x128 pow2 requantization
def test_block_requant_brute_force_tiny(orc):
    """The colwise copy from the rowwise codes and scales alone, recomputed
    here in float64: restore dec(q) * s (exact), take each 128-row column
    block's amax, e = floor(log2 a) - 8, and the brute-force nearest code of
    x_hat * 2^-e, stored transposed."""
    rng = np.random.default_rng(81)
    R, C = 128, 256
    x = (rng.standard_normal((R, C)) * np.exp2(rng.integers(-10, 10, (R, C)))).astype(np.float32)
    single = orc.quantize_block(x, (1, 128), pow2=True)
    rq = orc.requant_block_colwise(single["q_row"], single["s_row"])
    xhat = dec(orc, E4M3, single["q_row"]) * np.repeat(single["s_row"].astype(np.float64), 128, axis=1)
    for c in range(0, C, 17):
        col = xhat[:, c]
        e = int(np.floor(np.log2(np.abs(col).max()))) - 8
        assert rq["s_col"][c, 0] == np.float32(2.0 ** e)
        for r in range(R):
            y = col[r] * 2.0 ** -e                      # exact in float64
            want = nearest_positive(orc, E4M3, y) | (0x80 if np.signbit(y) else 0)
            assert rq["q_col"][c, r] == want, (c, r)


def test_block_requant_exact_on_grid(orc):
    """Values on the E4M3 grid whose every row tile and column block holds a
    +-256: every scale is 1 both ways, so the requantized colwise copy is
    the transpose of the rowwise codes, which is also the colwise copy
    quantized from the source."""
    rng = np.random.default_rng(83)
    R, C = 256, 384
    grid = np.array([orc.decode(E4M3, c) for c in range(0x08, 0x7F)])   # normal positives, 2^-6 .. 448
    grid = grid[grid < 256]
    x = (rng.choice(grid, (R, C)) * rng.choice([-1.0, 1.0], (R, C))).astype(np.float32)
    for r in range(R):
        x[r, (r * 3) % C] = 256.0 if r % 2 else -256.0      # every row tile of row r, and column block, gets one
        x[r, (r * 3 + 128) % C] = 256.0
        x[r, (r * 3 + 256) % C] = -256.0
    single = orc.quantize_block(x, (1, 128), outputs=ROW | COL, pow2=True)
    assert (single["s_row"] == 1.0).all() and (single["s_col"] == 1.0).all()
    rq = orc.requant_block_colwise(single["q_row"], single["s_row"])
    assert np.array_equal(rq["q_col"], single["q_row"].T)
    assert np.array_equal(rq["q_col"], single["q_col"]) and (rq["s_col"] == 1.0).all()


def test_block_requant_equals_single_quantization_where_exact(orc):
    """[MP] "FP8 通信": with power-of-two scales, the re-quantized colwise copy
    equals the colwise copy quantized from the source except at special
    values. Where an element's column block gets the same scale both ways and
    its scaled value is a normal, unsaturated E4M3 value in the row scaling
    and in the column scaling, the codes are equal."""
    R, C = 256, 384
    x = W.normal((R, C), 1.0, 85, W.BF16)
    xf = W.bf16_bits_to_f32(x).reshape(R, C)
    single = orc.quantize_block(x, (1, 128), outputs=ROW | COL, pow2=True)
    rq = orc.requant_block_colwise(single["q_row"], single["s_row"])
    s1 = np.repeat(single["s_col"].astype(np.float64), 128, axis=1)        # [C, R]
    s2 = np.repeat(rq["s_col"].astype(np.float64), 128, axis=1)
    sr = np.repeat(single["s_row"].astype(np.float64), 128, axis=1).T      # row-tile scale of each element, [C, R]
    xt = np.abs(xf.T).astype(np.float64)
    y_row, y_col = xt / sr, xt / s1
    exact = (s1 == s2) & (y_row >= 2.0 ** -6) & (y_col >= 2.0 ** -6) & (y_row <= 448) & (y_col <= 448)
    assert exact.mean() > 0.8
    assert np.array_equal(single["q_col"][exact], rq["q_col"][exact])
    assert (single["q_col"] == rq["q_col"]).mean() > 0.9


def test_block_requant_error_bound_and_zero(orc):
    x = W.normal((128, 256), 0.02, 87, W.BF16)
    single = orc.quantize_block(x, (1, 128), pow2=True)
    rq = orc.requant_block_colwise(single["q_row"], single["s_row"])
    xhat = orc.dequant_block(single["q_row"], single["s_row"], (1, 128)).T
    back = orc.dequant_block(rq["q_col"], rq["s_col"], (1, 128))
    ys = np.abs(xhat) / np.repeat(rq["s_col"].astype(np.float64), 128, axis=1)
    ok = (ys >= 2.0 ** -6) & (ys <= 448)
    assert ok.mean() > 0.9
    assert (np.abs(back - xhat)[ok] / np.abs(xhat)[ok]).max() <= 2.0 ** -4 * (1 + 1e-6)
    z = orc.quantize_block(np.zeros((128, 128), np.float32), (1, 128), pow2=True)
    rz = orc.requant_block_colwise(z["q_row"], z["s_row"])
    assert not rz["q_col"].any() and (rz["s_col"] == np.float32(2.0 ** -127)).all()
