"""Pins for the oracle's quantization recipes (CPU only).

Values the pages print (tests/golden), closed forms and invariants the
method implies, and brute force on tiny tensors.
"""
import numpy as np
import pytest

from conftest import golden
from fp8_fp4_tensor_amd import workloads as W

E4M3, E5M2, E2M1 = 0, 1, 2
ROW, COL = 1, 2


def f32bits(v):
    return int(np.array([v], np.float32).view(np.uint32)[0])


def dec(orc, fmt, q):
    return np.array([orc.decode(fmt, int(c)) for c in np.ravel(q)]).reshape(np.shape(q))


def nearest_positive(orc, fmt, a):
    """Brute-force nearest code magnitude over all positive codes, ties even."""
    vals = np.array([orc.decode(fmt, c) for c in range(orc.max_code(fmt) + 1)])
    a = min(abs(float(a)), vals[-1])
    d = np.abs(vals - a)
    cand = np.nonzero(d == d.min())[0]
    even = [c for c in cand if c % 2 == 0]
    return int(even[0] if even else cand[0])


# ------------------------------------------------------------ worked examples
def test_worked_example_current_scaling(orc):
    g = golden("cs_worked_example.json")
    x = np.array(g["x"], np.float32)
    r = orc.quantize_current(x, E4M3)
    assert r["amax"] == np.float32(g["amax"])
    alpha, s = orc.tensor_scales(r["amax"], orc.fmax(E4M3))
    assert alpha == np.float32(g["alpha"])                 # 0.448 in fp32
    assert s == np.float32(g["s_exact_ratio"][0]) / np.float32(g["s_exact_ratio"][1])
    assert round(float(s), 5) == g["s_approx"]
    assert r["s"] == s
    assert (f32bits(alpha), f32bits(s)) == (0x3EE56042, 0x400EDB6E)
    # scaled values and codes
    np.testing.assert_allclose((x * alpha).astype(np.float32), g["scaled"], rtol=1e-6)
    assert list(dec(orc, E4M3, r["q_row"]).ravel()) == g["q_values"]
    xhat = orc.dequant_tensor(r["q_row"], E4M3, r["s"]).ravel()
    assert [round(float(v), g["printed_decimals"]) for v in xhat] == g["xhat_approx"]
    # the page restores the extreme elements exactly
    assert xhat[0] == -1000.0 and xhat[2] == 1000.0


def test_error_example(orc):
    g = golden("cs_error_example.json")
    w = golden("cs_worked_example.json")
    x = np.array(w["x"], np.float32)
    r = orc.quantize_current(x, E4M3)
    alpha, _ = orc.tensor_scales(r["amax"], orc.fmax(E4M3))
    y = float(np.float32(x[1] * alpha))
    q = orc.decode(E4M3, r["q_row"].ravel()[1])
    assert round(q - y, 4) == g["scaled_error"]
    xhat = orc.dequant_tensor(r["q_row"], E4M3, r["s"]).ravel()[1]
    assert round(float(xhat - x[1]), 4) == g["restored_error_approx"]
    rel_scaled, rel_restored = abs(q - y) / abs(y), abs(float(xhat) - float(x[1])) / abs(float(x[1]))
    assert round(100 * rel_scaled, 2) == g["relative_error_percent_approx"]
    assert round(100 * rel_restored, 2) == g["relative_error_percent_approx"]


def test_underflow_example(orc):
    g = golden("cs_underflow_example.json")
    x = np.array(g["x"], np.float32)
    r = orc.quantize_current(x, E4M3)
    alpha, _ = orc.tensor_scales(r["amax"], orc.fmax(E4M3))
    np.testing.assert_allclose((x * alpha).astype(np.float32), g["scaled_approx"], rtol=1e-6)
    # both small values fall below half the smallest E4M3 subnormal (2^-10) and become +0
    assert list(r["q_row"].ravel()) == [0x00, 0x00, 0x7E]


def test_allgather_example_sharded_amax(orc):
    g = golden("cs_allgather_example.json")
    shards = [np.array(s, np.float32) for s in g["shards"]]
    local = [orc.amax(s) for s in shards]
    assert local == [np.float32(v) for v in g["local_amax"]]
    glob = max(local)
    assert glob == np.float32(g["global_amax"])
    alpha, _ = orc.tensor_scales(glob, orc.fmax(E4M3))
    assert alpha == np.float32(g["alpha_ratio"][0]) / np.float32(g["alpha_ratio"][1])
    # quantizing each shard with the global amax equals quantizing the whole tensor
    whole = orc.quantize_current(np.concatenate(shards), E4M3)
    parts = np.concatenate([orc.quantize_with_amax(s, E4M3, glob)["q_row"].ravel() for s in shards])
    assert np.array_equal(parts, whole["q_row"].ravel())
    assert list(dec(orc, E4M3, parts)) == [-44.0, 88.0, -448.0, 22.0]
    # with its own local amax, shard 0 quantizes differently (20 -> 448)
    own = orc.quantize_with_amax(shards[0], E4M3, local[0])["q_row"].ravel()
    assert list(own) == [0xF6, 0x7E]


# ------------------------------------------------------------ per-tensor current
def test_all_zero_tensor(orc):
    for fmt in (E4M3, E5M2):
        r = orc.quantize_current(np.zeros(4096, np.float32), fmt)
        assert r["amax"] == 0 and r["s"] == 1.0
        assert not r["q_row"].any()
    r = orc.quantize_current(-np.zeros(8, np.float32), E4M3)
    assert (r["q_row"] == 0x80).all()


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_amax_element_maps_to_fmax_and_error_bound(orc, fmt):
    std = 1.0 if fmt == E4M3 else 1e-3
    x = W.normal((64, 256), std, 123, W.BF16)
    r = orc.quantize_current(x, fmt, outputs=ROW | COL)
    xf = W.bf16_bits_to_f32(x).reshape(64, 256)
    a = np.abs(xf).max()
    assert r["amax"] == a
    top = orc.max_code(fmt)
    at = np.abs(xf) == a
    assert (r["q_row"][at] & 0x7F == top).all()
    assert ((r["q_row"][at] >> 7) == (xf[at] < 0)).all()
    # relative error: half an ulp of the mantissa (2^-4 for E4M3, 2^-3 for E5M2) in the normal range
    xhat = orc.dequant_tensor(r["q_row"], fmt, r["s"])
    min_normal = 2.0 ** -6 if fmt == E4M3 else 2.0 ** -14
    normal = np.abs(xf) * (orc.fmax(fmt) / a) >= min_normal
    rel = np.abs(xhat - xf)[normal] / np.abs(xf)[normal]
    assert rel.max() <= (2.0 ** -4 if fmt == E4M3 else 2.0 ** -3) * (1 + 2.0 ** -20)
    # colwise copy is the transposed rowwise bytes
    assert np.array_equal(r["q_col"], r["q_row"].T)


def test_current_brute_force_tiny(orc):
    rng = np.random.default_rng(5)
    for trial in range(200):
        n = int(rng.integers(1, 9))
        x = (rng.standard_normal(n) * 10.0 ** rng.integers(-6, 4)).astype(np.float32)
        fmt = int(rng.integers(0, 2))
        r = orc.quantize_current(x, fmt)
        a = max(abs(float(v)) for v in x)
        alpha = np.float32(orc.fmax(fmt)) / np.float32(a)
        for i in range(n):
            y = np.float32(x[i] * alpha)
            want = nearest_positive(orc, fmt, y) | (0x80 if np.signbit(y) else 0)
            assert r["q_row"].ravel()[i] == want


def test_small_workload_outliers(orc):
    w = W.SMALL_CURRENT
    x = w.make()
    r = orc.quantize_current(x.ravel(), E4M3)
    assert r["amax"] == 1000.0
    assert f32bits(r["s"]) == 0x400EDB6E
    assert (np.abs(x) == 1000.0).sum() == 64
    assert (r["q_row"].ravel()[np.abs(x.ravel()) == 1000.0] & 0x7F == 0x7E).all()


# ------------------------------------------------------------ delayed
def test_delayed_repeat_input_equals_current(orc):
    x = W.normal((32, 64), 1.0, 9, W.BF16)
    st = orc.DelayedState(1024)
    r0 = orc.quantize_delayed(x, E4M3, st)
    # step 0 used alpha = 1 (the initial state)
    xf = W.bf16_bits_to_f32(x)
    assert np.array_equal(r0["q_row"].ravel(), orc.encode_array(E4M3, xf).ravel())
    r1 = orc.quantize_delayed(x, E4M3, st)
    cur = orc.quantize_current(x, E4M3)
    assert np.array_equal(r1["q_row"], cur["q_row"])
    assert st.s == cur["s"]


def test_delayed_window_expiry(orc):
    """An outlier at step 0 shapes the scale of steps 1..H and no later one."""
    H = 1024
    big = np.full((1, 8), 1000.0, np.float32)
    small = np.array([[1.0, -0.5, 0.25, 2.0, -2.0, 0.1, 0.0, 1.5]], np.float32)
    st = orc.DelayedState(H)
    orc.quantize_delayed(big, E4M3, st)
    alphas = []
    for t in range(1, H + 2):
        r = orc.quantize_delayed(small, E4M3, st)
        alphas.append(st.alpha)
    a_big, _ = orc.tensor_scales(1000.0, 448.0)
    a_small, _ = orc.tensor_scales(2.0, 448.0)
    # alpha after step t (used by step t+1) is from max over the last H amaxes
    assert all(a == a_big for a in alphas[: H - 1])       # after steps 1..H-1
    assert alphas[H - 1] == a_small                        # after step H, hist[0] was overwritten
    # so step H+1 = 1025 is the first step cast with a scale free of the outlier
    assert len(alphas) == H + 1


def test_delayed_ring_matches_window_max(orc):
    rng = np.random.default_rng(3)
    H = 5
    st = orc.DelayedState(H)
    amaxes = []
    for t in range(23):
        x = (rng.standard_normal((4, 16)) * 10.0 ** rng.uniform(-2, 2)).astype(np.float32)
        alpha_used = st.alpha
        r = orc.quantize_delayed(x, E5M2, st)
        assert np.array_equal(r["q_row"].ravel(), orc.encode_array(E5M2, (x.ravel() * alpha_used).astype(np.float32)))
        amaxes.append(np.abs(x).max())
        assert r["amax"] == amaxes[-1]
        m = max(amaxes[-H:])
        assert (st.alpha, st.s) == orc.tensor_scales(m, 57344.0)
        assert sorted(st.hist.tolist()) == sorted(amaxes[-H:] + [0.0] * (H - len(amaxes[-H:])))
        # ring order (the state layout a checkpoint holds): step t's amax in slot t mod H
        assert st.hist[t % H] == amaxes[-1]
        assert all(st.hist[(t - k) % H] == amaxes[-1 - k] for k in range(min(H, t + 1)))


def test_delayed_zero_window_keeps_scale(orc):
    st = orc.DelayedState(4)
    for _ in range(3):
        r = orc.quantize_delayed(np.zeros((2, 8), np.float32), E4M3, st)
        assert st.alpha == 1.0 and st.s == 1.0 and not r["q_row"].any()
    # a window that empties after a nonzero step keeps the last scale (it is
    # not reset to 1): H = 2, one step of amax 3, then zeros
    st = orc.DelayedState(2)
    orc.quantize_delayed(np.full((2, 8), 3.0, np.float32), E4M3, st)
    kept = orc.tensor_scales(3.0, 448.0)
    for t in range(3):
        orc.quantize_delayed(np.zeros((2, 8), np.float32), E4M3, st)
        assert (st.alpha, st.s) == kept, t
    assert not st.hist.any()


# ------------------------------------------------------------ blockwise
@pytest.mark.parametrize("block", [(1, 128), (128, 128)])
def test_block_invariants(orc, block):
    br, bc = block
    R, C = 256, 384
    x = W.normal((R, C), 1.0 if br == 1 else 0.02, 77, W.BF16)
    r = orc.quantize_block(x, block, outputs=ROW | COL)
    xf = W.bf16_bits_to_f32(x).reshape(R, C)
    tiles = xf.reshape(R // br, br, C // bc, bc)
    qt = r["q_row"].reshape(R // br, br, C // bc, bc)
    a = np.abs(tiles).max(axis=(1, 3))
    assert np.array_equal(r["s_row"], (a / np.float32(448.0)).astype(np.float32))
    for i in range(R // br):
        for j in range(C // bc):
            m = np.abs(tiles[i, :, j, :]) == a[i, j]
            assert (qt[i, :, j, :][m] & 0x7F == 0x7E).all()
    xhat = orc.dequant_block(r["q_row"], r["s_row"], block)
    scaled = np.abs(xf) * np.repeat(np.repeat(448.0 / a, br, axis=0), bc, axis=1)
    ok = scaled >= 2.0 ** -6
    assert (np.abs(xhat - xf)[ok] / np.abs(xf)[ok]).max() <= 2.0 ** -4 * (1 + 2.0 ** -20)
    if br == 128:
        # a square tile quantizes to the same values in either direction
        rt = orc.quantize_block(np.ascontiguousarray(x.T), block)
        assert np.array_equal(r["q_col"], rt["q_row"]) and np.array_equal(r["s_col"], rt["s_row"])
        assert np.array_equal(r["q_col"], r["q_row"].T)
    else:
        # 1-D colwise tiles run down the columns of X
        rt = orc.quantize_block(np.ascontiguousarray(x.T), block)
        assert np.array_equal(r["q_col"], rt["q_row"]) and np.array_equal(r["s_col"], rt["s_row"])
        colamax = np.abs(xf).reshape(R // bc, bc, C).max(axis=1).T
        assert np.array_equal(r["s_col"], (colamax / np.float32(448.0)).astype(np.float32))


def test_block_brute_force_tiny(orc):
    rng = np.random.default_rng(17)
    x = (rng.standard_normal((2, 256)) * np.exp2(rng.integers(-8, 8, (2, 256)))).astype(np.float32)
    r = orc.quantize_block(x, (1, 128))
    for i in range(2):
        for j in range(2):
            blk = x[i, j * 128:(j + 1) * 128]
            a = np.abs(blk).max()
            alpha = np.float32(448.0) / a
            for k in range(128):
                y = np.float32(blk[k] * alpha)
                want = nearest_positive(orc, E4M3, y) | (0x80 if np.signbit(y) else 0)
                assert r["q_row"][i, j * 128 + k] == want


def test_block_zero_tile(orc):
    x = np.zeros((1, 256), np.float32)
    x[0, 200] = 3.0
    r = orc.quantize_block(x, (1, 128))
    assert r["s_row"][0, 0] == 1.0 and not r["q_row"][0, :128].any()
    assert r["q_row"][0, 200] == 0x7E


# ------------------------------------------------------------ MXFP8
def test_mx_code_closed_form_all_bf16(orc):
    """code = max(E - 8, 0), E the biased exponent field of the fp32 amax."""
    b = np.arange(0x0000, 0x7F80, dtype=np.uint32)        # every non-negative finite bf16
    a = (b << 16).view(np.float32)
    E = (a.view(np.uint32) >> 23) & 0xFF
    want = np.maximum(E.astype(np.int64) - 8, 0)
    got = np.array([orc.mx_code(v) for v in a])
    assert np.array_equal(got, want)


def test_mx_invariants(orc):
    R, C = 64, 96
    x = W.student_t((R, C), 3.0, 41, W.BF16)
    r = orc.quantize_mx(x)
    xf = W.bf16_bits_to_f32(x).reshape(R, C)
    for mat, q, codes in ((xf, r["q_row"], r["e_row"]), (xf.T.copy(), r["q_col"], r["e_col"])):
        rr, cc = mat.shape
        blocks = mat.reshape(rr, cc // 32, 32)
        a = np.abs(blocks).max(axis=2)
        assert np.array_equal(codes, np.array([[orc.mx_code(v) for v in row] for row in a]))
        scale = np.exp2(codes.astype(np.float64) - 127)
        # the largest element of a block scales into [256, 512) and codes to 256..448
        y = a / scale
        assert ((y >= 256) & (y < 512)).all()
        qb = q.reshape(rr, cc // 32, 32)
        for i in range(rr):
            for j in range(cc // 32):
                m = np.abs(blocks[i, j]) == a[i, j]
                vals = np.abs(dec(orc, E4M3, qb[i, j][m]))
                assert ((vals >= 256) & (vals <= 448)).all()
        xhat = orc.dequant_mx(q, codes)
        ys = np.abs(mat) / np.repeat(scale, 32, axis=1)
        ok = (ys >= 2.0 ** -6) & (ys <= 448)
        assert (np.abs(xhat - mat)[ok] / np.abs(mat)[ok]).max() <= 2.0 ** -4 * (1 + 1e-6)
    # colwise is the rowwise recipe on the transpose
    rt = orc.quantize_mx(np.ascontiguousarray(x.T), outputs=ROW)
    assert np.array_equal(r["q_col"], rt["q_row"]) and np.array_equal(r["e_col"], rt["e_row"])


def test_mx_brute_force_tiny(orc):
    rng = np.random.default_rng(23)
    x = (rng.standard_t(3, (2, 64)) * 10.0 ** rng.integers(-3, 3)).astype(np.float32)
    r = orc.quantize_mx(x, outputs=ROW)
    for i in range(2):
        for j in range(2):
            blk = x[i, j * 32:(j + 1) * 32]
            a = float(np.abs(blk).max())
            e = int(np.floor(np.log2(a))) - 8
            assert r["e_row"][i, j] == e + 127
            for k in range(32):
                y = np.float32(blk[k] * np.float32(2.0 ** -e))
                want = nearest_positive(orc, E4M3, y) | (0x80 if np.signbit(y) else 0)
                assert r["q_row"][i, j * 32 + k] == want


def test_mx_zero_block(orc):
    x = np.zeros((32, 32), np.float32)
    r = orc.quantize_mx(x)
    assert not r["e_row"].any() and not r["q_row"].any() and not r["e_col"].any()


# ------------------------------------------------------------ NVFP4
def unpack(p):
    lo, hi = p & 0xF, p >> 4
    out = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return out


@pytest.mark.parametrize("block", [(1, 16), (16, 16)])
def test_nvfp4_structure(orc, block):
    br, bc = block
    R, C = 64, 128
    x = W.normal((R, C), 1.0 if br == 1 else 0.02, 55, W.BF16)
    r = orc.quantize_nvfp4(x, block, outputs=ROW | COL)
    xf = W.bf16_bits_to_f32(x).reshape(R, C)
    A = np.abs(xf).max()
    assert r["amax"] == A
    nib = unpack(r["p_row"])
    tiles = xf.reshape(R // br, br, C // bc, bc)
    a = np.abs(tiles).max(axis=(1, 3))
    codes = r["c_row"]
    # the block holding the tensor amax gets the E4M3 code of 448
    assert (codes[a == A] == 0x7E).all()
    assert (codes < 0x7F).all()                            # block codes are positive E4M3
    dB = dec(orc, E4M3, codes).astype(np.float32) * r["S"]
    nb = nib.reshape(R // br, br, C // bc, bc)
    for i in range(R // br):
        for j in range(C // bc):
            if codes[i, j] < 0x08:
                continue                                   # E4M3 subnormal block scale: coarse
            m = np.abs(tiles[i, :, j, :]) == a[i, j]
            # every block's largest element lands on +-6
            assert (nb[i, :, j, :][m] & 0x7 == 0x7).all()
    # restored values are within a quarter of the block scale (half the widest FP4 gap
    # below 1) or 20 percent above it, unless the element sits at the top
    xhat = orc.dequant_nvfp4(r["p_row"], codes, r["S"], block)
    d = np.repeat(np.repeat(dB, br, axis=0), bc, axis=1)
    y = np.abs(xf) / d
    err = np.abs(xhat - xf)
    small = y < 1
    assert (err[small] <= 0.25 * d[small] * (1 + 1e-5)).all()
    mid = (y >= 1) & (y <= 6)
    assert (err[mid] <= 0.2 * np.abs(xf[mid]) * (1 + 1e-5)).all()
    if br == 16:
        assert np.array_equal(unpack(r["p_col"]), nib.T)
        assert np.array_equal(r["c_col"], codes.T)
    else:
        rt = orc.quantize_nvfp4(np.ascontiguousarray(x.T), block)
        assert np.array_equal(r["p_col"], rt["p_row"]) and np.array_equal(r["c_col"], rt["c_row"])
        assert rt["S"] == r["S"]


def test_nvfp4_nibble_order(orc):
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1] = 6.0, -3.0
    r = orc.quantize_nvfp4(x, (1, 16))
    # element 0 in the low nibble, element 1 in the high nibble
    assert r["p_row"][0, 0] == (0x7 | (0xD << 4))


def test_nvfp4_zero_tensor(orc):
    r = orc.quantize_nvfp4(np.zeros((16, 32), np.float32), (16, 16))
    assert r["S"] == 1.0 and not r["p_row"].any() and not r["c_row"].any()


# ------------------------------------------------------------ bf16 output, MX requantization
def test_f32_to_bf16_matches_torch(orc):
    import torch
    rng = np.random.default_rng(31)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    y = bits.view(np.float32)
    y = y[np.isfinite(y)]
    # values just below the bf16 overflow threshold round to the largest bf16 or to inf, as torch does
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f32_to_bf16(y), ref)
    ties = (np.arange(1, 4096, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    ref = torch.from_numpy(ties).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f32_to_bf16(ties), ref)


def test_mx_requant_equals_single_quantization_where_exact(orc):
    """[MP] "FP8 通信": with power-of-two scales, de-quantizing the rowwise copy
    and re-quantizing it down the columns gives the same bytes as quantizing
    the source down the columns, except for special values such as
    subnormals. Precisely: when an element's column block gets the same code
    both ways and its scaled value is a normal, unsaturated E4M3 value in
    both the row scaling and the column scaling, the codes are equal."""
    R, C = 96, 128
    x = W.student_t((R, C), 3.0, 61, W.BF16)
    xf = W.bf16_bits_to_f32(x).reshape(R, C)
    single = orc.quantize_mx(x)                      # colwise from the source
    rq = orc.requant_mx_colwise(single["q_row"], single["e_row"])
    q1, q2 = single["q_col"], rq["q_col"]            # both [C, R]
    c1 = np.repeat(single["e_col"].astype(np.int64), 32, axis=1)
    c2 = np.repeat(rq["e_col"].astype(np.int64), 32, axis=1)
    er = np.repeat(single["e_row"].astype(np.int64), 32, axis=1).T   # row-block code of each element, [C, R]
    xt = np.abs(xf.T).astype(np.float64)
    y_row = xt * 2.0 ** (127 - er)
    y_col = xt * 2.0 ** (127 - c1)
    exact = (c1 == c2) & (y_row >= 2.0 ** -6) & (y_col >= 2.0 ** -6) & (y_row <= 448) & (y_col <= 448)
    assert exact.mean() > 0.8
    assert np.array_equal(q1[exact], q2[exact])
    # and the codes agree for almost every element overall
    assert (q1 == q2).mean() > 0.9


def test_mx_requant_error_bound(orc):
    x = W.normal((64, 64), 1.0, 62, W.BF16)
    single = orc.quantize_mx(x)
    rq = orc.requant_mx_colwise(single["q_row"], single["e_row"])
    xhat = orc.dequant_mx(single["q_row"], single["e_row"]).T       # restored values, transposed
    back = orc.dequant_mx(rq["q_col"], rq["e_col"])
    scale = np.repeat(np.exp2(rq["e_col"].astype(np.float64) - 127), 32, axis=1)
    ys = np.abs(xhat) / scale
    ok = (ys >= 2.0 ** -6) & (ys <= 448)
    assert (np.abs(back - xhat)[ok] / np.abs(xhat)[ok]).max() <= 2.0 ** -4 * (1 + 1e-6)
