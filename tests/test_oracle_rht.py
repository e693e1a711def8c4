"""Pins of the oracle's random Hadamard transform (CPU only).

The pages ([LP] section 2.4 item 3) name an RHT on the weight-gradient GEMM
inputs before NVFP4 quantization, to spread block outliers, without size,
signs or arithmetic; the oracle's reading is y = (1/4) H16 diag(s) x per
16-element chunk along the contraction, computed by the fp32 fast
Walsh-Hadamard butterfly. These tests pin it against a Hadamard matrix built
here by Kronecker products (exact on integers, within the butterfly's
rounding bound on arbitrary fp32), against orthogonality (the fp64 inverse
recovers x, GEMM products are preserved), and the RHT recipe against the
plain NVFP4 recipe applied to the transformed tensor; a soft test checks
the pages' stated purpose (block outliers spread over the block, so they no
longer set the block amax alone)."""
import numpy as np
import pytest

ROW, COL = 1, 2


def hadamard16():
    H = np.array([[1.0]])
    for _ in range(4):
        H = np.kron(H, np.array([[1.0, 1.0], [1.0, -1.0]]))
    return H


H16 = hadamard16()


def sign_vec(signs):
    return np.array([-1.0 if (signs >> i) & 1 else 1.0 for i in range(16)])


def exact_rht(x, signs):
    """fp64 (1/4) H16 diag(s) x for each 16-chunk of x."""
    xc = x.reshape(-1, 16).astype(np.float64) * sign_vec(signs)
    return (xc @ H16.T / 4.0).reshape(x.shape)


def test_hadamard_is_sylvester_and_orthogonal():
    i = np.arange(16)
    pop = np.array([[bin(a & b).count("1") for b in i] for a in i])
    assert np.array_equal(H16, (-1.0) ** pop)
    assert np.array_equal(H16 @ H16.T, 16 * np.eye(16))


@pytest.mark.parametrize("signs", [0x0000, 0xFFFF, 0xA5C3, 0x1234])
def test_rht_exact_on_integers(orc, signs):
    rng = np.random.default_rng(signs)
    x = rng.integers(-1000, 1000, 16 * 64).astype(np.float32)
    assert np.array_equal(orc.rht16(x, signs).astype(np.float64), exact_rht(x, signs))


def test_rht_one_hot_columns(orc):
    for signs in (0, 0x8001, 0x7FFE):
        s = sign_vec(signs)
        for i in range(16):
            e = np.zeros(16, np.float32)
            e[i] = 1.0
            assert np.array_equal(orc.rht16(e, signs), (s[i] * H16[i] / 4).astype(np.float32))


def test_rht_rounding_bound_and_inverse(orc):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(16 * 4096) * np.exp2(rng.integers(-20, 20, 16 * 4096))).astype(np.float32)
    signs = 0xB00F
    y = orc.rht16(x, signs).astype(np.float64)
    ex = exact_rht(x, signs)
    # four rounded additions per output: |err| <= gamma_4 * sum|x_i| / 4
    u = 2.0 ** -24
    gamma4 = 4 * u / (1 - 4 * u)
    bound = gamma4 * np.abs(x.astype(np.float64)).reshape(-1, 16).sum(axis=1, keepdims=True) / 4
    assert np.all(np.abs(y - ex).reshape(-1, 16) <= bound)
    # orthogonal: x = diag(s) H16 y / 4
    back = (y.reshape(-1, 16) @ H16 / 4.0) * sign_vec(signs)
    scale = np.abs(x.astype(np.float64)).reshape(-1, 16).sum(axis=1, keepdims=True)
    assert np.all(np.abs(back - x.reshape(-1, 16)) <= 8 * u * scale)


def test_rht_preserves_gemm_along_the_contraction(orc):
    rng = np.random.default_rng(4)
    M, K, N = 64, 24, 40
    X = rng.standard_normal((M, K)).astype(np.float32)
    G = rng.standard_normal((M, N)).astype(np.float32)
    signs = 0x5A5A
    XT = orc.rht16(np.ascontiguousarray(X.T), signs).astype(np.float64)   # rows of X^T along M
    GT = orc.rht16(np.ascontiguousarray(G.T), signs).astype(np.float64)
    want = G.T.astype(np.float64) @ X.astype(np.float64)
    assert np.allclose(GT @ XT.T, want, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("sr", [None, (7, 3)])
def test_rht_recipe_is_nvfp4_of_the_transformed_tensor(orc, sr):
    rng = np.random.default_rng(5)
    R, C = 64, 48
    x = rng.standard_normal((R, C)).astype(np.float32)
    signs = 0x6C1B
    r = orc.quantize_nvfp4_rht(x, signs, sr=sr)
    yt = orc.rht16(np.ascontiguousarray(x.T), signs).reshape(C, R)
    plain = orc.quantize_nvfp4(np.ascontiguousarray(yt.T), (1, 16), outputs=COL, sr=sr)
    assert np.array_equal(r["p_col"], plain["p_col"]) and np.array_equal(r["c_col"], plain["c_col"])
    assert r["S"] == plain["S"] and r["amax"] == np.float32(np.abs(yt).max())
    # a given amax (e.g. reduced across shards) replaces the tensor's own
    g = orc.quantize_nvfp4_rht(x, signs, amax=4 * r["amax"], sr=sr)
    plain_g = orc.quantize_nvfp4(np.ascontiguousarray(yt.T), (1, 16), outputs=COL, sr=sr, amax=4 * r["amax"])
    assert np.array_equal(g["p_col"], plain_g["p_col"]) and g["S"] == plain_g["S"]


def test_rht_spreads_block_outliers(orc):
    """The pages' stated purpose: a block's outlier is spread over its 16
    values, so it no longer dominates the block amax. Checked as the crest
    factor max|v| / rms(v) of the blocks that hold an outlier (at most 4 for
    any 16 values, 4 times smaller after the transform for a lone spike).
    (Training-level benefits are outside what a CPU test can show.)"""
    rng = np.random.default_rng(6)
    R, C = 256, 64
    x = rng.standard_normal((R, C)).astype(np.float32)
    hot = rng.random((R, C)) < 1 / 128
    x[hot] *= 40.0
    signs = 0x3C96
    xt = np.ascontiguousarray(x.T).reshape(-1, 16).astype(np.float64)
    yt = orc.rht16(np.ascontiguousarray(x.T), signs).reshape(-1, 16).astype(np.float64)
    outlier_blocks = np.ascontiguousarray(hot.T).reshape(-1, 16).any(axis=1)
    assert outlier_blocks.sum() > 50

    def crest(b):
        return np.abs(b).max(axis=1) / np.sqrt((b ** 2).mean(axis=1))
    before, after = crest(xt[outlier_blocks]).mean(), crest(yt[outlier_blocks]).mean()
    assert before > 3.0 and after < 1.6, (before, after)
    # the transformed blocks carry the same energy (orthogonal transform)
    assert np.allclose((yt ** 2).sum(axis=1), (xt ** 2).sum(axis=1), rtol=1e-5)


def stage_factor(h):
    """The butterfly stage that pairs index i with i + h (bit h of i clear)
    as a matrix: I_(16/2h) kron H2 kron I_h, entries 0 and +-1."""
    return np.kron(np.kron(np.eye(16 // (2 * h)), np.array([[1.0, 1.0], [1.0, -1.0]])), np.eye(h))


def factored_rht_f32(x, signs, order):
    """(1/4) H16 diag(s) x with H16 applied as its four Kronecker factors,
    one float32 matrix product per factor in the given order. Each output of
    a factor has two nonzero terms, so each product rounds a + b or a - b
    once to float32, as one butterfly stage does. (The zero entries add +0
    terms, so the sign of an exact zero result may differ from a butterfly's;
    values compare equal.)"""
    w = (x.reshape(-1, 16) * sign_vec(signs).astype(np.float32)).astype(np.float32)
    for h in order:
        w = np.matmul(w, stage_factor(h).T.astype(np.float32)).astype(np.float32)
    return (w * np.float32(0.25)).reshape(x.shape)


def test_stage_factors_multiply_to_h16():
    P = np.eye(16)
    for h in (1, 2, 4, 8):
        P = stage_factor(h) @ P
    assert np.array_equal(P, H16)


def test_rht_fp32_stage_order(orc):
    """The oracle's fp32 arithmetic is the stated reading: stages h = 1, 2,
    4, 8 in that order (a different order rounds differently on inputs that
    span many binades, and the test checks that it would be caught)."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(16 * 8192) * np.exp2(rng.integers(-30, 30, 16 * 8192))).astype(np.float32)
    for signs in (0x0000, 0xB00F, 0x6C1B):
        y = orc.rht16(x, signs)
        assert np.array_equal(y, factored_rht_f32(x, signs, (1, 2, 4, 8)))
        assert not np.array_equal(y, factored_rht_f32(x, signs, (8, 4, 2, 1)))
        assert not np.array_equal(y, factored_rht_f32(x, signs, (2, 1, 4, 8)))
