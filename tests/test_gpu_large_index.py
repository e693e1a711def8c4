"""GPU parity beyond 2^31 elements: 64-bit indexing in every kernel family.

The input is 65664 x 32768 bf16 (2.15e9 elements, 4.3 GB), built on the GPU
row chunk by row chunk from an integer formula whose values are exact in
bf16: x[r, c] = (((1103 r + 2221 c) mod 256) - 128) / 64 * 2^((r + c // 128) mod 8).
The oracle regenerates sampled rows (and columns) exactly in numpy and checks
them bit for bit, including rows whose elements lie past index 2^31, and
colwise planes (rows of X^T) past that index: per-tensor, blockwise, MXFP8,
MXFP4, NVFP4 (with and without the RHT), dequantization, the MX and
power-of-two blockwise requantizations, and stochastic rounding of 8-bit
elements (per-tensor, MX and blockwise 1x128, both planes). The tensor amax is 256 by
construction (k = -128 at scale 2^7 occurs)."""
import numpy as np
import pytest
import torch

import oracle as orc
from fp8_fp4_tensor_amd import fq
from gpu_util import f32, host, same_bytes

pytestmark = pytest.mark.gpu

R, C = 65664, 32768          # R % 128 == 0; R * C > 2^31
AMAX = 256.0


def values(r, c):
    """The input at rows r (column vector) and columns c (row vector), fp32 (exact bf16)."""
    r = np.asarray(r, np.int64)
    c = np.asarray(c, np.int64)
    k = ((1103 * r + 2221 * c) % 256) - 128
    return (k.astype(np.float32) / np.float32(64.0)) * np.exp2(((r + c // 128) % 8).astype(np.float32))


def bf16_bits(v):
    return (np.ascontiguousarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.fixture(scope="module")
def big():
    x = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    c = torch.arange(C, device="cuda", dtype=torch.int32)
    step = 2048
    for r0 in range(0, R, step):
        r = torch.arange(r0, min(r0 + step, R), device="cuda", dtype=torch.int32)[:, None]
        k = ((1103 * r + 2221 * c) % 256) - 128
        e = ((r + c // 128) % 8).to(torch.float32)
        x[r0:r0 + step] = (k.to(torch.float32) / 64.0 * torch.exp2(e)).to(torch.bfloat16)
    torch.cuda.synchronize()
    # spot check the construction against the numpy formula
    rows = [0, R - 1]
    assert np.array_equal(host(x[rows].view(torch.int16)).view(np.uint16),
                          bf16_bits(values(np.array(rows)[:, None], np.arange(C)[None, :])))
    yield x
    del x
    torch.cuda.empty_cache()


SAMPLE_ROWS = np.array([0, 65536, R - 2, R - 1])       # rows past element 2^31 = row 65536
SAMPLE_COLS = np.array([0, 12345, C - 2, C - 1])        # colwise planes: X^T rows past element 2^31


def sample(xg_rows):
    return bf16_bits(values(SAMPLE_ROWS[:, None], np.arange(C)[None, :]))


def sample_cols():
    """Columns SAMPLE_COLS of X as rows ([len, R]): the rows of X^T that colwise planes hold."""
    return bf16_bits(values(np.arange(R)[:, None], SAMPLE_COLS[None, :]).T.copy())


def quantize(d, x):
    out = fq.alloc_quantized(d)
    fq.fq_quantize(d, x, out, fq.alloc_workspace(d))
    torch.cuda.synchronize()
    return out


def test_large_current(big):
    d = fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (0, 0), fq.FQ_ROWWISE)
    out = quantize(d, big)
    same_bytes(host(out.amax), f32(AMAX), "tensor amax")
    want = orc.quantize_with_amax(sample(None), orc.E4M3, AMAX, shape=(len(SAMPLE_ROWS), C))
    same_bytes(host(out.tensor_scale), f32(want["s"]), "scale")
    same_bytes(host(out.row_data[SAMPLE_ROWS]), want["q_row"], "codes of sampled rows")
    del out


@pytest.mark.parametrize("block", [(1, 128), (128, 128)])
def test_large_block(big, block):
    d = fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, block, fq.FQ_ROWWISE)
    out = quantize(d, big)
    br = block[0]
    rows = SAMPLE_ROWS if br == 1 else np.arange(R - 128, R)     # the last tile row
    xs = bf16_bits(values(rows[:, None], np.arange(C)[None, :]))
    want = orc.quantize_block(xs, block)
    same_bytes(host(out.row_data[rows]), want["q_row"], "codes")
    srow = rows if br == 1 else [R // 128 - 1]
    same_bytes(host(out.row_scale.view(R // br, C // 128)[srow]), want["s_row"], "scales")
    del out


def test_large_mx_both_planes(big):
    d = fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 32), fq.FQ_ROWWISE | fq.FQ_COLWISE)
    out = quantize(d, big)
    want = orc.quantize_mx(sample(None), outputs=orc.ROWWISE)
    same_bytes(host(out.row_data[SAMPLE_ROWS]), want["q_row"], "rowwise codes")
    same_bytes(host(out.row_scale.view(R, C // 32)[SAMPLE_ROWS]), want["e_row"], "rowwise E8M0")
    cols = np.array([0, 12345, C - 1])
    xc = bf16_bits(values(np.arange(R)[:, None], cols[None, :]).T.copy())   # X^T rows = columns of X
    wc = orc.quantize_mx(xc, outputs=orc.ROWWISE)
    same_bytes(host(out.col_data[cols]), wc["q_row"], "colwise codes (columns of X)")
    same_bytes(host(out.col_scale.view(C, R // 32)[cols]), wc["e_row"], "colwise E8M0")
    del out


def test_large_nvfp4(big):
    d = fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (1, 16), fq.FQ_ROWWISE)
    out = quantize(d, big)
    same_bytes(host(out.amax), f32(AMAX), "tensor amax")
    want = orc.quantize_nvfp4(sample(None), (1, 16), amax=AMAX)
    same_bytes(host(out.tensor_scale), f32(want["S"]), "tensor scale")
    same_bytes(host(out.row_data[SAMPLE_ROWS]), want["p_row"], "packed FP4")
    same_bytes(host(out.row_scale.view(R, C // 16)[SAMPLE_ROWS]), want["c_row"], "E4M3 block scales")
    del out


def test_large_nvfp4_1x16_both_planes(big):
    """Both planes of 1x16 blocks from one block pass: sampled rows of X and
    sampled rows of X^T, past element 2^31 in each plane."""
    d = fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (1, 16), fq.FQ_ROWWISE | fq.FQ_COLWISE)
    out = quantize(d, big)
    same_bytes(host(out.amax), f32(AMAX), "tensor amax")
    want_r = orc.quantize_nvfp4(sample(None), (1, 16), amax=AMAX)
    same_bytes(host(out.tensor_scale), f32(want_r["S"]), "tensor scale")
    same_bytes(host(out.row_data[SAMPLE_ROWS]), want_r["p_row"], "packed FP4 rows")
    same_bytes(host(out.row_scale.view(R, C // 16)[SAMPLE_ROWS]), want_r["c_row"], "E4M3 block scales of rows")
    want_c = orc.quantize_nvfp4(sample_cols(), (1, 16), amax=AMAX)
    same_bytes(host(out.col_data[SAMPLE_COLS]), want_c["p_row"], "packed FP4 of X^T rows")
    same_bytes(host(out.col_scale.view(C, R // 16)[SAMPLE_COLS]), want_c["c_row"], "E4M3 block scales of X^T rows")
    del out


def test_large_nvfp4_16x16_both_planes(big):
    """Both planes of 16x16 blocks from one block pass: the last block row of
    X and the last block column (the last 16 rows of X^T), past element 2^31
    in each plane."""
    d = fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (16, 16), fq.FQ_ROWWISE | fq.FQ_COLWISE)
    out = quantize(d, big)
    same_bytes(host(out.amax), f32(AMAX), "tensor amax")
    rows = np.arange(R - 16, R)
    want_r = orc.quantize_nvfp4(bf16_bits(values(rows[:, None], np.arange(C)[None, :])), (16, 16), amax=AMAX)
    same_bytes(host(out.tensor_scale), f32(want_r["S"]), "tensor scale")
    same_bytes(host(out.row_data[rows]), want_r["p_row"], "packed FP4, last block row")
    same_bytes(host(out.row_scale.view(R // 16, C // 16)[-1:]), want_r["c_row"], "E4M3 codes, last block row")
    cols = np.arange(C - 16, C)
    xc = bf16_bits(values(np.arange(R)[:, None], cols[None, :]))
    want_c = orc.quantize_nvfp4(xc, (16, 16), outputs=orc.COLWISE, amax=AMAX)
    same_bytes(host(out.col_data[cols]), want_c["p_col"], "packed FP4 of X^T, last block row")
    same_bytes(host(out.col_scale.view(C // 16, R // 16)[-1:]), want_c["c_col"], "E4M3 codes of X^T")
    del out


def test_large_current_colwise_and_dequant(big):
    d = fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (0, 0), fq.FQ_ROWWISE | fq.FQ_COLWISE)
    out = quantize(d, big)
    want_c = orc.quantize_with_amax(sample_cols(), orc.E4M3, AMAX, shape=(len(SAMPLE_COLS), R))
    same_bytes(host(out.col_data[SAMPLE_COLS]), want_c["q_row"], "colwise codes (columns of X)")
    want_r = orc.quantize_with_amax(sample(None), orc.E4M3, AMAX, shape=(len(SAMPLE_ROWS), C))
    same_bytes(host(out.row_data[SAMPLE_ROWS]), want_r["q_row"], "rowwise codes")
    y = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    fq.fq_dequantize(d, out, fq.FQ_ROWWISE, y)
    torch.cuda.synchronize()
    same_bytes(host(y[SAMPLE_ROWS].view(torch.int16)).view(np.uint16),
               orc.f32_to_bf16(orc.dequant_tensor(want_r["q_row"], orc.E4M3, want_r["s"])), "dequantized rows (bf16)")
    del out, y


def test_large_block_1x128_colwise(big):
    d = fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 128), fq.FQ_COLWISE)
    out = quantize(d, big)
    want = orc.quantize_block(sample_cols(), (1, 128))
    same_bytes(host(out.col_data[SAMPLE_COLS]), want["q_row"], "colwise codes (columns of X)")
    same_bytes(host(out.col_scale.view(C, R // 128)[SAMPLE_COLS]), want["s_row"], "colwise scales")
    del out


def test_large_block_1x128_both_planes(big):
    """Both planes from one read (the fused row + col tile kernel): sampled
    rows of X and sampled rows of X^T, past element 2^31 in each plane."""
    d = fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 128), fq.FQ_ROWWISE | fq.FQ_COLWISE)
    out = quantize(d, big)
    want_r = orc.quantize_block(sample(big), (1, 128))
    same_bytes(host(out.row_data[SAMPLE_ROWS]), want_r["q_row"], "rowwise codes")
    same_bytes(host(out.row_scale.view(R, C // 128)[SAMPLE_ROWS]), want_r["s_row"], "rowwise scales")
    want_c = orc.quantize_block(sample_cols(), (1, 128))
    same_bytes(host(out.col_data[SAMPLE_COLS]), want_c["q_row"], "colwise codes (columns of X)")
    same_bytes(host(out.col_scale.view(C, R // 128)[SAMPLE_COLS]), want_c["s_row"], "colwise scales")
    del out


def test_large_nvfp4_colwise(big):
    d = fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (1, 16), fq.FQ_COLWISE)
    out = quantize(d, big)
    same_bytes(host(out.amax), f32(AMAX), "tensor amax")
    want = orc.quantize_nvfp4(sample_cols(), (1, 16), amax=AMAX)
    same_bytes(host(out.tensor_scale), f32(want["S"]), "tensor scale")
    same_bytes(host(out.col_data[SAMPLE_COLS]), want["p_row"], "packed FP4 of X^T rows")
    same_bytes(host(out.col_scale.view(C, R // 16)[SAMPLE_COLS]), want["c_row"], "E4M3 block scales")
    del out


def test_large_nvfp4_colwise_rht_given_amax(big):
    """The RHT works along X^T rows, so sampled columns of X transform alone;
    a given amax (as after a cross-device max) replaces the tensor's own."""
    signs = 0x5AC3
    d = fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (1, 16), fq.FQ_COLWISE,
                transform=fq.FQ_TRANSFORM_RHT16, rht_signs=signs)
    out = fq.alloc_quantized(d)
    amax = torch.tensor([300.0], dtype=torch.float32, device="cuda")
    fq.fq_quantize_with_amax(d, big, amax, out)
    torch.cuda.synchronize()
    cols = np.concatenate([np.arange(4), 12345 + np.arange(4), C - 8 + np.arange(8)])   # 16 columns
    xs = bf16_bits(values(np.arange(R)[:, None], cols[None, :]))     # [R, 16]: those columns of X
    want = orc.quantize_nvfp4_rht(xs, signs, amax=300.0)
    same_bytes(host(out.col_data[cols]), want["p_col"], "packed FP4 of transformed X^T rows")
    same_bytes(host(out.col_scale.view(C, R // 16)[cols]), want["c_col"], "E4M3 block scales")
    del out


def test_large_mxfp4_both_planes(big):
    d = fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (1, 32), fq.FQ_ROWWISE | fq.FQ_COLWISE)
    out = quantize(d, big)
    want = orc.quantize_mx(sample(None), outputs=orc.ROWWISE, fmt=orc.E2M1)
    same_bytes(host(out.row_data[SAMPLE_ROWS]), want["q_row"], "rowwise packed FP4")
    same_bytes(host(out.row_scale.view(R, C // 32)[SAMPLE_ROWS]), want["e_row"], "rowwise E8M0")
    wc = orc.quantize_mx(sample_cols(), outputs=orc.ROWWISE, fmt=orc.E2M1)
    same_bytes(host(out.col_data[SAMPLE_COLS]), wc["q_row"], "colwise packed FP4 (columns of X)")
    same_bytes(host(out.col_scale.view(C, R // 32)[SAMPLE_COLS]), wc["e_row"], "colwise E8M0")
    del out


def test_large_mx_requantize(big):
    d = fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 32), fq.FQ_ROWWISE)
    src = quantize(d, big)
    dst = fq.alloc_quantized(fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 32), fq.FQ_COLWISE))
    fq.fq_requantize_transpose(d, src, dst)
    torch.cuda.synchronize()
    # the requantized columns from the oracle's rowwise codes of those columns' rows: every row
    # is needed, so rebuild the rowwise codes of the sampled columns' 32-column blocks
    blocks = np.unique(SAMPLE_COLS // 32)
    cols = (blocks[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    xs = bf16_bits(values(np.arange(R)[:, None], cols[None, :]))      # [R, 32 * len(blocks)]
    rw = orc.quantize_mx(xs, outputs=orc.ROWWISE)
    want = orc.requant_mx_colwise(rw["q_row"], rw["e_row"])
    pos = np.searchsorted(cols, SAMPLE_COLS)
    same_bytes(host(dst.col_data[SAMPLE_COLS]), want["q_col"][pos], "requantized colwise codes")
    same_bytes(host(dst.col_scale.view(C, R // 32)[SAMPLE_COLS]), want["e_col"].reshape(len(cols), R // 32)[pos],
               "requantized colwise E8M0")
    del src, dst


def test_large_block_pow2_requantize(big):
    pow2 = dict(scale_mode=fq.FQ_SCALE_POW2)
    d = fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 128), fq.FQ_ROWWISE, **pow2)
    src = quantize(d, big)
    dst = fq.alloc_quantized(fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 128), fq.FQ_COLWISE,
                                     **pow2))
    fq.fq_requantize_transpose(d, src, dst)
    torch.cuda.synchronize()
    # the oracle's rowwise copy of the sampled columns' 1x128 tiles (every row), then its requantization
    blocks = np.unique(SAMPLE_COLS // 128)
    cols = (blocks[:, None] * 128 + np.arange(128)[None, :]).reshape(-1)
    xs = bf16_bits(values(np.arange(R)[:, None], cols[None, :]))      # [R, 128 * len(blocks)]
    rw = orc.quantize_block(xs, (1, 128), pow2=True)
    want = orc.requant_block_colwise(rw["q_row"], rw["s_row"])
    pos = np.searchsorted(cols, SAMPLE_COLS)
    same_bytes(host(dst.col_data[SAMPLE_COLS]), want["q_col"][pos], "requantized colwise codes")
    same_bytes(host(dst.col_scale.view(C, R // 128)[SAMPLE_COLS]), want["s_col"][pos], "requantized colwise scales")
    del src, dst


# ---------------------------------------------------------------- stochastic rounding of 8-bit elements
SR = (31337, 12)


def sr_codes(fmt, y, plane, e0):
    """Stochastic codes of consecutive plane elements e0, e0+1, ... with scaled
    fp32 values y, from the oracle's generator and rounding."""
    u = np.array([orc.sr_bits(SR[0], SR[1], plane, e0 + i) for i in range(y.size)], np.uint16)
    return orc.encode_sr(fmt, np.ascontiguousarray(y, np.float32), u)


def sr_desc(recipe, fmt, block, outputs):
    return fq.desc(recipe, fq.FQ_IN_BF16, fmt, R, C, block, outputs, rounding=fq.FQ_ROUND_STOCHASTIC, seed=SR[0],
                   offset=SR[1])


def test_large_current_sr_both_planes(big):
    """Per-tensor E5M2 with stochastic rounding, both planes from one read;
    sampled rows and rows of X^T past element 2^31."""
    out = quantize(sr_desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_E5M2, (0, 0), fq.FQ_ROWWISE | fq.FQ_COLWISE), big)
    alpha = np.float32(57344.0) / np.float32(AMAX)
    same_bytes(host(out.amax), f32(AMAX), "tensor amax")
    same_bytes(host(out.tensor_scale), f32(np.float32(AMAX) / np.float32(57344.0)), "s")
    rows = host(out.row_data[SAMPLE_ROWS])
    for i, r in enumerate(SAMPLE_ROWS):
        y = values(np.array([r]), np.arange(C)).ravel() * alpha
        same_bytes(rows[i], sr_codes(orc.E5M2, y, 0, int(r) * C), f"rowwise row {r}")
    cols = host(out.col_data[SAMPLE_COLS])
    for i, c in enumerate(SAMPLE_COLS):
        y = values(np.arange(R), np.array([c])).ravel() * alpha
        same_bytes(cols[i], sr_codes(orc.E5M2, y, 1, int(c) * R), f"colwise row {c}")
    del out


def test_large_mx_sr_both_planes(big):
    out = quantize(sr_desc(fq.FQ_MX, fq.FQ_E4M3, (1, 32), fq.FQ_ROWWISE | fq.FQ_COLWISE), big)
    for plane, idx, data, scale in ((0, SAMPLE_ROWS, out.row_data, out.row_scale.view(R, C // 32)),
                                    (1, SAMPLE_COLS, out.col_data, out.col_scale.view(C, R // 32))):
        got, got_e = host(data[idx]), host(scale[idx])
        n = C if plane == 0 else R
        for i, k in enumerate(idx):
            v = (values(np.array([k]), np.arange(C)) if plane == 0 else values(np.arange(R), np.array([k]))).ravel()
            a = np.abs(v).reshape(-1, 32).max(1)
            codes = np.array([orc.mx_code(x) for x in a], np.uint8)
            same_bytes(got_e[i], codes, f"plane {plane} E8M0 {k}")
            y = (v.reshape(-1, 32).astype(np.float64) * np.exp2(127.0 - codes.astype(np.float64))[:, None])
            same_bytes(got[i], sr_codes(orc.E4M3, y.astype(np.float32).ravel(), plane, int(k) * n),
                       f"plane {plane} codes {k}")
    del out


def test_large_block_1x128_sr_both_planes(big):
    out = quantize(sr_desc(fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (1, 128), fq.FQ_ROWWISE | fq.FQ_COLWISE), big)
    for plane, idx, data, scale in ((0, SAMPLE_ROWS, out.row_data, out.row_scale.view(R, C // 128)),
                                    (1, SAMPLE_COLS, out.col_data, out.col_scale.view(C, R // 128))):
        got, got_s = host(data[idx]), host(scale[idx])
        n = C if plane == 0 else R
        for i, k in enumerate(idx):
            v = (values(np.array([k]), np.arange(C)) if plane == 0 else values(np.arange(R), np.array([k]))).ravel()
            a = np.abs(v).reshape(-1, 128).max(1).astype(np.float32)
            alpha = (np.float32(448.0) / a).astype(np.float32)          # every tile amax is nonzero here
            same_bytes(got_s[i], (a / np.float32(448.0)).astype(np.float32), f"plane {plane} scales {k}")
            y = (v.reshape(-1, 128) * alpha[:, None]).astype(np.float32).ravel()
            same_bytes(got[i], sr_codes(orc.E4M3, y, plane, int(k) * n), f"plane {plane} codes {k}")
    del out
