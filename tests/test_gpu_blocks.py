"""GPU parity: blockwise fp32, MXFP8 and NVFP4 against the oracle (bit-exact
codes, scales and packed nibbles), plus dequantization."""
import numpy as np
import pytest
import torch

import oracle as orc
from fp8_fp4_tensor_amd import fq
from fp8_fp4_tensor_amd import workloads as W
from gpu_util import dev, f32, host, in_dtype, same_bytes

pytestmark = pytest.mark.gpu

BOTH = fq.FQ_ROWWISE | fq.FQ_COLWISE


def run(recipe, fmt, x, block, outputs, amax_in=None):
    R, C = x.shape
    d = fq.desc(recipe, in_dtype(x), fmt, R, C, block, outputs)
    out = fq.alloc_quantized(d)
    ws = fq.alloc_workspace(d)
    if amax_in is None:
        fq.fq_quantize(d, dev(x), out, ws)
    else:
        fq.fq_quantize_with_amax(d, dev(x), torch.tensor([amax_in], dtype=torch.float32, device="cuda"), out, ws)
    torch.cuda.synchronize()
    return d, out


def dequant_check(d, out, want_fn):
    """fp32 and bf16 dequantization of every selected plane vs the oracle
    (bf16: the oracle's fp32 values rounded to nearest even)."""
    for which in (fq.FQ_ROWWISE, fq.FQ_COLWISE):
        if not d.outputs & which:
            continue
        shape = (d.rows, d.cols) if which == fq.FQ_ROWWISE else (d.cols, d.rows)
        want = want_fn(which)
        y = torch.empty(shape, dtype=torch.float32, device="cuda")
        fq.fq_dequantize(d, out, which, y)
        yb = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        fq.fq_dequantize(d, out, which, yb)
        torch.cuda.synchronize()
        name = "rowwise" if which == 1 else "colwise"
        same_bytes(host(y), want, f"dequantized {name} fp32")
        same_bytes(host(yb.view(torch.int16)).view(np.uint16), orc.f32_to_bf16(want), f"dequantized {name} bf16")


# ---------------------------------------------------------------- blockwise
def check_block(x, block, outputs, dq=False):
    d, out = run(fq.FQ_BLOCK_FP32, fq.FQ_E4M3, x, block, outputs)
    want = orc.quantize_block(x, block, outputs=outputs)
    if outputs & fq.FQ_ROWWISE:
        same_bytes(host(out.row_data), want["q_row"], "rowwise codes")
        same_bytes(host(out.row_scale), want["s_row"], "rowwise scales")
    if outputs & fq.FQ_COLWISE:
        same_bytes(host(out.col_data), want["q_col"], "colwise codes")
        same_bytes(host(out.col_scale), want["s_col"], "colwise scales")
    if dq:
        def want_fn(which):
            if which == fq.FQ_ROWWISE:
                return orc.dequant_block(want["q_row"], want["s_row"], block)
            return orc.dequant_block(want["q_col"], want["s_col"], block)
        dequant_check(d, out, want_fn)


@pytest.mark.parametrize("block", [(1, 128), (128, 128)])
@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (384, 640), (128, 1152)])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_block_small(block, shape, dt):
    x = W.normal(shape, 1.0, shape[0] + shape[1], dt)
    check_block(x, block, BOTH, dq=True)
    check_block(x, block, fq.FQ_ROWWISE)


def test_block_1x128_odd_rows():
    x = W.normal((3, 256), 1.0, 5, W.BF16)
    check_block(x, (1, 128), fq.FQ_ROWWISE)


def test_block_all_bf16_patterns():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    x = b[np.isfinite(f)]
    x = np.concatenate([x, np.zeros(128 - x.size % 128, np.uint16)]).reshape(-1, 128)
    check_block(x, (1, 128), fq.FQ_ROWWISE)
    rng = np.random.default_rng(2)
    check_block(x[rng.permutation(x.shape[0])][: (x.shape[0] // 128) * 128], (128, 128), BOTH)


def test_block_zero_tiles():
    x = np.zeros((256, 256), np.float32)
    x[200, 7] = -3.0
    check_block(x, (1, 128), BOTH)
    check_block(x, (128, 128), BOTH)


@pytest.mark.parametrize("w", [w for w in W.LARGE if w.recipe == "block"], ids=lambda w: w.name)
def test_full_size_block(w):
    check_block(w.make(), w.block, fq.FQ_ROWWISE)


def test_full_size_block_1x128_both_planes():
    """The activation workload with its colwise copy too (one read for both)."""
    w = W.BY_NAME["block1x128_act_16384x7168"]
    check_block(w.make(), w.block, BOTH)


# ---------------------------------------------------------------- MXFP8
def check_mx(x, outputs, dq=False):
    d, out = run(fq.FQ_MX, fq.FQ_E4M3, x, (1, 32), outputs)
    want = orc.quantize_mx(x, outputs=outputs)
    if outputs & fq.FQ_ROWWISE:
        same_bytes(host(out.row_data), want["q_row"], "rowwise codes")
        same_bytes(host(out.row_scale), want["e_row"], "rowwise E8M0")
    if outputs & fq.FQ_COLWISE:
        same_bytes(host(out.col_data), want["q_col"], "colwise codes")
        same_bytes(host(out.col_scale), want["e_col"], "colwise E8M0")
    if dq:
        def want_fn(which):
            if which == fq.FQ_ROWWISE:
                return orc.dequant_mx(want["q_row"], want["e_row"])
            return orc.dequant_mx(want["q_col"], want["e_col"])
        dequant_check(d, out, want_fn)


@pytest.mark.parametrize("shape", [(32, 32), (64, 96), (96, 64), (160, 288), (128, 128), (256, 384)])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_mx_small(shape, dt):
    x = W.student_t(shape, 3.0, shape[0] * 3 + shape[1], dt)
    check_mx(x, BOTH, dq=True)
    check_mx(x, fq.FQ_ROWWISE)
    check_mx(x, fq.FQ_COLWISE)


def test_mx_rowwise_odd_rows():
    check_mx(W.student_t((7, 64), 3.0, 1, W.BF16), fq.FQ_ROWWISE)


def test_mx_wide_range():
    """Blocks spread over the whole bf16 exponent range (E8M0 clamp at 0)."""
    x = W.uniform_bits_bf16((256, 256), 3, max_abs=3e38)
    check_mx(x, BOTH)
    tiny = W.to_bf16_bits((W.bf16_bits_to_f32(x) * np.float32(1e-38)).astype(np.float32)).reshape(256, 256)
    check_mx(tiny, BOTH)
    z = np.zeros((64, 64), np.uint16)
    check_mx(z, BOTH)


@pytest.mark.parametrize("w", [w for w in W.LARGE if w.recipe == "mx"], ids=lambda w: w.name)
def test_full_size_mx(w):
    x = w.make()
    check_mx(x, BOTH)
    check_mx(x, fq.FQ_ROWWISE)


# ---------------------------------------------------------------- NVFP4
def check_nvfp4(x, block, outputs, amax_in=None, dq=False):
    d, out = run(fq.FQ_NVFP4, fq.FQ_E2M1, x, block, outputs, amax_in)
    want = orc.quantize_nvfp4(x, block, outputs=outputs, amax=amax_in)
    if outputs & fq.FQ_ROWWISE:
        same_bytes(host(out.row_data), want["p_row"], "rowwise packed FP4")
        same_bytes(host(out.row_scale), want["c_row"], "rowwise E4M3 block scales")
    if outputs & fq.FQ_COLWISE:
        same_bytes(host(out.col_data), want["p_col"], "colwise packed FP4")
        same_bytes(host(out.col_scale), want["c_col"], "colwise E4M3 block scales")
    same_bytes(host(out.tensor_scale), f32(want["S"]), "tensor scale S")
    if dq:
        def want_fn(which):
            if which == fq.FQ_ROWWISE:
                return orc.dequant_nvfp4(want["p_row"], want["c_row"], want["S"], block)
            return orc.dequant_nvfp4(want["p_col"], want["c_col"], want["S"], block)
        dequant_check(d, out, want_fn)


# (128, 128) and (256, 384) take the one-read both-planes pass for 1x16 blocks
# (bf16, R and C multiples of 128)
@pytest.mark.parametrize("block", [(1, 16), (16, 16)])
@pytest.mark.parametrize("shape", [(16, 16), (32, 64), (48, 80), (64, 4096 + 16), (16, 2064), (128, 128), (256, 384)])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_nvfp4_small(block, shape, dt):
    x = W.normal(shape, 1.0, shape[0] * 5 + shape[1], dt)
    check_nvfp4(x, block, BOTH, dq=True)
    check_nvfp4(x, block, fq.FQ_ROWWISE)
    check_nvfp4(x, block, fq.FQ_COLWISE)


@pytest.mark.parametrize("block", [(1, 16), (16, 16)])
@pytest.mark.parametrize("shape", [(64, 128), (128, 256)])
def test_nvfp4_with_amax(block, shape):
    """The block pass at a given tensor amax (e.g. reduced across shards)."""
    x = W.normal(shape, 1.0, 21, W.BF16)
    a = float(np.abs(W.bf16_bits_to_f32(x)).max())
    for amax_in in (a, 2.5 * a, 0.5 * a):
        check_nvfp4(x, block, BOTH, amax_in=amax_in)


def test_nvfp4_rowwise_1x16_odd_rows():
    check_nvfp4(W.normal((5, 48), 1.0, 3, W.BF16), (1, 16), fq.FQ_ROWWISE)


def test_nvfp4_wide_range_and_zero():
    x = W.uniform_bits_bf16((64, 256), 9, max_abs=1e6)
    check_nvfp4(x, (1, 16), BOTH)
    check_nvfp4(x, (16, 16), BOTH)
    x = W.uniform_bits_bf16((128, 256), 10, max_abs=1e6)
    for block in ((1, 16), (16, 16)):
        check_nvfp4(x, block, BOTH)
        check_nvfp4(x, block, fq.FQ_COLWISE)
        check_nvfp4(np.zeros((128, 128), np.uint16), block, BOTH)
    check_nvfp4(np.zeros((32, 32), np.uint16), (16, 16), BOTH)
    check_nvfp4(np.zeros((32, 32), np.float32), (1, 16), BOTH)


@pytest.mark.parametrize("w", [w for w in W.LARGE if w.recipe == "nvfp4"], ids=lambda w: w.name)
def test_full_size_nvfp4(w):
    check_nvfp4(w.make(), w.block, fq.FQ_ROWWISE)


def test_full_size_nvfp4_1x16_both_planes():
    """The activation workload with its colwise copy too (one block pass for both)."""
    w = W.BY_NAME["nvfp4_1x16_act_8192x14336"]
    check_nvfp4(w.make(), w.block, BOTH)


def test_full_size_nvfp4_16x16_both_planes():
    """The weight workload with its colwise copy too (one block pass for both)."""
    w = W.BY_NAME["nvfp4_16x16_wgt_14336x4096"]
    check_nvfp4(w.make(), w.block, BOTH)


# ---------------------------------------------------------------- per-tensor dequant
@pytest.mark.parametrize("fmt", [fq.FQ_E4M3, fq.FQ_E5M2])
def test_dequant_per_tensor(fmt):
    x = W.normal((96, 160), 2.0, 77, W.BF16)
    d, out = run(fq.FQ_PER_TENSOR_CURRENT, fmt, x, (0, 0), BOTH)
    ofmt = orc.E4M3 if fmt == fq.FQ_E4M3 else orc.E5M2
    want = orc.quantize_current(x, ofmt, outputs=BOTH)
    dequant_check(d, out, lambda w: orc.dequant_tensor(want["q_row"] if w == 1 else want["q_col"], ofmt, want["s"]))


# ---------------------------------------------------------------- MX requantize (rowwise -> colwise)
def check_requant(x):
    """The GPU's rowwise copy must equal the oracle's; the oracle then
    requantizes its own rowwise copy, the GPU its own."""
    R, C = x.shape
    d, out = run(fq.FQ_MX, fq.FQ_E4M3, x, (1, 32), fq.FQ_ROWWISE)
    single = orc.quantize_mx(x, outputs=fq.FQ_ROWWISE)
    same_bytes(host(out.row_data), single["q_row"], "rowwise codes")
    same_bytes(host(out.row_scale), single["e_row"], "rowwise E8M0")
    dst = fq.alloc_quantized(fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 32), fq.FQ_COLWISE))
    fq.fq_requantize_transpose(d, out, dst)
    torch.cuda.synchronize()
    want = orc.requant_mx_colwise(single["q_row"], single["e_row"])
    same_bytes(host(dst.col_data), want["q_col"], "requantized colwise codes")
    same_bytes(host(dst.col_scale), want["e_col"], "requantized colwise E8M0")


# ragged tiles, one full tile, and full tiles with several per workgroup walk
@pytest.mark.parametrize("shape", [(32, 32), (64, 96), (96, 64), (160, 288), (256, 384), (256, 512), (512, 1024)])
def test_mx_requant_small(shape):
    check_requant(W.student_t(shape, 3.0, shape[0] * 7 + shape[1], W.BF16))


def test_mx_requant_wide_range():
    check_requant(W.uniform_bits_bf16((256, 256), 13, max_abs=3e38))
    check_requant(np.zeros((64, 64), np.uint16))


@pytest.mark.parametrize("w", [w for w in W.LARGE if w.recipe == "mx"], ids=lambda w: w.name)
def test_full_size_mx_requant(w):
    check_requant(w.make())


@pytest.mark.parametrize("shape", [(1, 37), (3, 1000), (257, 129)])
@pytest.mark.parametrize("fmt", [fq.FQ_E4M3, fq.FQ_E5M2])
def test_dequant_per_tensor_ragged(shape, fmt):
    x = W.normal(shape, 3.0, shape[0] + 17 * shape[1], W.F32)
    d, out = run(fq.FQ_PER_TENSOR_CURRENT, fmt, x, (0, 0), fq.FQ_ROWWISE)
    ofmt = orc.E4M3 if fmt == fq.FQ_E4M3 else orc.E5M2
    want = orc.quantize_current(x, ofmt)
    dequant_check(d, out, lambda w: orc.dequant_tensor(want["q_row"], ofmt, want["s"]))
