"""GPU parity of the format variants against the oracle (bit-exact codes and
scales, plus fp32/bf16 dequantization): MX with E5M2 elements, MXFP4 (E2M1
elements packed two per byte), and blockwise E4M3 with power-of-two tile
scales, including its requantization in the other direction (the colwise
copy from the rowwise copy alone). Small, ragged-tile, wide-range,
every-bf16-pattern, all-zero and full-size cases, fp32 and bf16 inputs."""
import numpy as np
import pytest
import torch

import oracle as orc
from fp8_fp4_tensor_amd import fq
from fp8_fp4_tensor_amd import workloads as W
from gpu_util import dev, host, in_dtype, same_bytes
from test_gpu_blocks import dequant_check

pytestmark = pytest.mark.gpu

BOTH = fq.FQ_ROWWISE | fq.FQ_COLWISE
MX_FMTS = [fq.FQ_E5M2, fq.FQ_E2M1]
NAMES = {fq.FQ_E5M2: "e5m2", fq.FQ_E2M1: "e2m1"}


def quantize(recipe, fmt, x, block, outputs, scale_mode=fq.FQ_SCALE_DEFAULT):
    R, C = x.shape
    d = fq.desc(recipe, in_dtype(x), fmt, R, C, block, outputs, scale_mode=scale_mode)
    out = fq.alloc_quantized(d)
    fq.fq_quantize(d, dev(x), out, fq.alloc_workspace(d))
    torch.cuda.synchronize()
    return d, out


# ---------------------------------------------------------------- MX E5M2 / MXFP4
def check_mx(x, fmt, outputs, dq=False):
    d, out = quantize(fq.FQ_MX, fmt, x, (1, 32), outputs)
    want = orc.quantize_mx(x, outputs=outputs, fmt=fmt)
    tag = NAMES[fmt]
    if outputs & fq.FQ_ROWWISE:
        same_bytes(host(out.row_data), want["q_row"], f"{tag} rowwise codes")
        same_bytes(host(out.row_scale), want["e_row"], f"{tag} rowwise E8M0")
    if outputs & fq.FQ_COLWISE:
        same_bytes(host(out.col_data), want["q_col"], f"{tag} colwise codes")
        same_bytes(host(out.col_scale), want["e_col"], f"{tag} colwise E8M0")
    if dq:
        def want_fn(which):
            if which == fq.FQ_ROWWISE:
                return orc.dequant_mx(want["q_row"], want["e_row"], fmt)
            return orc.dequant_mx(want["q_col"], want["e_col"], fmt)
        dequant_check(d, out, want_fn)


@pytest.mark.parametrize("fmt", MX_FMTS, ids=lambda f: NAMES[f])
@pytest.mark.parametrize("shape", [(32, 32), (64, 96), (96, 64), (160, 288), (128, 128), (256, 384), (64, 4128)])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_mx_variant_small(fmt, shape, dt):
    x = W.student_t(shape, 3.0, shape[0] * 7 + shape[1] + fmt, dt)
    check_mx(x, fmt, BOTH, dq=True)
    check_mx(x, fmt, fq.FQ_ROWWISE)
    check_mx(x, fmt, fq.FQ_COLWISE)


@pytest.mark.parametrize("fmt", MX_FMTS, ids=lambda f: NAMES[f])
def test_mx_variant_odd_rows(fmt):
    check_mx(W.student_t((7, 64), 3.0, 1, W.BF16), fmt, fq.FQ_ROWWISE)


@pytest.mark.parametrize("fmt", MX_FMTS, ids=lambda f: NAMES[f])
def test_mx_variant_all_bf16_patterns(fmt):
    """Every finite bf16 value, in blocks whose scales span the E8M0 range."""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    x = b[np.isfinite(f)]
    x = np.concatenate([x, np.zeros(4096 - x.size % 4096, np.uint16)]).reshape(-1, 128)
    check_mx(x, fmt, BOTH)
    rng = np.random.default_rng(5)
    check_mx(x.reshape(-1)[rng.permutation(x.size)].reshape(-1, 128), fmt, BOTH)


@pytest.mark.parametrize("fmt", MX_FMTS, ids=lambda f: NAMES[f])
def test_mx_variant_wide_range_and_zero(fmt):
    x = W.uniform_bits_bf16((256, 256), 3 + fmt, max_abs=3e38)
    check_mx(x, fmt, BOTH)
    tiny = W.to_bf16_bits((W.bf16_bits_to_f32(x) * np.float32(1e-38)).astype(np.float32)).reshape(256, 256)
    check_mx(tiny, fmt, BOTH)
    check_mx(np.zeros((64, 64), np.uint16), fmt, BOTH)
    check_mx(np.zeros((64, 64), np.float32), fmt, BOTH)


@pytest.mark.parametrize("fmt", MX_FMTS, ids=lambda f: NAMES[f])
@pytest.mark.parametrize("w", [w for w in W.LARGE if w.recipe == "mx"], ids=lambda w: w.name)
def test_full_size_mx_variant(fmt, w):
    check_mx(w.make(), fmt, BOTH)


# ---------------------------------------------------------------- blockwise, power-of-two scales
def check_block_pow2(x, block, outputs, dq=False):
    d, out = quantize(fq.FQ_BLOCK_FP32, fq.FQ_E4M3, x, block, outputs, fq.FQ_SCALE_POW2)
    want = orc.quantize_block(x, block, outputs=outputs, pow2=True)
    if outputs & fq.FQ_ROWWISE:
        same_bytes(host(out.row_data), want["q_row"], "pow2 rowwise codes")
        same_bytes(host(out.row_scale), want["s_row"], "pow2 rowwise scales")
    if outputs & fq.FQ_COLWISE:
        same_bytes(host(out.col_data), want["q_col"], "pow2 colwise codes")
        same_bytes(host(out.col_scale), want["s_col"], "pow2 colwise scales")
    if dq:
        def want_fn(which):
            if which == fq.FQ_ROWWISE:
                return orc.dequant_block(want["q_row"], want["s_row"], block)
            return orc.dequant_block(want["q_col"], want["s_col"], block)
        dequant_check(d, out, want_fn)


@pytest.mark.parametrize("block", [(1, 128), (128, 128)])
@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (384, 640), (128, 1152)])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_block_pow2_small(block, shape, dt):
    x = W.normal(shape, 0.02, shape[0] + 3 * shape[1], dt)
    check_block_pow2(x, block, BOTH, dq=True)
    check_block_pow2(x, block, fq.FQ_ROWWISE)


def test_block_pow2_all_bf16_patterns_and_zero():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    x = b[np.isfinite(f)]
    x = np.concatenate([x, np.zeros(128 - x.size % 128, np.uint16)]).reshape(-1, 128)
    check_block_pow2(x, (1, 128), fq.FQ_ROWWISE)
    rng = np.random.default_rng(4)
    check_block_pow2(x[rng.permutation(x.shape[0])][: (x.shape[0] // 128) * 128], (128, 128), BOTH)
    z = np.zeros((256, 256), np.float32)
    z[3, 200] = 5.0
    check_block_pow2(z, (1, 128), BOTH)
    check_block_pow2(z, (128, 128), BOTH)


@pytest.mark.parametrize("w", [w for w in W.LARGE if w.recipe == "block"], ids=lambda w: w.name)
def test_full_size_block_pow2(w):
    check_block_pow2(w.make(), w.block, fq.FQ_ROWWISE)


# ---------------------------------------------------------------- blockwise 1x128 pow2 requantize
def check_block_requant(x):
    """The GPU's rowwise copy must equal the oracle's; the oracle then
    requantizes its own rowwise copy, the GPU its own."""
    R, C = x.shape
    d, out = quantize(fq.FQ_BLOCK_FP32, fq.FQ_E4M3, x, (1, 128), fq.FQ_ROWWISE, fq.FQ_SCALE_POW2)
    single = orc.quantize_block(x, (1, 128), pow2=True)
    same_bytes(host(out.row_data), single["q_row"], "pow2 rowwise codes")
    same_bytes(host(out.row_scale), single["s_row"], "pow2 rowwise scales")
    dst = fq.alloc_quantized(fq.desc(fq.FQ_BLOCK_FP32, in_dtype(x), fq.FQ_E4M3, R, C, (1, 128), fq.FQ_COLWISE,
                                     scale_mode=fq.FQ_SCALE_POW2))
    dst.col_data.fill_(0xA5)
    dst.col_scale.fill_(-3.0)
    fq.fq_requantize_transpose(d, out, dst)
    torch.cuda.synchronize()
    want = orc.requant_block_colwise(single["q_row"], single["s_row"])
    same_bytes(host(dst.col_data), want["q_col"], "requantized colwise codes")
    same_bytes(host(dst.col_scale), want["s_col"], "requantized colwise scales")


@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (384, 128), (128, 1152)])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_block_requant_small(shape, dt):
    check_block_requant(W.normal(shape, 0.02, 5 * shape[0] + shape[1], dt))


def test_block_requant_wide_range_and_zero():
    check_block_requant(W.uniform_bits_bf16((256, 256), 17, max_abs=3e38))
    check_block_requant(W.student_t((384, 256), 3.0, 19, W.BF16))
    check_block_requant(np.zeros((128, 256), np.uint16))
    z = np.zeros((256, 128), np.float32)
    z[5, 7] = -3.0e-30
    check_block_requant(z)


@pytest.mark.parametrize("w", [w for w in W.LARGE if w.recipe == "block" and w.block == (1, 128)],
                         ids=lambda w: w.name)
def test_full_size_block_requant(w):
    check_block_requant(w.make())
