"""The dequantized relative error of the 8-bit recipes at full size, on the GPU.

[CS] "FP8 Current Scaling：量化、缩放与精度边界", section "缩放会不会把误差放大":
dequantizing multiplies the rounding error and the value by the same scale,
so the relative error of a restored element is its relative rounding error
in the scaled space. [MP] "混合精度训练：fp16 到 fp8", section "FP8 数据格式":
E4M3 keeps three mantissa bits and E5M2 two, so round to nearest even of a
scaled value inside the format's normal range errs by at most half a unit
in the last place: 2^-4 relative for E4M3, 2^-3 for E5M2 (the scale's own
fp32 roundings add a few units of 2^-24). Each workload is quantized and
dequantized (fp32) by the library; every element whose scaled magnitude
lies in [min normal, Fmax], with a small margin for the scale's rounding,
must meet the bound.
"""
import pytest
import torch

from fp8_fp4_tensor_amd import fq
from fp8_fp4_tensor_amd import workloads as W
from gpu_util import dev

pytestmark = pytest.mark.gpu

ROW = fq.FQ_ROWWISE
FMT = {"e4m3": (fq.FQ_E4M3, 448.0, 2.0 ** -6, 2.0 ** -4), "e5m2": (fq.FQ_E5M2, 57344.0, 2.0 ** -14, 2.0 ** -3)}
SLACK = 1 + 2.0 ** -20
MARGIN = 2.0 ** -10


def expand(scale, R, C, br, bc):
    """A per-block scale plane [R/br, C/bc] to one value per element."""
    return scale.reshape(R // br, C // bc).repeat_interleave(br, 0).repeat_interleave(bc, 1)


def check_bound(x, y, s, fmax, min_normal, bound, what):
    """Elements with x/s in range meet |y - x| <= bound * |x|."""
    xs = x.abs() / s
    inr = (xs >= min_normal * (1 + MARGIN)) & (xs <= fmax * (1 - MARGIN))
    assert int(inr.sum()) > x.numel() // 2, f"{what}: too few in-range elements to mean anything"
    rel = ((y - x).abs() / x.abs())[inr]
    worst = float(rel.max())
    assert worst <= bound * SLACK, f"{what}: relative error {worst:.6g} above {bound:.6g}"


def quantize_dequantize(recipe, fmt, block, xh):
    R, C = xh.shape
    d = fq.desc(recipe, fq.FQ_IN_BF16, fmt, R, C, block, ROW)
    out = fq.alloc_quantized(d)
    fq.fq_quantize(d, dev(xh), out, fq.alloc_workspace(d))
    y = torch.empty((R, C), dtype=torch.float32, device="cuda")
    fq.fq_dequantize(d, out, ROW, y)
    torch.cuda.synchronize()
    return out, y


@pytest.mark.parametrize("name", ["current_e4m3_act_8192x4096", "current_e5m2_grad_8192x4096"])
def test_error_bound_per_tensor(name):
    w = W.BY_NAME[name]
    fmt, fmax, mn, bound = FMT[w.fmt]
    xh = w.make()
    out, y = quantize_dequantize(fq.FQ_PER_TENSOR_CURRENT, fmt, (0, 0), xh)
    x = dev(xh).float()
    check_bound(x, y, out.tensor_scale, fmax, mn, bound, name)


@pytest.mark.parametrize("name", ["block1x128_act_16384x7168", "block128x128_wgt_7168x18432"])
def test_error_bound_blockwise(name):
    w = W.BY_NAME[name]
    fmt, fmax, mn, bound = FMT["e4m3"]
    xh = w.make()
    R, C = xh.shape
    out, y = quantize_dequantize(fq.FQ_BLOCK_FP32, fmt, w.block, xh)
    x = dev(xh).float()
    check_bound(x, y, expand(out.row_scale, R, C, *w.block), fmax, mn, bound, name)


@pytest.mark.parametrize("fmt_name", ["e4m3", "e5m2"])
def test_error_bound_mx(fmt_name):
    """MX: the scale is a power of two chosen from the block's exponent, so
    the block maximum can land above Fmax and saturate; those elements are
    outside the range and excluded like any other."""
    w = W.BY_NAME["mxfp8_rowcol_8192x8192"]
    fmt, fmax, mn, bound = FMT[fmt_name]
    xh = w.make()
    R, C = xh.shape
    out, y = quantize_dequantize(fq.FQ_MX, fmt, (1, 32), xh)
    x = dev(xh).float()
    scale = torch.exp2(out.row_scale.to(torch.float32) - 127.0)
    check_bound(x, y, expand(scale, R, C, 1, 32), fmax, mn, bound, f"mx {fmt_name}")
