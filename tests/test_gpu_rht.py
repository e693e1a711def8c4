"""GPU parity: NVFP4 1x16 colwise copy with the random Hadamard transform
(weight-gradient inputs) against the oracle: bit-exact packed nibbles,
block scales, tensor scale and amax of the transformed tensor, with and
without stochastic rounding, with a given amax, through fq_amax, and
dequantized; small, half-slab, wide-range, all-zero and full-size cases."""
import numpy as np
import pytest
import torch

import oracle as orc
from fp8_fp4_tensor_amd import fq
from fp8_fp4_tensor_amd import workloads as W
from gpu_util import dev, f32, host, in_dtype, same_bytes

pytestmark = pytest.mark.gpu

SIGNS = [0x0000, 0xFFFF, 0xA5C3]


def rht_desc(x, signs, sr=None):
    R, C = x.shape
    seed, off = (0, 0) if sr is None else sr
    return fq.desc(fq.FQ_NVFP4, in_dtype(x), fq.FQ_E2M1, R, C, (1, 16), fq.FQ_COLWISE,
                   rounding=fq.FQ_ROUND_NEAREST_EVEN if sr is None else fq.FQ_ROUND_STOCHASTIC, seed=seed,
                   offset=off, transform=fq.FQ_TRANSFORM_RHT16, rht_signs=signs)


def check_rht(x, signs, sr=None, amax_in=None, dq=False):
    d = rht_desc(x, signs, sr)
    out = fq.alloc_quantized(d)
    ws = fq.alloc_workspace(d)
    if amax_in is None:
        fq.fq_quantize(d, dev(x), out, ws)
    else:
        fq.fq_quantize_with_amax(d, dev(x), torch.tensor([amax_in], dtype=torch.float32, device="cuda"), out, ws)
    torch.cuda.synchronize()
    want = orc.quantize_nvfp4_rht(x, signs, amax=amax_in, sr=sr)
    tag = f"signs {signs:#06x} sr {sr}"
    same_bytes(host(out.col_data), want["p_col"], f"RHT colwise packed FP4 ({tag})")
    same_bytes(host(out.col_scale), want["c_col"], f"RHT colwise E4M3 block scales ({tag})")
    same_bytes(host(out.tensor_scale), f32(want["S"]), f"RHT tensor scale ({tag})")
    same_bytes(host(out.amax), f32(want["amax"]), f"RHT amax ({tag})")
    if dq:
        R, C = x.shape
        y = torch.empty((C, R), dtype=torch.float32, device="cuda")
        fq.fq_dequantize(d, out, fq.FQ_COLWISE, y)
        torch.cuda.synchronize()
        same_bytes(host(y), orc.dequant_nvfp4(want["p_col"], want["c_col"], want["S"], (1, 16)),
                   "RHT dequantized (transformed values)")
    return d


# (128, 128) and (256, 384) in bf16 take the 128x128-tile colwise pass
@pytest.mark.parametrize("shape", [(16, 16), (32, 64), (48, 80), (64, 4096 + 16), (16, 2064), (96, 272), (128, 128),
                                   (256, 384)])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_rht_small(shape, dt):
    x = W.normal(shape, 1.0, shape[0] * 11 + shape[1], dt)
    for signs in SIGNS:
        check_rht(x, signs, dq=(signs == SIGNS[-1]))
    check_rht(x, 0x3C96, sr=(99, 4))


def test_rht_given_amax_and_fq_amax():
    x = W.normal((64, 128), 1.0, 23, W.BF16)
    d = check_rht(x, 0x1357)
    a = orc.quantize_nvfp4_rht(x, 0x1357)["amax"]
    got = torch.empty(1, dtype=torch.float32, device="cuda")
    fq.fq_amax(d, dev(x), got, fq.alloc_workspace(d))
    torch.cuda.synchronize()
    same_bytes(host(got), f32(a), "fq_amax of the transformed tensor")
    for amax_in in (float(a), 3.0 * float(a)):
        check_rht(x, 0x1357, amax_in=amax_in)
        check_rht(x, 0x1357, sr=(5, 6), amax_in=amax_in)


def test_rht_wide_range_and_zero():
    x = W.uniform_bits_bf16((64, 256), 29, max_abs=1e30)
    check_rht(x, 0xBEEF)
    x = W.uniform_bits_bf16((128, 256), 30, max_abs=1e30)
    check_rht(x, 0xBEEF)
    check_rht(x, 0x00FF, sr=(3, 4), amax_in=float(orc.quantize_nvfp4_rht(x, 0x00FF)["amax"]) * 2.0)
    check_rht(np.zeros((32, 32), np.uint16), 0xBEEF)
    check_rht(np.zeros((32, 32), np.float32), 0x0001, sr=(1, 1))


@pytest.mark.parametrize("w", [w for w in W.LARGE if w.name.startswith("nvfp4_1x16")], ids=lambda w: w.name)
def test_full_size_rht(w):
    check_rht(w.make(), 0xA5C3, sr=(2024, 7))
