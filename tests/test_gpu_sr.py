"""GPU parity: NVFP4 1x16 with stochastically rounded elements against the
oracle (bit-exact packed nibbles, block scales and tensor scale), for both
planes, several seeds and offsets, fp32 and bf16 inputs, ragged grids and the
full-size gradient workload shape."""
import numpy as np
import pytest
import torch

import oracle as orc
from fp8_fp4_tensor_amd import fq
from fp8_fp4_tensor_amd import workloads as W
from gpu_util import dev, f32, host, in_dtype, same_bytes

pytestmark = pytest.mark.gpu

BOTH = fq.FQ_ROWWISE | fq.FQ_COLWISE
SEEDS = [(0, 0), (12345, 7), (2**64 - 1, 2**63 + 11)]


def run_sr(x, outputs, seed, offset, amax_in=None):
    R, C = x.shape
    d = fq.desc(fq.FQ_NVFP4, in_dtype(x), fq.FQ_E2M1, R, C, (1, 16), outputs,
                rounding=fq.FQ_ROUND_STOCHASTIC, seed=seed, offset=offset)
    out = fq.alloc_quantized(d)
    ws = fq.alloc_workspace(d)
    if amax_in is None:
        fq.fq_quantize(d, dev(x), out, ws)
    else:
        fq.fq_quantize_with_amax(d, dev(x), torch.tensor([amax_in], dtype=torch.float32, device="cuda"), out, ws)
    torch.cuda.synchronize()
    return d, out


def check_sr(x, outputs, seed, offset, amax_in=None):
    d, out = run_sr(x, outputs, seed, offset, amax_in)
    want = orc.quantize_nvfp4(x, (1, 16), outputs=outputs, amax=amax_in, sr=(seed, offset))
    tag = f"seed {seed} offset {offset}"
    if outputs & fq.FQ_ROWWISE:
        same_bytes(host(out.row_data), want["p_row"], f"rowwise packed FP4 ({tag})")
        same_bytes(host(out.row_scale), want["c_row"], f"rowwise E4M3 block scales ({tag})")
    if outputs & fq.FQ_COLWISE:
        same_bytes(host(out.col_data), want["p_col"], f"colwise packed FP4 ({tag})")
        same_bytes(host(out.col_scale), want["c_col"], f"colwise E4M3 block scales ({tag})")
    same_bytes(host(out.tensor_scale), f32(want["S"]), "tensor scale S")
    return d, out


@pytest.mark.parametrize("shape", [(16, 16), (32, 64), (48, 80), (64, 4096 + 16), (16, 2064), (5, 48)])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_nvfp4_sr_small(shape, dt):
    x = W.normal(shape, 1.0, shape[0] * 3 + shape[1], dt)
    outputs = BOTH if shape[0] % 16 == 0 else fq.FQ_ROWWISE
    for seed, offset in SEEDS:
        check_sr(x, outputs, seed, offset)


@pytest.mark.parametrize("shape", [(128, 128), (256, 384)])
def test_nvfp4_sr_colwise_tiles(shape):
    """bf16, R and C multiples of 128: the 128x128-tile colwise pass with
    stochastic rounding, alone and after the rowwise SR pass (both planes)."""
    x = W.normal(shape, 1.0, shape[0] * 7 + shape[1], W.BF16)
    for seed, offset in SEEDS:
        check_sr(x, fq.FQ_COLWISE, seed, offset)
        check_sr(x, BOTH, seed, offset)
    a = 3.0 * float(np.abs(W.bf16_bits_to_f32(x)).max())
    check_sr(x, fq.FQ_COLWISE, 11, 12, amax_in=a)
    check_sr(x, BOTH, 11, 12, amax_in=a)


def test_nvfp4_sr_with_amax_and_special_values():
    x = W.normal((64, 128), 1.0, 31, W.F32)
    x[0, :16] = 0.0
    x[1, :16] = -0.0
    x[2, :8] = -1e-30
    x[3, 3] = -x[3, 3]
    a = float(np.abs(x).max())
    for amax_in in (a, 3.0 * a):
        check_sr(x, BOTH, 77, 3, amax_in=amax_in)
    check_sr(np.zeros((32, 32), np.float32), BOTH, 1, 1)


def test_nvfp4_sr_wide_range():
    x = W.uniform_bits_bf16((64, 256), 19, max_abs=1e6)
    check_sr(x, BOTH, 5, 6)


def test_nvfp4_sr_differs_from_nearest_and_dequantizes():
    x = W.normal((64, 512), 1.0, 41, W.BF16)
    d, out = check_sr(x, BOTH, 9, 9)
    want = orc.quantize_nvfp4(x, (1, 16), outputs=BOTH, sr=(9, 9))
    y = torch.empty((64, 512), dtype=torch.float32, device="cuda")
    fq.fq_dequantize(d, out, fq.FQ_ROWWISE, y)
    torch.cuda.synchronize()
    same_bytes(host(y), orc.dequant_nvfp4(want["p_row"], want["c_row"], want["S"], (1, 16)), "dequantized SR")
    rt = orc.quantize_nvfp4(x, (1, 16), outputs=BOTH)
    assert not np.array_equal(host(out.row_data), rt["p_row"])


@pytest.mark.parametrize("w", [w for w in W.LARGE if w.name.startswith("nvfp4_1x16")], ids=lambda w: w.name)
def test_full_size_nvfp4_sr(w):
    check_sr(w.make(), w.outputs, 2024, 1)
