"""GPU parity: stochastic rounding of 8-bit elements (per-tensor current
scaling E4M3 / E5M2, blockwise 1x128 with fp32 or power-of-two scales, MX
E4M3 / E5M2) against the oracle, bit-exact: codes of both planes (each with
its own random bits), scales, s and the amax; ragged and tile-multiple
shapes, fp32 and bf16 input, a given amax, several seeds and offsets, the
gradient workloads at full size, and repeatability."""
import numpy as np
import pytest
import torch

import oracle as orc
from fp8_fp4_tensor_amd import fq
from fp8_fp4_tensor_amd import workloads as W
from gpu_util import dev, f32, host, in_dtype, same_bytes

pytestmark = pytest.mark.gpu

ROW, COL = fq.FQ_ROWWISE, fq.FQ_COLWISE
BOTH = ROW | COL
OFMT = {fq.FQ_E4M3: orc.E4M3, fq.FQ_E5M2: orc.E5M2}
SEEDS = [(0, 0), (2026, 7), (2 ** 64 - 3, 2 ** 40 + 5)]


def run(recipe, fmt, x, outputs, sr, block=(0, 0), pow2=False, amax_in=None):
    R, C = x.shape
    d = fq.desc(recipe, in_dtype(x), fmt, R, C, block, outputs, rounding=fq.FQ_ROUND_STOCHASTIC, seed=sr[0],
                offset=sr[1], scale_mode=fq.FQ_SCALE_POW2 if pow2 else fq.FQ_SCALE_DEFAULT)
    out = fq.alloc_quantized(d)
    ws = fq.alloc_workspace(d)
    if amax_in is None:
        fq.fq_quantize(d, dev(x), out, ws)
    else:
        fq.fq_quantize_with_amax(d, dev(x), torch.tensor([amax_in], dtype=torch.float32, device="cuda"), out, ws)
    torch.cuda.synchronize()
    return d, out


def planes(out, outputs, want, data_keys, scale_keys=(None, None)):
    for plane, dk, sk in ((ROW, data_keys[0], scale_keys[0]), (COL, data_keys[1], scale_keys[1])):
        if not outputs & plane:
            continue
        name = "rowwise" if plane == ROW else "colwise"
        same_bytes(host(out.row_data if plane == ROW else out.col_data), want[dk], f"{name} codes")
        if sk:
            same_bytes(host(out.row_scale if plane == ROW else out.col_scale), want[sk], f"{name} scales")


def check_current(x, fmt, outputs, sr, amax_in=None):
    d, out = run(fq.FQ_PER_TENSOR_CURRENT, fmt, x, outputs, sr, amax_in=amax_in)
    if amax_in is None:
        want = orc.quantize_current(x, OFMT[fmt], outputs=outputs, sr=sr)
        same_bytes(host(out.amax), f32(want["amax"]), "amax")
    else:
        want = orc.quantize_with_amax(x, OFMT[fmt], amax_in, outputs=outputs, sr=sr)
    want.setdefault("q_row", None)
    planes(out, outputs, want, ("q_row", "q_col"))
    same_bytes(host(out.tensor_scale), f32(want["s"]), "s")
    return out


def check_block(x, outputs, sr, pow2=False):
    d, out = run(fq.FQ_BLOCK_FP32, fq.FQ_E4M3, x, outputs, sr, block=(1, 128), pow2=pow2)
    want = orc.quantize_block(x, (1, 128), outputs=outputs, pow2=pow2, sr=sr)
    planes(out, outputs, want, ("q_row", "q_col"), ("s_row", "s_col"))
    return out


def check_mx(x, fmt, outputs, sr):
    d, out = run(fq.FQ_MX, fmt, x, outputs, sr, block=(1, 32))
    want = orc.quantize_mx(x, outputs=outputs, fmt=OFMT[fmt], sr=sr)
    planes(out, outputs, want, ("q_row", "q_col"), ("e_row", "e_col"))
    return out


@pytest.mark.parametrize("fmt", [fq.FQ_E4M3, fq.FQ_E5M2])
@pytest.mark.parametrize("shape", [(1, 1), (3, 7), (17, 33), (130, 70), (129, 1000), (256, 384)])
@pytest.mark.parametrize("dt", [W.F32, W.BF16])
def test_current_sr(fmt, shape, dt):
    x = W.normal(shape, 2.0, shape[0] * 13 + shape[1], dt)
    for i, sr in enumerate(SEEDS):
        check_current(x, fmt, (ROW, COL, BOTH)[i], sr)


@pytest.mark.parametrize("fmt", [fq.FQ_E4M3, fq.FQ_E5M2])
def test_current_sr_with_amax(fmt):
    x = W.normal((96, 160), 1.0, 31, W.BF16)
    a = float(np.abs(W.bf16_bits_to_f32(x)).max())
    for amax_in in (a, 3.0 * a):
        check_current(x, fmt, BOTH, (11, 3), amax_in=amax_in)


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (384, 640), (128, 1152)])
@pytest.mark.parametrize("dt", [W.F32, W.BF16])
def test_block_1x128_sr(pow2, shape, dt):
    x = W.normal(shape, 1.0, shape[0] + 7 * shape[1], dt)
    for i, sr in enumerate(SEEDS):
        check_block(x, (ROW, COL, BOTH)[i], sr, pow2=pow2)


def test_block_1x128_sr_rowwise_odd_rows():
    check_block(W.normal((3, 256), 1.0, 5, W.BF16), ROW, (4, 4))
    check_block(W.normal((5, 384), 1.0, 6, W.F32), ROW, (4, 5))


@pytest.mark.parametrize("fmt", [fq.FQ_E4M3, fq.FQ_E5M2])
@pytest.mark.parametrize("shape", [(32, 32), (64, 96), (96, 64), (160, 288), (256, 512)])
@pytest.mark.parametrize("dt", [W.F32, W.BF16])
def test_mx_sr(fmt, shape, dt):
    x = W.student_t(shape, 3.0, shape[0] * 3 + shape[1], dt)
    for i, sr in enumerate(SEEDS):
        check_mx(x, fmt, (ROW, COL, BOTH)[i], sr)


def test_sr_wide_range_and_zero():
    x = W.uniform_bits_bf16((128, 256), 17, max_abs=1e6)
    check_current(x, fq.FQ_E4M3, BOTH, (1, 2))
    check_block(x, BOTH, (1, 2))
    check_mx(x, fq.FQ_E5M2, BOTH, (1, 2))
    z = np.zeros((128, 128), np.uint16)
    check_current(z, fq.FQ_E5M2, BOTH, (3, 4))
    check_block(z, BOTH, (3, 4))
    check_mx(z, fq.FQ_E4M3, BOTH, (3, 4))


def test_sr_repeatable_and_seeded():
    x = W.normal((256, 512), 1.0, 41, W.BF16)
    a = host(check_mx(x, fq.FQ_E4M3, BOTH, (9, 9)).row_data).copy()
    b = host(check_mx(x, fq.FQ_E4M3, BOTH, (9, 9)).row_data).copy()
    c = host(check_mx(x, fq.FQ_E4M3, BOTH, (9, 10)).row_data).copy()
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_full_size_current_e5m2_gradient_sr():
    """The E5M2 gradient workload (8192x4096 bf16) with both planes rounded stochastically."""
    check_current(W.BY_NAME["current_e5m2_grad_8192x4096"].make(), fq.FQ_E5M2, BOTH, (2027, 1))


def test_full_size_block_1x128_sr_rowwise():
    """The 1x128 activation/gradient workload (16384x7168 bf16), rowwise, stochastic."""
    check_block(W.BY_NAME["block1x128_act_16384x7168"].make(), ROW, (5, 77))


def test_full_size_mx_sr_both_planes():
    """The MXFP8 workload (8192x8192 bf16) with both planes rounded stochastically."""
    check_mx(W.BY_NAME["mxfp8_rowcol_8192x8192"].make(), fq.FQ_E4M3, BOTH, (6, 78))
