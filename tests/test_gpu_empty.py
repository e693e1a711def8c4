"""GPU: empty tensors (a zero row or column count) for every recipe and entry
point. Nothing is read or written but the scalars an empty tensor still has:
its amax is 0, so NVFP4's tensor scale is 1 (the all-zero reading of the
per-tensor scale: alpha = s = 1 when a = 0), and a delayed step records 0 in
its window slot."""
import numpy as np
import pytest
import torch

import oracle as orc
from fp8_fp4_tensor_amd import fq
from gpu_util import host

pytestmark = pytest.mark.gpu

BOTH = fq.FQ_ROWWISE | fq.FQ_COLWISE
SHAPES = [(0, 0), (0, 256), (256, 0)]

# (id, recipe, format, block, outputs, extra desc fields)
CASES = [
    ("current_e4m3", fq.FQ_PER_TENSOR_CURRENT, fq.FQ_E4M3, (0, 0), BOTH, {}),
    ("block_1x128", fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (1, 128), BOTH, {}),
    ("block_128x128", fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (128, 128), BOTH, {}),
    ("block_128x128_pow2", fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (128, 128), BOTH, {"scale_mode": fq.FQ_SCALE_POW2}),
    ("mxfp8", fq.FQ_MX, fq.FQ_E4M3, (1, 32), BOTH, {}),
    ("mx_e5m2", fq.FQ_MX, fq.FQ_E5M2, (1, 32), BOTH, {}),
    ("mxfp4", fq.FQ_MX, fq.FQ_E2M1, (1, 32), BOTH, {}),
    ("nvfp4_1x16", fq.FQ_NVFP4, fq.FQ_E2M1, (1, 16), BOTH, {}),
    ("nvfp4_16x16", fq.FQ_NVFP4, fq.FQ_E2M1, (16, 16), BOTH, {}),
    ("nvfp4_1x16_sr", fq.FQ_NVFP4, fq.FQ_E2M1, (1, 16), BOTH,
     {"rounding": fq.FQ_ROUND_STOCHASTIC, "seed": 7, "offset": 1}),
    ("nvfp4_rht", fq.FQ_NVFP4, fq.FQ_E2M1, (1, 16), fq.FQ_COLWISE,
     {"transform": fq.FQ_TRANSFORM_RHT16, "rht_signs": 0x5A3C}),
    ("current_sr", fq.FQ_PER_TENSOR_CURRENT, fq.FQ_E5M2, (0, 0), BOTH,
     {"rounding": fq.FQ_ROUND_STOCHASTIC, "seed": 7, "offset": 1}),
    ("block_1x128_sr", fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (1, 128), BOTH,
     {"rounding": fq.FQ_ROUND_STOCHASTIC, "seed": 7, "offset": 1}),
    ("mx_sr", fq.FQ_MX, fq.FQ_E4M3, (1, 32), BOTH, {"rounding": fq.FQ_ROUND_STOCHASTIC, "seed": 7, "offset": 1}),
]

SENTINEL = -7.0


def sentinel_scalars(out):
    out.tensor_scale.fill_(SENTINEL)
    out.amax.fill_(SENTINEL)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_empty_quantize_and_dequantize(case, shape, dt):
    name, recipe, fmt, block, outputs, extra = case
    R, C = shape
    d = fq.desc(recipe, fq.FQ_IN_BF16 if dt == torch.bfloat16 else fq.FQ_IN_F32, fmt, R, C, block, outputs,
                **extra)
    z = fq.fq_sizes(d)
    assert z.row_data == z.row_scale == z.col_data == z.col_scale == 0, z
    out = fq.alloc_quantized(d)
    sentinel_scalars(out)
    ws = fq.alloc_workspace(d)
    x = torch.empty(16, dtype=dt, device="cuda")  # a valid pointer; no element is read
    fq.fq_quantize(d, x, out, ws)
    torch.cuda.synchronize()
    if recipe in (fq.FQ_PER_TENSOR_CURRENT, fq.FQ_NVFP4):
        assert host(out.tensor_scale)[0] == 1.0 and host(out.amax)[0] == 0.0
        a0 = torch.zeros(1, dtype=torch.float32, device="cuda")
        sentinel_scalars(out)
        fq.fq_quantize_with_amax(d, x, a0, out, ws)
        a1 = torch.full((1,), SENTINEL, dtype=torch.float32, device="cuda")
        fq.fq_amax(d, x, a1, ws if ws is not None else torch.empty(4096, dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        assert host(out.tensor_scale)[0] == 1.0 and host(a1)[0] == 0.0
    else:
        # the block recipes have no tensor scalars: they stay untouched
        assert host(out.tensor_scale)[0] == SENTINEL and host(out.amax)[0] == SENTINEL
    for which in (fq.FQ_ROWWISE, fq.FQ_COLWISE):
        if d.outputs & which:
            for ydt in (torch.float32, torch.bfloat16):
                fq.fq_dequantize(d, out, which, torch.empty(16, dtype=ydt, device="cuda"))
    if recipe == fq.FQ_MX and fmt == fq.FQ_E4M3 and not extra.get("rounding"):
        fq.fq_requantize_transpose(d, out, fq.alloc_quantized(d))
    torch.cuda.synchronize()


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("fmt", [fq.FQ_E4M3, fq.FQ_E5M2], ids=["e4m3", "e5m2"])
def test_empty_delayed_step(shape, fmt):
    """Empty steps between real ones, in a window of 2: an empty step records
    amax 0 in its slot and takes the scale from what the window still holds,
    as the oracle does for a step whose tensor is all zeros (its amax is 0
    too); once the window holds only zeros the scale stays as it was."""
    rng = np.random.default_rng(11)
    x1 = (rng.standard_normal((8, 32)) * 3).astype(np.float32)
    H = 2
    st, ost = fq.DelayedState(H), orc.DelayedState(H)
    ofmt = orc.E4M3 if fmt == fq.FQ_E4M3 else orc.E5M2
    d1 = fq.desc(fq.FQ_PER_TENSOR_DELAYED, fq.FQ_IN_F32, fmt, 8, 32)
    out1, ws1 = fq.alloc_quantized(d1), fq.alloc_workspace(d1)
    d0 = fq.desc(fq.FQ_PER_TENSOR_DELAYED, fq.FQ_IN_F32, fmt, shape[0], shape[1], outputs=BOTH)
    out0, ws0 = fq.alloc_quantized(d0), fq.alloc_workspace(d0)
    zero = np.zeros((1, 1), np.float32)
    fq.fq_quantize_delayed(d1, torch.from_numpy(x1).cuda(), st, out1, ws1)
    orc.quantize_delayed(x1, ofmt, ost)
    for t in range(3):  # the window of 2 forgets x1 after the second empty step
        out0.amax.fill_(SENTINEL)
        fq.fq_quantize_delayed(d0, torch.empty(16, dtype=torch.float32, device="cuda"), st, out0, ws0)
        orc.quantize_delayed(zero, ofmt, ost)
        fq.fq_delayed_flush(d0, st)
        torch.cuda.synchronize()
        assert host(out0.amax)[0] == 0.0
        assert np.array_equal(host(st.amax_history).view(np.uint32), ost.hist.view(np.uint32)), t
        assert host(st.scale).view(np.uint32)[0] == np.float32(ost.alpha).view(np.uint32), t
        assert host(st.scale_inv).view(np.uint32)[0] == np.float32(ost.s).view(np.uint32), t
    assert ost.hist.max() == 0.0 and ost.alpha != 1.0  # the scale from x1 was kept
