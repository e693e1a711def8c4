"""GPU parity for narrow, tall tensors: more 16-row strips, 32-row slabs,
128-row regions or 128x64 tiles than one grid holds, so the workgroups of the
NVFP4 16x16 kernels (both planes), the fp32 MXFP4 colwise kernel, the bf16 MX
and MXFP4 region walk and the stochastic-rounding tile kernel for 8-bit
elements stride over several of them. Every byte and scale is compared with
the oracle."""
import numpy as np
import pytest
import torch

import oracle as orc
from fp8_fp4_tensor_amd import fq
from fp8_fp4_tensor_amd import workloads as W
from gpu_util import dev, f32, host, same_bytes
from test_gpu_sr8 import check_current, check_mx

pytestmark = pytest.mark.gpu

BOTH = fq.FQ_ROWWISE | fq.FQ_COLWISE
# 2^21 + 64 rows: 131076 strips of 16 rows, 65538 slabs of 32 rows (more
# than the 65536 workgroups a strip or slab grid is capped at), 16385
# regions or tiles of 128 rows at up to 256 or 64 columns (more than the
# 16384 of the region walk's and the SR tile kernel's grids)
R_TALL = (1 << 21) + 64


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_nvfp4_16x16_narrow_tall(dtype):
    x = W.normal((R_TALL, 16), 0.02, 81, dtype)
    d = fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16 if dtype == W.BF16 else fq.FQ_IN_F32, fq.FQ_E2M1, R_TALL, 16,
                (16, 16), BOTH)
    out = fq.alloc_quantized(d)
    print(f"nvfp4 16x16 {R_TALL}x16 {dtype}", flush=True)
    fq.fq_quantize(d, dev(x), out, fq.alloc_workspace(d))
    torch.cuda.synchronize()
    want = orc.quantize_nvfp4(x, (16, 16), outputs=orc.ROWWISE | orc.COLWISE)
    same_bytes(host(out.row_data), want["p_row"], "packed rowwise")
    same_bytes(host(out.row_scale), want["c_row"], "block codes rowwise")
    same_bytes(host(out.col_data), want["p_col"], "packed colwise")
    same_bytes(host(out.col_scale), want["c_col"], "block codes colwise")
    same_bytes(host(out.tensor_scale), f32(want["S"]), "S")


def test_mxfp4_f32_colwise_narrow_tall():
    x = W.student_t((R_TALL, 32), 3.0, 82, W.F32)
    d = fq.desc(fq.FQ_MX, fq.FQ_IN_F32, fq.FQ_E2M1, R_TALL, 32, (1, 32), BOTH)
    out = fq.alloc_quantized(d)
    print(f"mxfp4 {R_TALL}x32 f32", flush=True)
    fq.fq_quantize(d, dev(x), out)
    torch.cuda.synchronize()
    want = orc.quantize_mx(x, outputs=orc.ROWWISE | orc.COLWISE, fmt=orc.E2M1)
    same_bytes(host(out.row_data), want["q_row"], "packed rowwise")
    same_bytes(host(out.row_scale), want["e_row"], "E8M0 rowwise")
    same_bytes(host(out.col_data), want["q_col"], "packed colwise")
    same_bytes(host(out.col_scale), want["e_col"], "E8M0 colwise")


@pytest.mark.parametrize("fmt", [fq.FQ_E4M3, fq.FQ_E2M1], ids=["mxfp8", "mxfp4"])
def test_mx_bf16_narrow_tall(fmt):
    x = W.student_t((R_TALL, 32), 3.0, 83 + fmt, W.BF16)
    d = fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fmt, R_TALL, 32, (1, 32), BOTH)
    out = fq.alloc_quantized(d)
    print(f"mx fmt {fmt} {R_TALL}x32 bf16", flush=True)
    fq.fq_quantize(d, dev(x), out)
    torch.cuda.synchronize()
    want = orc.quantize_mx(x, outputs=orc.ROWWISE | orc.COLWISE, fmt=orc.E4M3 if fmt == fq.FQ_E4M3 else orc.E2M1)
    same_bytes(host(out.row_data), want["q_row"], "rowwise codes")
    same_bytes(host(out.row_scale), want["e_row"], "E8M0 rowwise")
    same_bytes(host(out.col_data), want["q_col"], "colwise codes")
    same_bytes(host(out.col_scale), want["e_col"], "E8M0 colwise")


def test_sr8_narrow_tall():
    x = W.normal((R_TALL, 1), 2.0, 84, W.BF16)
    print(f"per-tensor E5M2 stochastic {R_TALL}x1 bf16", flush=True)
    check_current(x, fq.FQ_E5M2, BOTH, (41, 2))
    check_current(x, fq.FQ_E5M2, fq.FQ_COLWISE, (41, 3))
    x = W.student_t((R_TALL, 32), 3.0, 85, W.BF16)
    print(f"MX E4M3 stochastic {R_TALL}x32 bf16", flush=True)
    check_mx(x, fq.FQ_E4M3, BOTH, (42, 4))
