"""One GPU's share of the sharded path, at the workloads' full shapes.

[CS] "FP8 Current Scaling：量化、缩放与精度边界", section "成本与多 GPU 使用":
with the tensor split across devices, each computes its local amax, the
amaxes are reduced with max, and every shard is cast with that common scale,
so the result equals quantizing the whole tensor. Here the tensor is split
by rows into shards on one GPU; each shard's `fq_amax` goes into a device
vector whose max stands in for the all-reduce, and `fq_quantize_with_amax`
casts each shard. The shards' codes, scales and planes, put back together,
must equal the whole tensor quantized in one `fq_quantize` call (whose bytes
the other GPU tests check against the oracle). Block-local recipes need no
exchange: shards split at a multiple of the block height quantize alone.
"""
import numpy as np
import pytest
import torch

from fp8_fp4_tensor_amd import fq
from fp8_fp4_tensor_amd import workloads as W
from gpu_util import dev, f32, host, same_bytes

pytestmark = pytest.mark.gpu

ROW, COL = fq.FQ_ROWWISE, fq.FQ_COLWISE
BOTH = ROW | COL


def whole(d, x):
    out = fq.alloc_quantized(d)
    fq.fq_quantize(d, x, out, fq.alloc_workspace(d))
    return out


def split_rows(R, sizes):
    """Row ranges of the shards, in order."""
    assert sum(sizes) == R
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    return [(int(a), int(a + s)) for a, s in zip(starts, sizes)]


def sharded_two_pass(recipe, fmt, block, outputs, x, sizes):
    """fq_amax per shard, the max of the amaxes, fq_quantize_with_amax per shard."""
    R, C = x.shape
    ranges = split_rows(R, sizes)
    amax = torch.empty(len(ranges), dtype=torch.float32, device="cuda")
    for i, (a, b) in enumerate(ranges):
        d = fq.desc(recipe, fq.FQ_IN_BF16, fmt, b - a, C, block, outputs)
        fq.fq_amax(d, x[a:b], amax[i:i + 1], fq.alloc_workspace(d))
    glob = amax.max().reshape(1)  # what an all-reduce with max returns on every rank
    outs = []
    for a, b in ranges:
        d = fq.desc(recipe, fq.FQ_IN_BF16, fmt, b - a, C, block, outputs)
        out = fq.alloc_quantized(d)
        fq.fq_quantize_with_amax(d, x[a:b], glob, out, fq.alloc_workspace(d))
        outs.append(out)
    torch.cuda.synchronize()
    return ranges, glob, outs


def check_planes(ranges, outs, ref, what, rows_per_scale_row=1, col_scale_rows=1):
    """Rowwise planes concatenate by rows; colwise planes ([C, R]) by columns."""
    if outs[0].row_data is not None:
        same_bytes(np.concatenate([host(o.row_data).reshape(b - a, -1) for (a, b), o in zip(ranges, outs)]),
                   host(ref.row_data), f"{what}: rowwise codes")
        if outs[0].row_scale is not None:
            same_bytes(np.concatenate([host(o.row_scale).reshape((b - a) // rows_per_scale_row, -1)
                                       for (a, b), o in zip(ranges, outs)]),
                       host(ref.row_scale), f"{what}: rowwise scales")
    if outs[0].col_data is not None:
        C = host(ref.col_data).reshape(-1).size // ranges[-1][1]
        got = np.concatenate([host(o.col_data).reshape(C, -1) for o in outs], axis=1)
        same_bytes(got, host(ref.col_data).reshape(C, -1), f"{what}: colwise codes")
        if outs[0].col_scale is not None:
            got = np.concatenate([host(o.col_scale).reshape(C // col_scale_rows, -1) for o in outs], axis=1)
            same_bytes(got, host(ref.col_scale).reshape(C // col_scale_rows, -1), f"{what}: colwise scales")


@pytest.mark.parametrize("name,fmt", [("current_e4m3_act_8192x4096", fq.FQ_E4M3),
                                      ("current_e5m2_grad_8192x4096", fq.FQ_E5M2)], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("sizes", [[1024] * 8, [1000, 1048, 2000, 96, 1, 4047]], ids=["even", "ragged"])
def test_sharded_current(name, fmt, sizes):
    xh = W.BY_NAME[name].make()
    x = dev(xh)
    d = fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_BF16, fmt, *xh.shape, (0, 0), BOTH)
    ref = whole(d, x)
    ranges, glob, outs = sharded_two_pass(fq.FQ_PER_TENSOR_CURRENT, fmt, (0, 0), BOTH, x, sizes)
    same_bytes(host(glob), f32(np.abs(W.bf16_bits_to_f32(xh)).max()), "max of the shard amaxes")
    for o in outs:
        same_bytes(host(o.tensor_scale), host(ref.tensor_scale), "s")
    check_planes(ranges, outs, ref, name)


@pytest.mark.parametrize("name,block,sizes", [
    ("nvfp4_1x16_act_8192x14336", (1, 16), [1024] * 8),
    ("nvfp4_16x16_wgt_14336x4096", (16, 16), [1792] * 8),
], ids=["nvfp4_1x16", "nvfp4_16x16"])
def test_sharded_nvfp4(name, block, sizes):
    xh = W.BY_NAME[name].make()
    x = dev(xh)
    d = fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, *xh.shape, block, ROW)
    ref = whole(d, x)
    ranges, glob, outs = sharded_two_pass(fq.FQ_NVFP4, fq.FQ_E2M1, block, ROW, x, sizes)
    for o in outs:
        same_bytes(host(o.tensor_scale), host(ref.tensor_scale), "S")
    check_planes(ranges, outs, ref, name, rows_per_scale_row=block[0])


@pytest.mark.parametrize("name,recipe,fmt,block,outputs,sizes", [
    ("block1x128_act_16384x7168", fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (1, 128), ROW, [2048] * 8),
    ("block128x128_wgt_7168x18432", fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (128, 128), BOTH, [896] * 8),
    ("mxfp8_rowcol_8192x8192", fq.FQ_MX, fq.FQ_E4M3, (1, 32), BOTH, [1024] * 8),
], ids=["block1x128", "block128x128", "mxfp8"])
def test_sharded_block_local(name, recipe, fmt, block, outputs, sizes):
    xh = W.BY_NAME[name].make()
    x = dev(xh)
    R, C = xh.shape
    ref = whole(fq.desc(recipe, fq.FQ_IN_BF16, fmt, R, C, block, outputs), x)
    ranges = split_rows(R, sizes)
    outs = [whole(fq.desc(recipe, fq.FQ_IN_BF16, fmt, b - a, C, block, outputs), x[a:b]) for a, b in ranges]
    torch.cuda.synchronize()
    # colwise scale planes: [C/128, R/128] for 128x128 tiles, [C, R/32] for MX
    check_planes(ranges, outs, ref, name, rows_per_scale_row=block[0],
                 col_scale_rows=128 if block == (128, 128) else 1)


@pytest.mark.parametrize("sizes", [[1024] * 8, [1000, 1048, 2000, 96, 1, 4047]], ids=["even", "ragged"])
def test_sharded_delayed(sizes):
    """Delayed scaling across shards: after each step, an all-reduce with max
    over the shards' pending records (viewed as 32-bit integers: every word
    is a non-negative float or the same on every shard) gives every shard the
    whole tensor's record, so its next step scales with the global window."""
    w = W.BY_NAME["delayed_e4m3_act_8192x4096"]
    R, C = w.shape
    H = w.extra["history_len"]
    # steps of different magnitude (power-of-two factors keep bf16 exact)
    xs = [dev(w.make(w.seed + t)) * f for t, f in enumerate([1.0, 4.0, 0.25, 2.0, 0.5])]
    d = fq.desc(fq.FQ_PER_TENSOR_DELAYED, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C)
    st, out = fq.DelayedState(H), fq.alloc_quantized(d)
    ranges = split_rows(R, sizes)
    ds = [fq.desc(fq.FQ_PER_TENSOR_DELAYED, fq.FQ_IN_BF16, fq.FQ_E4M3, b - a, C) for a, b in ranges]
    sts = [fq.DelayedState(H) for _ in ranges]
    outs = [fq.alloc_quantized(dd) for dd in ds]
    for t, x in enumerate(xs):
        fq.fq_quantize_delayed(d, x, st, out)
        for (a, b), dd, s, o in zip(ranges, ds, sts, outs):
            fq.fq_quantize_delayed(dd, x[a:b], s, o)
        red = torch.stack([s.pending for s in sts]).view(torch.int32).amax(0).view(torch.float32)
        for s in sts:
            s.pending.copy_(red)
        torch.cuda.synchronize()
        same_bytes(np.concatenate([host(o.row_data) for o in outs]), host(out.row_data), f"step {t} codes")
        for o in outs:
            same_bytes(host(o.tensor_scale), host(out.tensor_scale), f"step {t} s used")
    fq.fq_delayed_flush(d, st)
    for dd, s in zip(ds, sts):
        fq.fq_delayed_flush(dd, s)
    torch.cuda.synchronize()
    for s in sts:
        same_bytes(host(s.amax_history), host(st.amax_history), "window")
        same_bytes(host(s.scale), host(st.scale), "scale")
        same_bytes(host(s.scale_inv), host(st.scale_inv), "scale_inv")
