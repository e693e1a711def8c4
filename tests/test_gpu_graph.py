"""GPU: quantize calls captured in a HIP graph replay correctly.

The library enqueues kernels only (no allocation, no memset, no
synchronization), so a sequence of calls can be captured once and replayed.
Per-tensor current scaling (two kernels and a workspace), blockwise (both
tile shapes, power-of-two scales), MX (E4M3, E5M2, E2M1 elements), NVFP4
(both block shapes, stochastic rounding, the Hadamard transform) and the
stochastic rounding of 8-bit elements are captured together; every replay follows eager work on the same
buffers (outputs cleared, a new input copied in) and a synchronization, and
each replay's bytes are checked against an eager call on that input."""
import numpy as np
import pytest
import torch

from fp8_fp4_tensor_amd import fq
from fp8_fp4_tensor_amd import workloads as W
from gpu_util import dev, host, same_bytes

pytestmark = pytest.mark.gpu

BOTH = fq.FQ_ROWWISE | fq.FQ_COLWISE
R, C = 512, 1024

DESCS = [
    fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (0, 0), BOTH),
    fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_BF16, fq.FQ_E5M2, R, C, (0, 0), fq.FQ_COLWISE),
    fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (128, 128), BOTH),
    fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 128), BOTH),
    fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 128), fq.FQ_ROWWISE,
            scale_mode=fq.FQ_SCALE_POW2),
    fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 32), BOTH),
    fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E5M2, R, C, (1, 32), BOTH),
    fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (1, 32), BOTH),
    fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (1, 16), BOTH),
    fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (16, 16), BOTH),
    fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (1, 16), BOTH,
            rounding=fq.FQ_ROUND_STOCHASTIC, seed=77, offset=5),
    fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (1, 16), fq.FQ_COLWISE,
            rounding=fq.FQ_ROUND_STOCHASTIC, seed=78, offset=6, transform=fq.FQ_TRANSFORM_RHT16, rht_signs=0xA5C3),
    fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_BF16, fq.FQ_E5M2, R, C, (0, 0), BOTH,
            rounding=fq.FQ_ROUND_STOCHASTIC, seed=79, offset=7),
    fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 128), BOTH,
            rounding=fq.FQ_ROUND_STOCHASTIC, seed=80, offset=8),
    fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 32), BOTH,
            rounding=fq.FQ_ROUND_STOCHASTIC, seed=81, offset=9),
]


def planes(out, d):
    """The planes d's recipe writes (tensor_scale only for per-tensor and NVFP4)."""
    ts = out.tensor_scale if d.recipe in (fq.FQ_PER_TENSOR_CURRENT, fq.FQ_NVFP4) else None
    return [t for t in (out.row_data, out.row_scale, out.col_data, out.col_scale, ts) if t is not None]


def eager(x):
    """Bytes of every plane of every desc, from ordinary calls on x."""
    res = []
    for d in DESCS:
        out = fq.alloc_quantized(d)
        fq.fq_quantize(d, x, out, fq.alloc_workspace(d))
        torch.cuda.synchronize()
        res.append([host(p).copy() for p in planes(out, d)])
    return res


def test_graph_replays_match_eager_calls():
    x = dev(W.normal((R, C), 2.0, 501, W.BF16))
    outs = [fq.alloc_quantized(d) for d in DESCS]
    wss = [fq.alloc_workspace(d) for d in DESCS]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                 # warm-up outside the capture
        for d, o, w in zip(DESCS, outs, wss):
            fq.fq_quantize(d, x, o, w)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for d, o, w in zip(DESCS, outs, wss):
            fq.fq_quantize(d, x, o, w)

    for replay in range(3):
        new = dev(W.student_t((R, C), 3.0, 600 + replay, W.BF16))
        x.copy_(new)                           # eager work on the captured buffers
        for o, d in zip(outs, DESCS):
            for p in planes(o, d):
                p.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = eager(new)
        for k, (o, d) in enumerate(zip(outs, DESCS)):
            for j, p in enumerate(planes(o, d)):
                same_bytes(host(p), want[k][j], f"replay {replay}, desc {k}, plane {j}")


def split_calls(x, bufs):
    """The sharded two-call path (fq_amax, then fq_quantize_with_amax for a
    per-tensor and an NVFP4 desc), dequantization to fp32 and bf16, and the
    MX rowwise -> colwise requantization, all on one stream."""
    d_cur, d_nv, d_mx, d_mxc = bufs["descs"]
    fq.fq_amax(d_cur, x, bufs["amax"], bufs["ws_cur"])
    fq.fq_quantize_with_amax(d_cur, x, bufs["amax"], bufs["out_cur"], bufs["ws_cur"])
    fq.fq_quantize_with_amax(d_nv, x, bufs["amax"], bufs["out_nv"], bufs["ws_nv"])
    fq.fq_dequantize(d_nv, bufs["out_nv"], fq.FQ_COLWISE, bufs["y"])
    fq.fq_dequantize(d_cur, bufs["out_cur"], fq.FQ_ROWWISE, bufs["yb"])
    fq.fq_quantize(d_mx, x, bufs["out_mx"], bufs["ws_mx"])
    fq.fq_requantize_transpose(d_mx, bufs["out_mx"], bufs["dst_mx"])


def split_buffers():
    d_cur = fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (0, 0), fq.FQ_ROWWISE)
    d_nv = fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (1, 16), BOTH)
    d_mx = fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 32), fq.FQ_ROWWISE)
    d_mxc = fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 32), fq.FQ_COLWISE)
    return {"descs": (d_cur, d_nv, d_mx, d_mxc),
            "amax": torch.empty(1, dtype=torch.float32, device="cuda"),
            "ws_cur": fq.alloc_workspace(d_cur), "ws_nv": fq.alloc_workspace(d_nv), "ws_mx": fq.alloc_workspace(d_mx),
            "out_cur": fq.alloc_quantized(d_cur), "out_nv": fq.alloc_quantized(d_nv),
            "out_mx": fq.alloc_quantized(d_mx), "dst_mx": fq.alloc_quantized(d_mxc),
            "y": torch.empty((C, R), dtype=torch.float32, device="cuda"),
            "yb": torch.empty((R, C), dtype=torch.bfloat16, device="cuda")}


def split_results(b):
    return [host(t).copy() for t in (b["amax"], b["out_cur"].row_data, b["out_cur"].tensor_scale,
                                     b["out_nv"].row_data, b["out_nv"].row_scale, b["out_nv"].col_data,
                                     b["out_nv"].col_scale, b["out_nv"].tensor_scale, b["y"],
                                     b["yb"].view(torch.int16), b["out_mx"].row_data, b["dst_mx"].col_data,
                                     b["dst_mx"].col_scale)]


def test_graph_split_amax_dequantize_requantize():
    x = dev(W.normal((R, C), 1.5, 701, W.BF16))
    b = split_buffers()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                 # warm-up outside the capture
        split_calls(x, b)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        split_calls(x, b)

    for replay in range(3):
        new = dev(W.student_t((R, C), 3.0, 710 + replay, W.BF16))
        x.copy_(new)
        for key in ("out_cur", "out_nv", "out_mx", "dst_mx"):
            o = b[key]
            for p in (o.row_data, o.row_scale, o.col_data, o.col_scale, o.tensor_scale):
                if p is not None:
                    p.zero_()
        b["y"].zero_()
        b["yb"].zero_()
        b["amax"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = split_results(b)
        e = split_buffers()
        split_calls(new, e)
        torch.cuda.synchronize()
        for j, (g_, w_) in enumerate(zip(got, split_results(e))):
            same_bytes(g_, w_, f"replay {replay}, result {j}")
