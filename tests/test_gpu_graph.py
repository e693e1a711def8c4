"""GPU: quantize calls captured in a HIP graph replay correctly.

The library enqueues kernels only (no allocation, no memset, no
synchronization), so a sequence of calls can be captured once and replayed.
Per-tensor current scaling (two kernels and a workspace), blockwise, MX and
NVFP4 are captured together; every replay follows eager work on the same
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
    fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (128, 128), BOTH),
    fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 32), BOTH),
    fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (1, 16), BOTH),
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
