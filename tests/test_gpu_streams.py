"""GPU: every entry point enqueues all of its work on the stream it is given.

Calls are made on side streams (default priority), the default stream is
left idle, and only the side streams are synchronized before the results are
read; two calls on two streams at once, each with its own workspace and
outputs, must both match the oracle byte for byte."""
import numpy as np
import pytest
import torch

import oracle as orc
from fp8_fp4_tensor_amd import fq
from fp8_fp4_tensor_amd import workloads as W
from gpu_util import dev, host, same_bytes

pytestmark = pytest.mark.gpu

BOTH = fq.FQ_ROWWISE | fq.FQ_COLWISE


def on_stream(s, fn):
    s.wait_stream(torch.cuda.current_stream())   # inputs and outputs were made on the default stream
    fn()
    s.synchronize()


def test_current_on_a_side_stream():
    x = W.normal((512, 1024), 3.0, 91, W.BF16)
    xd = dev(x)
    d = fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_BF16, fq.FQ_E4M3, 512, 1024, (0, 0), BOTH)
    out, ws = fq.alloc_quantized(d), fq.alloc_workspace(d)
    s = torch.cuda.Stream()
    on_stream(s, lambda: fq.fq_quantize(d, xd, out, ws, stream=s))
    want = orc.quantize_current(x, orc.E4M3, outputs=BOTH)
    same_bytes(host(out.row_data), want["q_row"], "rowwise codes")
    same_bytes(host(out.col_data), want["q_col"], "colwise codes")
    same_bytes(host(out.tensor_scale), np.float32(want["s"]), "scale")


def test_delayed_steps_on_a_side_stream():
    d = fq.desc(fq.FQ_PER_TENSOR_DELAYED, fq.FQ_IN_BF16, fq.FQ_E5M2, 256, 512, (0, 0), fq.FQ_ROWWISE)
    st, ost = fq.DelayedState(16), orc.DelayedState(16)
    ws = fq.alloc_workspace(d)
    s = torch.cuda.Stream()
    for t in range(3):
        x = W.normal((256, 512), 0.5 + t, 300 + t, W.BF16)
        xd = dev(x)
        out = fq.alloc_quantized(d)
        on_stream(s, lambda: fq.fq_quantize_delayed(d, xd, st, out, ws, stream=s))
        want = orc.quantize_delayed(x, orc.E5M2, ost)
        same_bytes(host(out.row_data), want["q_row"], f"step {t} codes")
    on_stream(s, lambda: fq.fq_delayed_flush(d, st, stream=s))
    same_bytes(host(st.scale), np.float32(ost.alpha), "next alpha")


def test_two_streams_at_once():
    xa = W.normal((1024, 2048), 1.0, 92, W.BF16)
    xb = W.student_t((1024, 2048), 3.0, 93, W.BF16)
    da = fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, 1024, 2048, (1, 16), fq.FQ_ROWWISE,
                 rounding=fq.FQ_ROUND_STOCHASTIC, seed=5, offset=7)
    db = fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, 1024, 2048, (1, 32), BOTH)
    xad, xbd = dev(xa), dev(xb)
    oa, ob = fq.alloc_quantized(da), fq.alloc_quantized(db)
    wa, wb = fq.alloc_workspace(da), fq.alloc_workspace(db)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    cur = torch.cuda.current_stream()
    sa.wait_stream(cur)
    sb.wait_stream(cur)
    for _ in range(4):                     # repeated: the last call of each stream must still be right
        fq.fq_quantize(da, xad, oa, wa, stream=sa)
        fq.fq_quantize(db, xbd, ob, wb, stream=sb)
    sa.synchronize()
    sb.synchronize()
    want_a = orc.quantize_nvfp4(xa, (1, 16), sr=(5, 7))
    same_bytes(host(oa.row_data), want_a["p_row"], "NVFP4 SR packed codes")
    same_bytes(host(oa.row_scale), want_a["c_row"], "NVFP4 block scales")
    want_b = orc.quantize_mx(xb, outputs=BOTH)
    same_bytes(host(ob.row_data), want_b["q_row"], "MX rowwise codes")
    same_bytes(host(ob.col_data), want_b["q_col"], "MX colwise codes")
