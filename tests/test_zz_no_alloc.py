"""fq_quantize_noalloc against fq_quantize, through the C ABI.

The no-allocation entry point takes its amax scratch from the library's own
per-GPU array instead of a caller workspace. Its bytes and scales must equal
fq_quantize's on the same input, bit for bit, on two calls in a row (the
second smaller, so it reuses the array the first left behind), on the
recipes that use the scratch (per-tensor current, NVFP4) and on one that
does not (blockwise)."""
import ctypes

import pytest
import torch

from fp8_fp4_tensor_amd import fq
from fp8_fp4_tensor_amd import workloads as W
from gpu_util import dev, host, same_bytes

pytestmark = pytest.mark.gpu

PLANES = ("row_data", "row_scale", "col_data", "col_scale", "tensor_scale", "amax")


def both_ways(d, x):
    """(fq_quantize result, fq_quantize_noalloc result) on one input."""
    xd = dev(x)
    ref = fq.alloc_quantized(d)
    fq.fq_quantize(d, xd, ref, fq.alloc_workspace(d))
    got = fq.alloc_quantized(d)
    # the raw C call, as a caller that cannot allocate would make it
    q = got.c()
    rc = fq.lib().fq_quantize_noalloc(ctypes.byref(d), ctypes.c_void_p(xd.data_ptr()), ctypes.byref(q),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == fq.FQ_OK, fq.status_str(rc)
    torch.cuda.synchronize()
    return ref, got


def check_same(ref, got, what, d):
    """Every plane the recipe writes (block recipes write no tensor scale or amax)."""
    names = PLANES if d.recipe in (fq.FQ_PER_TENSOR_CURRENT, fq.FQ_NVFP4) else PLANES[:4]
    for name in names:
        a, b = getattr(ref, name), getattr(got, name)
        if a is None:
            continue
        same_bytes(host(b), host(a), f"{what}: {name}")


CASES = [
    ("current e4m3 bf16", lambda R, C: fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C),
     [(2048, 4096), (1000, 333)], lambda s, seed: W.normal(s, 1.0, seed, W.BF16)),
    ("current e5m2 f32 both planes",
     lambda R, C: fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_F32, fq.FQ_E5M2, R, C,
                          outputs=fq.FQ_ROWWISE | fq.FQ_COLWISE),
     [(1024, 1536), (96, 80)], lambda s, seed: W.normal(s, 1e-3, seed, W.F32)),
    ("nvfp4 1x16 both planes",
     lambda R, C: fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (1, 16), fq.FQ_ROWWISE | fq.FQ_COLWISE),
     [(2048, 2048), (256, 512)], lambda s, seed: W.normal(s, 1.0, seed, W.BF16)),
    ("nvfp4 16x16", lambda R, C: fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (16, 16)),
     [(1024, 4096), (64, 128)], lambda s, seed: W.normal(s, 0.02, seed, W.BF16)),
    ("block 1x128", lambda R, C: fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 128)),
     [(512, 1024), (128, 256)], lambda s, seed: W.normal(s, 1.0, seed, W.BF16)),
    ("current e5m2 bf16 stochastic both planes",
     lambda R, C: fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_BF16, fq.FQ_E5M2, R, C,
                          outputs=fq.FQ_ROWWISE | fq.FQ_COLWISE, rounding=fq.FQ_ROUND_STOCHASTIC, seed=3, offset=4),
     [(1024, 2048), (130, 70)], lambda s, seed: W.normal(s, 1e-3, seed, W.BF16)),
]


@pytest.mark.parametrize("name,make_desc,shapes,make_x", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_quantize_two_calls(name, make_desc, shapes, make_x):
    for k, (R, C) in enumerate(shapes):
        print(f"noalloc {name} call {k} {R}x{C}", flush=True)
        x = make_x((R, C), 600 + 10 * k)
        d = make_desc(R, C)
        ref, got = both_ways(d, x)
        check_same(ref, got, f"{name} call {k} {R}x{C}", d)


def test_noalloc_on_a_side_stream_and_errors():
    """On a non-default stream; an invalid desc is rejected before anything runs."""
    s = torch.cuda.Stream()
    x = W.normal((512, 768), 1.0, 650, W.BF16)
    d = fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_BF16, fq.FQ_E4M3, 512, 768)
    ref = fq.alloc_quantized(d)
    xd = dev(x)
    fq.fq_quantize(d, xd, ref, fq.alloc_workspace(d))
    got = fq.alloc_quantized(d)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        fq.fq_quantize_noalloc(d, xd, got, stream=s)
    s.synchronize()
    check_same(ref, got, "side stream", d)
    bad = fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, 64, 48, (1, 32))   # cols % 32 != 0
    q = got.c()
    rc = fq.lib().fq_quantize_noalloc(ctypes.byref(bad), ctypes.c_void_p(xd.data_ptr()), ctypes.byref(q), None)
    assert rc == fq.FQ_E_SHAPE
    dd = fq.desc(fq.FQ_PER_TENSOR_DELAYED, fq.FQ_IN_BF16, fq.FQ_E4M3, 64, 64)
    rc = fq.lib().fq_quantize_noalloc(ctypes.byref(dd), ctypes.c_void_p(xd.data_ptr()), ctypes.byref(q), None)
    assert rc == fq.FQ_E_UNSUPPORTED
