"""The C ABI on the host (no GPU): exports, sizes and argument validation.

Every call here fails validation (or is fq_sizes / fq_status_str), so no HIP
call is made.
"""
import ctypes
import os
import re

import pytest

from conftest import ROOT
from fp8_fp4_tensor_amd import fq

HEADER = os.path.join(ROOT, "include", "fq.h")
B = 0x10000  # an aligned fake device address: only reached by failing calls


@pytest.fixture(scope="module")
def L():
    return fq.lib()


def declared_functions():
    with open(HEADER, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fq_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert {"fq_sizes", "fq_quantize", "fq_amax", "fq_quantize_with_amax", "fq_quantize_delayed",
            "fq_dequantize", "fq_requantize_transpose", "fq_status_str"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_binding_has_every_entry_point_by_name():
    for n in declared_functions():
        assert callable(getattr(fq, n, None)), n


def test_status_strings(L):
    for s in range(7):
        assert fq.status_str(s).startswith("FQ_")
    assert fq.status_str(99) == "unknown fq_status"


def sizes(recipe, fmt, R, C, block=(0, 0), outputs=fq.FQ_ROWWISE, dt=fq.FQ_IN_BF16):
    return fq.fq_sizes(fq.desc(recipe, dt, fmt, R, C, block, outputs))


def test_sizes_per_recipe():
    both = fq.FQ_ROWWISE | fq.FQ_COLWISE
    z = sizes(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_E4M3, 8192, 4096)
    assert (z.row_data, z.row_scale, z.col_data, z.col_scale) == (8192 * 4096, 0, 0, 0) and z.workspace == 4096
    assert sizes(fq.FQ_PER_TENSOR_DELAYED, fq.FQ_E4M3, 8192, 4096).workspace == 4096
    z = sizes(fq.FQ_BLOCK_FP32, fq.FQ_E4M3, 16384, 7168, (1, 128), both)
    assert (z.row_data, z.row_scale) == (16384 * 7168, 16384 * 56 * 4)
    # block and MX quantization need no workspace, but fq_amax on the same desc does
    assert (z.col_data, z.col_scale) == (16384 * 7168, 7168 * 128 * 4) and z.workspace == 4096
    z = sizes(fq.FQ_BLOCK_FP32, fq.FQ_E4M3, 7168, 18432, (128, 128), both)
    assert (z.row_scale, z.col_scale) == (56 * 144 * 4, 144 * 56 * 4)
    z = sizes(fq.FQ_MX, fq.FQ_E4M3, 8192, 8192, (1, 32), both)
    assert (z.row_data, z.row_scale, z.col_data, z.col_scale) == (8192 ** 2, 8192 * 256, 8192 ** 2, 8192 * 256)
    assert z.workspace == 4096
    z = sizes(fq.FQ_NVFP4, fq.FQ_E2M1, 8192, 14336, (1, 16), both)
    assert (z.row_data, z.row_scale) == (8192 * 7168, 8192 * 896)
    assert (z.col_data, z.col_scale) == (8192 * 7168, 14336 * 512) and z.workspace == 4096
    z = sizes(fq.FQ_NVFP4, fq.FQ_E2M1, 14336, 4096, (16, 16))
    assert (z.row_data, z.row_scale) == (14336 * 2048, 896 * 256)
    z = sizes(fq.FQ_PER_TENSOR_DELAYED, fq.FQ_E5M2, 0, 0)
    assert z.row_data == 0


@pytest.mark.parametrize("recipe,fmt,R,C,block,outputs,want", [
    (9, 0, 4, 4, (0, 0), 1, fq.FQ_E_INVALID),
    (0, 7, 4, 4, (0, 0), 1, fq.FQ_E_INVALID),
    (0, 0, -1, 4, (0, 0), 1, fq.FQ_E_INVALID),
    (0, 0, 4, 4, (0, 0), 0, fq.FQ_E_INVALID),
    (0, 0, 4, 4, (0, 0), 4, fq.FQ_E_INVALID),
    (0, fq.FQ_E2M1, 4, 4, (0, 0), 1, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_BLOCK_FP32, fq.FQ_E5M2, 128, 128, (1, 128), 1, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_BLOCK_FP32, fq.FQ_E4M3, 128, 128, (1, 64), 1, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_BLOCK_FP32, fq.FQ_E4M3, 128, 100, (1, 128), 1, fq.FQ_E_SHAPE),
    (fq.FQ_BLOCK_FP32, fq.FQ_E4M3, 100, 128, (128, 128), 1, fq.FQ_E_SHAPE),
    (fq.FQ_BLOCK_FP32, fq.FQ_E4M3, 100, 128, (1, 128), 2, fq.FQ_E_SHAPE),
    (fq.FQ_MX, fq.FQ_E4M3, 32, 48, (1, 32), 1, fq.FQ_E_SHAPE),
    (fq.FQ_MX, fq.FQ_E4M3, 48, 64, (1, 32), 3, fq.FQ_E_SHAPE),
    (fq.FQ_MX, fq.FQ_E4M3, 32, 64, (32, 32), 1, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_NVFP4, fq.FQ_E4M3, 16, 16, (1, 16), 1, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_NVFP4, fq.FQ_E2M1, 8, 16, (16, 16), 1, fq.FQ_E_SHAPE),
    (fq.FQ_NVFP4, fq.FQ_E2M1, 16, 24, (1, 16), 1, fq.FQ_E_SHAPE),
    (fq.FQ_NVFP4, fq.FQ_E2M1, 16, 32, (1, 8), 1, fq.FQ_E_UNSUPPORTED),
    (0, 0, 1 << 21, 1 << 20, (0, 0), 1, fq.FQ_E_SHAPE),
    (0, 0, (1 << 18) + 1, 1 << 18, (0, 0), 1, fq.FQ_E_SHAPE),
])
def test_desc_validation(L, recipe, fmt, R, C, block, outputs, want):
    d = fq.desc(recipe, fq.FQ_IN_BF16, fmt, R, C, block, outputs)
    z = [ctypes.c_size_t() for _ in range(5)]
    assert L.fq_sizes(ctypes.byref(d), *[ctypes.byref(v) for v in z]) == want
    q = fq.FqQuantized(fq.FqPlane(B, B), fq.FqPlane(B, B), B, B)
    assert L.fq_quantize(ctypes.byref(d), B, ctypes.byref(q), B, 1 << 20, None) == want


@pytest.mark.parametrize("recipe,fmt,block,rounding,scale_mode,want", [
    (fq.FQ_NVFP4, fq.FQ_E2M1, (1, 16), fq.FQ_ROUND_STOCHASTIC, 0, fq.FQ_OK),
    (fq.FQ_NVFP4, fq.FQ_E2M1, (16, 16), fq.FQ_ROUND_STOCHASTIC, 0, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_PER_TENSOR_CURRENT, fq.FQ_E4M3, (0, 0), fq.FQ_ROUND_STOCHASTIC, 0, fq.FQ_OK),
    (fq.FQ_PER_TENSOR_CURRENT, fq.FQ_E5M2, (0, 0), fq.FQ_ROUND_STOCHASTIC, 0, fq.FQ_OK),
    (fq.FQ_PER_TENSOR_DELAYED, fq.FQ_E5M2, (0, 0), fq.FQ_ROUND_STOCHASTIC, 0, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (1, 128), fq.FQ_ROUND_STOCHASTIC, 0, fq.FQ_OK),
    (fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (1, 128), fq.FQ_ROUND_STOCHASTIC, fq.FQ_SCALE_POW2, fq.FQ_OK),
    (fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (128, 128), fq.FQ_ROUND_STOCHASTIC, 0, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_MX, fq.FQ_E4M3, (1, 32), fq.FQ_ROUND_STOCHASTIC, 0, fq.FQ_OK),
    (fq.FQ_MX, fq.FQ_E5M2, (1, 32), fq.FQ_ROUND_STOCHASTIC, 0, fq.FQ_OK),
    (fq.FQ_MX, fq.FQ_E2M1, (1, 32), fq.FQ_ROUND_STOCHASTIC, 0, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_NVFP4, fq.FQ_E2M1, (1, 16), 2, 0, fq.FQ_E_INVALID),
    (fq.FQ_NVFP4, fq.FQ_E2M1, (1, 16), -1, 0, fq.FQ_E_INVALID),
    (fq.FQ_NVFP4, fq.FQ_E2M1, (1, 16), 0, 7, fq.FQ_E_INVALID),
    (fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (1, 128), 0, fq.FQ_SCALE_POW2, fq.FQ_OK),
    (fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (128, 128), 0, fq.FQ_SCALE_POW2, fq.FQ_OK),
    (fq.FQ_MX, fq.FQ_E4M3, (1, 32), 0, fq.FQ_SCALE_POW2, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_NVFP4, fq.FQ_E2M1, (1, 16), 0, fq.FQ_SCALE_POW2, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_PER_TENSOR_CURRENT, fq.FQ_E4M3, (0, 0), 0, fq.FQ_SCALE_POW2, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_MX, fq.FQ_E5M2, (1, 32), 0, 0, fq.FQ_OK),
    (fq.FQ_MX, fq.FQ_E2M1, (1, 32), 0, 0, fq.FQ_OK),
])
def test_rounding_and_scale_mode_validation(L, recipe, fmt, block, rounding, scale_mode, want):
    d = fq.desc(recipe, fq.FQ_IN_BF16, fmt, 256, 256, block, 3, rounding=rounding, seed=1, offset=2,
                scale_mode=scale_mode)
    z = [ctypes.c_size_t() for _ in range(5)]
    assert L.fq_sizes(ctypes.byref(d), *[ctypes.byref(v) for v in z]) == want
    if want != fq.FQ_OK:
        q = fq.FqQuantized(fq.FqPlane(B, B), fq.FqPlane(B, B), B, B)
        assert L.fq_quantize(ctypes.byref(d), B, ctypes.byref(q), B, 1 << 20, None) == want
        assert L.fq_quantize_with_amax(ctypes.byref(d), B, B, ctypes.byref(q), B, 1 << 20, None) == want


def test_mx_variant_sizes():
    both = fq.FQ_ROWWISE | fq.FQ_COLWISE
    z = sizes(fq.FQ_MX, fq.FQ_E2M1, 8192, 8192, (1, 32), both)
    assert (z.row_data, z.row_scale, z.col_data, z.col_scale) == (8192 * 4096, 8192 * 256, 8192 * 4096, 8192 * 256)
    z = sizes(fq.FQ_MX, fq.FQ_E5M2, 64, 96, (1, 32), both)
    assert (z.row_data, z.row_scale, z.col_data, z.col_scale) == (64 * 96, 64 * 3, 64 * 96, 96 * 2)


def test_desc_layout():
    # the C struct: three int32, two int64, two int32, uint32, two int32, two uint64, int32, uint32
    assert ctypes.sizeof(fq.FqDesc) == 80
    assert fq.FqDesc.seed.offset == 56 and fq.FqDesc.offset.offset == 64
    assert fq.FqDesc.transform.offset == 72 and fq.FqDesc.rht_signs.offset == 76


@pytest.mark.parametrize("recipe,fmt,block,outputs,transform,want", [
    (fq.FQ_NVFP4, fq.FQ_E2M1, (1, 16), fq.FQ_COLWISE, fq.FQ_TRANSFORM_RHT16, fq.FQ_OK),
    (fq.FQ_NVFP4, fq.FQ_E2M1, (1, 16), fq.FQ_ROWWISE, fq.FQ_TRANSFORM_RHT16, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_NVFP4, fq.FQ_E2M1, (1, 16), 3, fq.FQ_TRANSFORM_RHT16, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_NVFP4, fq.FQ_E2M1, (16, 16), fq.FQ_COLWISE, fq.FQ_TRANSFORM_RHT16, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_MX, fq.FQ_E4M3, (1, 32), fq.FQ_COLWISE, fq.FQ_TRANSFORM_RHT16, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (1, 128), fq.FQ_COLWISE, fq.FQ_TRANSFORM_RHT16, fq.FQ_E_UNSUPPORTED),
    (fq.FQ_NVFP4, fq.FQ_E2M1, (1, 16), fq.FQ_COLWISE, 2, fq.FQ_E_INVALID),
])
def test_transform_validation(L, recipe, fmt, block, outputs, transform, want):
    d = fq.desc(recipe, fq.FQ_IN_BF16, fmt, 256, 256, block, outputs, transform=transform, rht_signs=0x1234)
    z = [ctypes.c_size_t() for _ in range(5)]
    assert L.fq_sizes(ctypes.byref(d), *[ctypes.byref(v) for v in z]) == want
    if want != fq.FQ_OK:
        q = fq.FqQuantized(fq.FqPlane(B, B), fq.FqPlane(B, B), B, B)
        assert L.fq_quantize(ctypes.byref(d), B, ctypes.byref(q), B, 1 << 20, None) == want
        assert L.fq_amax(ctypes.byref(d), B, B, B, 1 << 20, None) == want


def test_null_desc(L):
    assert L.fq_sizes(None, None, None, None, None, None) == fq.FQ_E_INVALID
    assert L.fq_quantize(None, B, None, B, 4096, None) == fq.FQ_E_INVALID


def test_pointer_checks(L):
    d = fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_BF16, fq.FQ_E4M3, 64, 64)
    ok = fq.FqQuantized(fq.FqPlane(B, None), fq.FqPlane(None, None), B, None)
    # misaligned input, output plane, scalar output
    assert L.fq_quantize(ctypes.byref(d), B + 8, ctypes.byref(ok), B, 4096, None) == fq.FQ_E_ALIGN
    bad = fq.FqQuantized(fq.FqPlane(B + 4, None), fq.FqPlane(None, None), B, None)
    assert L.fq_quantize(ctypes.byref(d), B, ctypes.byref(bad), B, 4096, None) == fq.FQ_E_ALIGN
    bad = fq.FqQuantized(fq.FqPlane(B, None), fq.FqPlane(None, None), B + 2, None)
    assert L.fq_quantize(ctypes.byref(d), B, ctypes.byref(bad), B, 4096, None) == fq.FQ_E_ALIGN
    # missing pieces
    assert L.fq_quantize(ctypes.byref(d), None, ctypes.byref(ok), B, 4096, None) == fq.FQ_E_INVALID
    nodata = fq.FqQuantized(fq.FqPlane(None, None), fq.FqPlane(None, None), B, None)
    assert L.fq_quantize(ctypes.byref(d), B, ctypes.byref(nodata), B, 4096, None) == fq.FQ_E_INVALID
    noscale = fq.FqQuantized(fq.FqPlane(B, None), fq.FqPlane(None, None), None, None)
    assert L.fq_quantize(ctypes.byref(d), B, ctypes.byref(noscale), B, 4096, None) == fq.FQ_E_INVALID
    # workspace
    assert L.fq_quantize(ctypes.byref(d), B, ctypes.byref(ok), None, 4096, None) == fq.FQ_E_WORKSPACE
    assert L.fq_quantize(ctypes.byref(d), B, ctypes.byref(ok), B, 4095, None) == fq.FQ_E_WORKSPACE
    # block recipes need their scale planes
    db = fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, 128, 128, (1, 128))
    assert L.fq_quantize(ctypes.byref(db), B, ctypes.byref(ok), None, 0, None) == fq.FQ_E_INVALID
    # delayed has its own entry point
    dd = fq.desc(fq.FQ_PER_TENSOR_DELAYED, fq.FQ_IN_BF16, fq.FQ_E4M3, 64, 64)
    assert L.fq_quantize(ctypes.byref(dd), B, ctypes.byref(ok), B, 4096, None) == fq.FQ_E_UNSUPPORTED


def test_delayed_and_amax_checks(L):
    d = fq.desc(fq.FQ_PER_TENSOR_DELAYED, fq.FQ_IN_BF16, fq.FQ_E4M3, 64, 64)
    ok = fq.FqQuantized(fq.FqPlane(B, None), fq.FqPlane(None, None), None, None)
    call = lambda st, ws=None, n=0: L.fq_quantize_delayed(ctypes.byref(d), B, ctypes.byref(st), ctypes.byref(ok),
                                                          ws, n, None)
    assert call(fq.FqDelayedState(B, 0, B, B, B, 0)) == fq.FQ_E_INVALID            # empty window
    assert call(fq.FqDelayedState(B, 1024, B, B, B, -1)) == fq.FQ_E_INVALID        # negative step
    assert call(fq.FqDelayedState(B, 1024, B + 2, B, B, 0)) == fq.FQ_E_ALIGN       # scale
    assert call(fq.FqDelayedState(B, 1024, B, B, None, 0)) == fq.FQ_E_INVALID      # no pending records
    assert call(fq.FqDelayedState(B, 1024, B, B, B + 4, 0)) == fq.FQ_E_ALIGN       # pending 16-byte aligned
    st = fq.FqDelayedState(B, 1024, B, B, B, 0)
    # fq_delayed_flush checks the same state and the recipe
    assert L.fq_delayed_flush(ctypes.byref(d), ctypes.byref(fq.FqDelayedState(B, 1024, B, B, None, 3)),
                              None) == fq.FQ_E_INVALID
    assert L.fq_delayed_flush(ctypes.byref(d), ctypes.byref(fq.FqDelayedState(B, 1024, B, B, B + 8, 3)),
                              None) == fq.FQ_E_ALIGN
    assert L.fq_delayed_flush(ctypes.byref(d), ctypes.byref(st), None) == fq.FQ_OK  # step 0: nothing to do
    dcur = fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_BF16, fq.FQ_E4M3, 64, 64)
    assert L.fq_delayed_flush(ctypes.byref(dcur), ctypes.byref(st), None) == fq.FQ_E_UNSUPPORTED
    assert fq.fq_sizes(d).workspace == 4096 and ctypes.sizeof(fq.FqDelayedState) == 48
    dc = fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_BF16, fq.FQ_E4M3, 64, 64)
    assert L.fq_quantize_delayed(ctypes.byref(dc), B, ctypes.byref(st), ctypes.byref(ok), B, 4096, None) \
        == fq.FQ_E_UNSUPPORTED
    assert L.fq_amax(ctypes.byref(dc), B, None, B, 4096, None) == fq.FQ_E_INVALID
    assert L.fq_amax(ctypes.byref(dc), B, B + 1, B, 4096, None) == fq.FQ_E_ALIGN
    assert L.fq_amax(ctypes.byref(dc), B, B, B, 100, None) == fq.FQ_E_WORKSPACE
    # fq_amax takes any desc; the workspace fq_sizes reports for it is enough
    for dx in (fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, 128, 128, (1, 128)),
               fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, 64, 64, (1, 32))):
        need = fq.fq_sizes(dx).workspace
        assert need == 4096
        assert L.fq_amax(ctypes.byref(dx), B, B, B, need - 1, None) == fq.FQ_E_WORKSPACE
        assert L.fq_amax(ctypes.byref(dx), B, B, None, need, None) == fq.FQ_E_WORKSPACE
    db = fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, 128, 128, (1, 128))
    assert L.fq_quantize_with_amax(ctypes.byref(db), B, B, ctypes.byref(ok), None, 0, None) == fq.FQ_E_UNSUPPORTED
    assert L.fq_quantize_with_amax(ctypes.byref(dc), B, None, ctypes.byref(ok), None, 0, None) == fq.FQ_E_INVALID


def test_dequantize_checks(L):
    d = fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, 64, 64, (1, 32), fq.FQ_ROWWISE)
    q = fq.FqQuantized(fq.FqPlane(B, B), fq.FqPlane(None, None), None, None)
    assert L.fq_dequantize(ctypes.byref(d), ctypes.byref(q), 3, B, 0, None) == fq.FQ_E_INVALID
    assert L.fq_dequantize(ctypes.byref(d), ctypes.byref(q), fq.FQ_COLWISE, B, 0, None) == fq.FQ_E_INVALID
    assert L.fq_dequantize(ctypes.byref(d), ctypes.byref(q), fq.FQ_ROWWISE, None, 0, None) == fq.FQ_E_INVALID
    assert L.fq_dequantize(ctypes.byref(d), ctypes.byref(q), fq.FQ_ROWWISE, B + 4, 0, None) == fq.FQ_E_ALIGN
    assert L.fq_dequantize(ctypes.byref(d), ctypes.byref(q), fq.FQ_ROWWISE, B, 2, None) == fq.FQ_E_INVALID


def test_requantize_checks(L):
    ok = fq.FqQuantized(fq.FqPlane(B, B), fq.FqPlane(B, B), None, None)
    d = fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, 64, 64, (1, 32), fq.FQ_ROWWISE)
    assert L.fq_requantize_transpose(None, ctypes.byref(ok), ctypes.byref(ok), None) == fq.FQ_E_INVALID
    assert L.fq_requantize_transpose(ctypes.byref(d), None, ctypes.byref(ok), None) == fq.FQ_E_INVALID
    for bad in (fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, 128, 128, (1, 128)),
                fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, 64, 64, (1, 16)),
                fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E5M2, 64, 64, (1, 32))):
        assert L.fq_requantize_transpose(ctypes.byref(bad), ctypes.byref(ok), ctypes.byref(ok), None) \
            == fq.FQ_E_UNSUPPORTED
    d48 = fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, 48, 64, (1, 32), fq.FQ_ROWWISE)
    assert L.fq_requantize_transpose(ctypes.byref(d48), ctypes.byref(ok), ctypes.byref(ok), None) == fq.FQ_E_SHAPE
    mis = fq.FqQuantized(fq.FqPlane(B, B + 1), fq.FqPlane(B, B), None, None)
    assert L.fq_requantize_transpose(ctypes.byref(d), ctypes.byref(mis), ctypes.byref(ok), None) == fq.FQ_E_ALIGN
    sr = fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, 64, 64, (1, 32), fq.FQ_ROWWISE, rounding=1)
    assert L.fq_requantize_transpose(ctypes.byref(sr), ctypes.byref(ok), ctypes.byref(ok), None) \
        == fq.FQ_E_UNSUPPORTED
    for fmt in (fq.FQ_E5M2, fq.FQ_E2M1):
        v = fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fmt, 64, 64, (1, 32), fq.FQ_ROWWISE)
        assert L.fq_requantize_transpose(ctypes.byref(v), ctypes.byref(ok), ctypes.byref(ok), None) \
            == fq.FQ_E_UNSUPPORTED
    nocol = fq.FqQuantized(fq.FqPlane(B, B), fq.FqPlane(None, None), None, None)
    assert L.fq_requantize_transpose(ctypes.byref(d), ctypes.byref(ok), ctypes.byref(nocol), None) \
        == fq.FQ_E_INVALID


def test_requantize_checks_blockwise(L):
    """Blockwise requantization: 1x128 tiles with power-of-two scales only
    (the restored values are exact only then), 128-aligned shapes."""
    ok = fq.FqQuantized(fq.FqPlane(B, B), fq.FqPlane(B, B), None, None)
    pow2 = dict(scale_mode=fq.FQ_SCALE_POW2)
    for bad in (fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, 128, 128, (1, 128)),
                fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, 128, 128, (128, 128), **pow2),
                fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, 128, 128, (1, 128), rounding=1, **pow2),
                fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, 128, 128, (1, 32), **pow2)):
        assert L.fq_requantize_transpose(ctypes.byref(bad), ctypes.byref(ok), ctypes.byref(ok), None) \
            in (fq.FQ_E_UNSUPPORTED, fq.FQ_E_INVALID)
    for R, C in ((64, 128), (128, 96), (192, 128)):
        d = fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 128), **pow2)
        assert L.fq_requantize_transpose(ctypes.byref(d), ctypes.byref(ok), ctypes.byref(ok), None) \
            == fq.FQ_E_SHAPE
    d = fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, 256, 128, (1, 128), **pow2)
    mis = fq.FqQuantized(fq.FqPlane(B, B + 4), fq.FqPlane(B, B), None, None)
    assert L.fq_requantize_transpose(ctypes.byref(d), ctypes.byref(mis), ctypes.byref(ok), None) == fq.FQ_E_ALIGN
    nocol = fq.FqQuantized(fq.FqPlane(B, B), fq.FqPlane(B, None), None, None)
    assert L.fq_requantize_transpose(ctypes.byref(d), ctypes.byref(ok), ctypes.byref(nocol), None) \
        == fq.FQ_E_INVALID
    empty = fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, 0, 128, (1, 128), **pow2)
    assert L.fq_requantize_transpose(ctypes.byref(empty), ctypes.byref(ok), ctypes.byref(ok), None) == fq.FQ_OK
