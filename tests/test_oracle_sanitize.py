"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

orc.c is built a second time with -fsanitize=address,undefined into a
temporary library, and a child Python process (the sanitizer runtime
preloaded) runs every oracle entry point through the package's own wrappers:
all recipes and planes, block shapes at the tile edges, all-zero,
huge and tiny values, delayed steps that wrap the window, stochastic
rounding, the transform, dequantization, requantization and the codecs. Any
out-of-bounds access, use after free, signed overflow, misaligned access or
other undefined behaviour ends the child with an error and fails the test.
The child never imports torch, so no other runtime is sanitized."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r'''
import sys
sys.path.insert(0, sys.argv[2])
import numpy as np
import oracle as orc
orc._LIB_PATH = sys.argv[1]
orc._load()
E4M3, E5M2, E2M1, BOTH = orc.E4M3, orc.E5M2, orc.E2M1, orc.ROWWISE | orc.COLWISE
rng = np.random.default_rng(5)

def f32(shape, lo=-12, hi=12):
    return (rng.standard_normal(shape) * np.exp2(rng.integers(lo, hi, shape))).astype(np.float32)

def bf16(shape):
    b = rng.integers(0, 1 << 16, shape, dtype=np.uint32).astype(np.uint16)
    return np.where((b & 0x7F80) == 0x7F80, b & 0x807F, b).astype(np.uint16)   # finite patterns only

inputs = [f32((256, 384)), bf16((256, 384)), np.zeros((256, 384), np.float32),
          np.full((256, 384), 3.0e38, np.float32), np.full((256, 384), 1.0e-40, np.float32)]
for x in inputs:
    for fmt in (E4M3, E5M2):
        r = orc.quantize_current(x, fmt, outputs=BOTH)
        orc.dequant_tensor(r["q_row"], fmt, r["s"])
        orc.quantize_with_amax(x, fmt, 1000.0, outputs=BOTH)
    st = orc.DelayedState(4)
    for t in range(6):
        orc.quantize_delayed(x * np.float32(0.5 ** t) if x.dtype == np.float32 else x, E4M3, st, outputs=BOTH)
    for block in ((1, 128), (128, 128)):
        for pow2 in (False, True):
            r = orc.quantize_block(x, block, outputs=BOTH, pow2=pow2)
            orc.dequant_block(r["q_row"], r["s_row"], block)
            orc.dequant_block(r["q_col"], r["s_col"], block)
            if pow2 and block == (1, 128):
                orc.requant_block_colwise(r["q_row"], r["s_row"])
    for fmt in (E4M3, E5M2, E2M1):
        r = orc.quantize_mx(x, outputs=BOTH, fmt=fmt)
        orc.dequant_mx(r["q_row"], r["e_row"], fmt)
        orc.dequant_mx(r["q_col"], r["e_col"], fmt)
        if fmt == E4M3:
            orc.requant_mx_colwise(r["q_row"], r["e_row"])
    for block in ((1, 16), (16, 16)):
        r = orc.quantize_nvfp4(x, block, outputs=BOTH)
        orc.quantize_nvfp4(x, block, outputs=BOTH, amax=7.0)
    orc.quantize_nvfp4(x, (1, 16), outputs=BOTH, sr=(11, 3))
    orc.quantize_nvfp4_rht(x, 0xA5C3)
    orc.quantize_nvfp4_rht(x, 0x0F0F, amax=50.0, sr=(2, 1))
# shapes at the minimum and with ragged per-tensor tails
for shape in ((1, 1), (3, 1001), (37, 61), (1, 128), (128, 128), (32, 32), (16, 16), (1, 16)):
    x = f32(shape)
    orc.quantize_current(x, E4M3, outputs=BOTH)
    if shape[1] % 128 == 0:
        orc.quantize_block(x, (1, 128), outputs=orc.ROWWISE)
    if shape[1] % 32 == 0:
        orc.quantize_mx(x, outputs=orc.ROWWISE)
    if shape[1] % 16 == 0:
        orc.quantize_nvfp4(x, (1, 16), outputs=orc.ROWWISE)
# codecs
y = f32((1 << 14,), -30, 30)
for fmt in (E4M3, E5M2, E2M1):
    orc.encode_array(fmt, y)
    for c in range(orc.max_code(fmt) + 1):
        orc.decode(fmt, c)
for c in range(256):
    orc.decode_e8m0(c)
orc.f32_to_bf16(y)
orc.philox4x32_10([1, 2, 3, 4], [5, 6])
orc.sr_bits(7, 8, 1, 12345)
orc.encode_e2m1_sr(2.7, 40000)
orc.rht16(f32((16,)), 0x1234)
print("sanitized oracle run: ok")
'''


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed to build the sanitized oracle")
def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    lib = str(tmp_path / "liborc_sanitized.so")
    build = [gcc, "-std=c99", "-O1", "-g", "-fPIC", "-shared", "-ffp-contract=off", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             os.path.join(ROOT, "oracle", "orc.c"), "-o", lib, "-lm"]
    r = subprocess.run(build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no AddressSanitizer runtime next to gcc")
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", SCRIPT, lib, ROOT], env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0 and "sanitized oracle run: ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
