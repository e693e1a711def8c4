"""GPU parity over a seeded sweep: every recipe, format, plane selection,
rounding (stochastic rounding of FP4 and FP8 elements included), transform
and input dtype, at random shapes (whole 128x128 tiles,
which take the one-read tile kernels for bf16, and ragged multiples of each
recipe's block), with random value scales and distributions; each case
compared byte for byte with the oracle. The cases are drawn once from a
fixed seed, and each case's id names everything needed to repeat it."""
import os

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
PLANES = {ROW: "row", COL: "col", BOTH: "both"}

# kind -> (recipe, format, block, rows multiple without / with the colwise
# plane, cols multiple, plane selections allowed)
KINDS = {
    "current_e4m3": (fq.FQ_PER_TENSOR_CURRENT, fq.FQ_E4M3, (0, 0), 1, 1, 1, (ROW, COL, BOTH)),
    "current_e5m2": (fq.FQ_PER_TENSOR_CURRENT, fq.FQ_E5M2, (0, 0), 1, 1, 1, (ROW, COL, BOTH)),
    "delayed_e4m3": (fq.FQ_PER_TENSOR_DELAYED, fq.FQ_E4M3, (0, 0), 1, 1, 1, (ROW, COL, BOTH)),
    "block_1x128": (fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (1, 128), 1, 128, 128, (ROW, COL, BOTH)),
    "block_1x128_pow2": (fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (1, 128), 1, 128, 128, (ROW, COL, BOTH)),
    "block_128x128": (fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (128, 128), 128, 128, 128, (ROW, BOTH)),
    "block_128x128_pow2": (fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (128, 128), 128, 128, 128, (ROW, BOTH)),
    "mx_e4m3": (fq.FQ_MX, fq.FQ_E4M3, (1, 32), 1, 32, 32, (ROW, COL, BOTH)),
    "mx_e5m2": (fq.FQ_MX, fq.FQ_E5M2, (1, 32), 1, 32, 32, (ROW, COL, BOTH)),
    "mx_e2m1": (fq.FQ_MX, fq.FQ_E2M1, (1, 32), 1, 32, 32, (ROW, COL, BOTH)),
    "nvfp4_1x16": (fq.FQ_NVFP4, fq.FQ_E2M1, (1, 16), 1, 16, 16, (ROW, COL, BOTH)),
    "nvfp4_16x16": (fq.FQ_NVFP4, fq.FQ_E2M1, (16, 16), 16, 16, 16, (ROW, COL, BOTH)),
    "nvfp4_1x16_sr": (fq.FQ_NVFP4, fq.FQ_E2M1, (1, 16), 1, 16, 16, (ROW, COL, BOTH)),
    "nvfp4_1x16_rht": (fq.FQ_NVFP4, fq.FQ_E2M1, (1, 16), 16, 16, 16, (COL,)),
    "nvfp4_1x16_rht_sr": (fq.FQ_NVFP4, fq.FQ_E2M1, (1, 16), 16, 16, 16, (COL,)),
    "current_e4m3_sr": (fq.FQ_PER_TENSOR_CURRENT, fq.FQ_E4M3, (0, 0), 1, 1, 1, (ROW, COL, BOTH)),
    "current_e5m2_sr": (fq.FQ_PER_TENSOR_CURRENT, fq.FQ_E5M2, (0, 0), 1, 1, 1, (ROW, COL, BOTH)),
    "block_1x128_sr": (fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (1, 128), 1, 128, 128, (ROW, COL, BOTH)),
    "block_1x128_pow2_sr": (fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (1, 128), 1, 128, 128, (ROW, COL, BOTH)),
    "mx_e4m3_sr": (fq.FQ_MX, fq.FQ_E4M3, (1, 32), 1, 32, 32, (ROW, COL, BOTH)),
    "mx_e5m2_sr": (fq.FQ_MX, fq.FQ_E5M2, (1, 32), 1, 32, 32, (ROW, COL, BOTH)),
}
OFMT = {fq.FQ_E4M3: orc.E4M3, fq.FQ_E5M2: orc.E5M2, fq.FQ_E2M1: orc.E2M1}
# FQ_SWEEP_CASES / FQ_SWEEP_SEED draw a larger or another sweep
N_CASES = int(os.environ.get("FQ_SWEEP_CASES", "600"))
SEED = int(os.environ.get("FQ_SWEEP_SEED", "20261203"))


def draw_cases(n, seed=SEED):
    rng = np.random.default_rng(seed)
    names = sorted(KINDS)
    cases = []
    for i in range(n):
        kind = names[i % len(names)]
        _, _, _, rg_row, rg_col, cg, planes = KINDS[kind]
        outputs = planes[rng.integers(len(planes))]
        rg = rg_col if outputs & COL else rg_row
        dt = W.BF16 if rng.random() < 0.6 else W.F32
        if rng.random() < 0.5:   # whole 128x128 tiles
            R, C = 128 * int(rng.integers(1, 5)), 128 * int(rng.integers(1, 9))
        else:
            R = rg * int(rng.integers(1, max(2, 520 // rg)))
            C = cg * int(rng.integers(1, max(2, 1100 // cg)))
        dist = ("normal", "student_t", "wide")[rng.integers(3)]
        cases.append(dict(kind=kind, outputs=outputs, dt=dt, R=R, C=C, dist=dist,
                          scale=float(10.0 ** rng.uniform(-4, 4)), seed=int(rng.integers(1 << 30)),
                          given_amax=bool(rng.random() < 0.25), sr=(int(rng.integers(1 << 62)), int(rng.integers(1 << 40))),
                          signs=int(rng.integers(1 << 16))))
    return cases


CASES = draw_cases(N_CASES)


def uses_given_amax(c):
    """The case passes 1.5x its amax to fq_quantize_with_amax (per-tensor
    current scaling and NVFP4 without the transform)."""
    recipe = KINDS[c["kind"]][0]
    return c["given_amax"] and recipe in (fq.FQ_PER_TENSOR_CURRENT, fq.FQ_NVFP4) and "_rht" not in c["kind"]


def case_id(c):
    return (f"{c['kind']}-{PLANES[c['outputs']]}-{c['dt']}-{c['R']}x{c['C']}-{c['dist']}"
            f"-s{c['seed']}{'-amax' if uses_given_amax(c) else ''}")


def make_input(c):
    shape = (c["R"], c["C"])
    if c["dist"] == "wide":
        x = W.uniform_bits_bf16(shape, c["seed"], max_abs=1e6)
        return x if c["dt"] == W.BF16 else W.bf16_bits_to_f32(x)
    if c["dist"] == "student_t":
        x = W.student_t(shape, 3.0, c["seed"], W.F32)
    else:
        x = W.normal(shape, 1.0, c["seed"], W.F32)
    x = (x * np.float32(c["scale"])).astype(np.float32)
    return W.to_bf16_bits(x) if c["dt"] == W.BF16 else x


def host_amax(x):
    f = W.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x
    return float(np.abs(f).max()) if f.size else 0.0


def compare_planes(out, outputs, pairs, tag):
    """pairs: plane -> [(gpu tensor, oracle array, name)]"""
    for plane in (ROW, COL):
        if outputs & plane:
            for got, want, name in pairs[plane]:
                same_bytes(host(got), want, f"{tag}: {name}")


@pytest.mark.parametrize("c", CASES, ids=case_id)
def test_sweep(c):
    recipe, fmt, block, _, _, _, _ = KINDS[c["kind"]]
    x = make_input(c)
    R, C = x.shape
    outputs = c["outputs"]
    tag = case_id(c)
    sr = "_sr" in c["kind"]
    rht = "_rht" in c["kind"]
    pow2 = "_pow2" in c["kind"]
    d = fq.desc(recipe, in_dtype(x), fmt, R, C, block, outputs,
                rounding=fq.FQ_ROUND_STOCHASTIC if sr else fq.FQ_ROUND_NEAREST_EVEN,
                seed=c["sr"][0] if sr else 0, offset=c["sr"][1] if sr else 0,
                scale_mode=fq.FQ_SCALE_POW2 if pow2 else fq.FQ_SCALE_DEFAULT,
                transform=fq.FQ_TRANSFORM_RHT16 if rht else fq.FQ_TRANSFORM_NONE,
                rht_signs=c["signs"] if rht else 0)
    out = fq.alloc_quantized(d)
    xd = dev(x)

    if recipe == fq.FQ_PER_TENSOR_DELAYED:
        # three steps on a window of two, the last one checked after a flush
        st, ost = fq.DelayedState(2), orc.DelayedState(2)
        xs = [x, make_input(dict(c, seed=c["seed"] + 1)), x]
        for t, xt in enumerate(xs):
            s_before = ost.s
            fq.fq_quantize_delayed(d, dev(xt), st, out)
            want = orc.quantize_delayed(xt, OFMT[fmt], ost, outputs=outputs)
        fq.fq_delayed_flush(d, st)
        torch.cuda.synchronize()
        compare_planes(out, outputs, {ROW: [(out.row_data, want["q_row"], "codes")],
                                      COL: [(out.col_data, want["q_col"], "colwise codes")]}, tag)
        same_bytes(host(out.tensor_scale), f32(s_before), f"{tag}: s used")
        same_bytes(host(st.amax_history), ost.hist, f"{tag}: window")
        same_bytes(host(st.scale_inv), f32(ost.s), f"{tag}: next s")
        return

    ws = fq.alloc_workspace(d)
    amax_in = None
    if uses_given_amax(c):
        amax_in = np.float32(host_amax(x) * 1.5 + 1e-30)
        fq.fq_quantize_with_amax(d, xd, torch.tensor([amax_in], dtype=torch.float32, device="cuda"), out, ws)
    else:
        fq.fq_quantize(d, xd, out, ws)
    torch.cuda.synchronize()

    if recipe == fq.FQ_PER_TENSOR_CURRENT:
        srp = c["sr"] if sr else None
        if amax_in is None:
            want = orc.quantize_current(x, OFMT[fmt], outputs=outputs, sr=srp)
            same_bytes(host(out.amax), f32(want["amax"]), f"{tag}: amax")
        else:
            want = orc.quantize_with_amax(x, OFMT[fmt], amax_in, outputs=outputs, sr=srp)
        compare_planes(out, outputs, {ROW: [(out.row_data, want["q_row"], "codes")],
                                      COL: [(out.col_data, want["q_col"], "colwise codes")]}, tag)
        same_bytes(host(out.tensor_scale), f32(want["s"]), f"{tag}: s")
    elif recipe == fq.FQ_BLOCK_FP32:
        want = orc.quantize_block(x, block, outputs=outputs, pow2=pow2, sr=c["sr"] if sr else None)
        compare_planes(out, outputs, {ROW: [(out.row_data, want["q_row"], "codes"),
                                            (out.row_scale, want["s_row"], "tile scales")],
                                      COL: [(out.col_data, want["q_col"], "colwise codes"),
                                            (out.col_scale, want["s_col"], "colwise tile scales")]}, tag)
    elif recipe == fq.FQ_MX:
        want = orc.quantize_mx(x, outputs=outputs, fmt=OFMT[fmt], sr=c["sr"] if sr else None)
        compare_planes(out, outputs, {ROW: [(out.row_data, want["q_row"], "codes"),
                                            (out.row_scale, want["e_row"], "E8M0")],
                                      COL: [(out.col_data, want["q_col"], "colwise codes"),
                                            (out.col_scale, want["e_col"], "colwise E8M0")]}, tag)
    elif rht:
        want = orc.quantize_nvfp4_rht(x, c["signs"], sr=c["sr"] if sr else None)
        compare_planes(out, outputs, {COL: [(out.col_data, want["p_col"], "RHT packed FP4"),
                                            (out.col_scale, want["c_col"], "RHT block scales")]}, tag)
        same_bytes(host(out.tensor_scale), f32(want["S"]), f"{tag}: S")
        same_bytes(host(out.amax), f32(want["amax"]), f"{tag}: amax of the transformed tensor")
    else:
        want = orc.quantize_nvfp4(x, block, outputs=outputs, amax=amax_in, sr=c["sr"] if sr else None)
        compare_planes(out, outputs, {ROW: [(out.row_data, want["p_row"], "packed FP4"),
                                            (out.row_scale, want["c_row"], "block scales")],
                                      COL: [(out.col_data, want["p_col"], "colwise packed FP4"),
                                            (out.col_scale, want["c_col"], "colwise block scales")]}, tag)
        same_bytes(host(out.tensor_scale), f32(want["S"]), f"{tag}: S")
