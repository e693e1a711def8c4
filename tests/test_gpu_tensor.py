"""GPU parity: per-tensor current and delayed scaling against the oracle.

Bit-exact: every code byte and every fp32 scale/amax bit must equal the
oracle's on the same seeded input.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from conftest import golden
from fp8_fp4_tensor_amd import fq
from fp8_fp4_tensor_amd import workloads as W
from gpu_util import dev, f32, host, in_dtype, same_bytes, shape2

pytestmark = pytest.mark.gpu

FMTS = {fq.FQ_E4M3: orc.E4M3, fq.FQ_E5M2: orc.E5M2}


def run_current(x: np.ndarray, fmt: int, outputs=fq.FQ_ROWWISE):
    R, C = shape2(x)
    d = fq.desc(fq.FQ_PER_TENSOR_CURRENT, in_dtype(x), fmt, R, C, outputs=outputs)
    out = fq.alloc_quantized(d)
    ws = fq.alloc_workspace(d)
    xd = dev(x)
    fq.fq_quantize(d, xd, out, ws)
    torch.cuda.synchronize()
    return out


def check_current(x: np.ndarray, fmt: int, outputs=fq.FQ_ROWWISE):
    R, C = shape2(x)
    out = run_current(x, fmt, outputs)
    want = orc.quantize_current(x.reshape(-1), FMTS[fmt], outputs=outputs, shape=(R, C))
    if outputs & fq.FQ_ROWWISE:
        same_bytes(host(out.row_data), want["q_row"], "rowwise codes")
    if outputs & fq.FQ_COLWISE:
        same_bytes(host(out.col_data), want["q_col"], "colwise codes")
    same_bytes(host(out.tensor_scale), f32(want["s"]), "s")
    same_bytes(host(out.amax), f32(want["amax"]), "amax")
    return out


def test_worked_example():
    g = golden("cs_worked_example.json")
    out = check_current(np.array(g["x"], np.float32), fq.FQ_E4M3)
    assert list(host(out.row_data).ravel()) == [0xFE, 0x63, 0x7E]
    assert host(out.tensor_scale)[0] == np.float32(1000.0) / np.float32(448.0)


def test_all_zero_tensor():
    out = check_current(np.zeros(1 << 20, np.float32), fq.FQ_E4M3)
    assert host(out.tensor_scale)[0] == 1.0 and not host(out.row_data).any()


@pytest.mark.parametrize("fmt", [fq.FQ_E4M3, fq.FQ_E5M2])
def test_small_outlier_workload(fmt):
    check_current(W.SMALL_CURRENT.make().reshape(-1), fmt)


@pytest.mark.parametrize("shape", [(1, 1), (3, 7), (17, 33), (1000, 1000), (1, 4097), (513, 1)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", [fq.FQ_E4M3, fq.FQ_E5M2])
def test_ragged_shapes(shape, dt, fmt):
    seed = shape[0] * 7919 + shape[1]
    x = W.normal(shape, 3.0 if fmt == fq.FQ_E4M3 else 1e-2, seed, W.BF16 if dt == "bf16" else W.F32)
    check_current(x, fmt)


@pytest.mark.parametrize("shape,dt", [((2048, 1000), "bf16"), ((1024, 1025), "f32"), ((1024, 1025), "bf16"),
                                      ((1023, 1025), "bf16"), ((4100, 10000), "bf16"), ((4096, 4096), "f32")])
@pytest.mark.parametrize("fmt", [fq.FQ_E4M3, fq.FQ_E5M2])
def test_mid_and_large_sizes(shape, dt, fmt):
    """Multi-megabyte tensors, with and without a ragged tail of elements
    beyond the last whole 16-byte load of a wave."""
    x = W.normal(shape, 2.0, shape[0] + shape[1], W.BF16 if dt == "bf16" else W.F32)
    check_current(x, fmt)


@pytest.mark.parametrize("shape", [(65, 130), (64, 64), (1, 300), (200, 3)])
@pytest.mark.parametrize("fmt", [fq.FQ_E4M3, fq.FQ_E5M2])
def test_colwise_transpose(shape, fmt):
    x = W.normal(shape, 1.0, 11 + shape[0], W.BF16)
    check_current(x, fmt, outputs=fq.FQ_ROWWISE | fq.FQ_COLWISE)
    check_current(W.normal(shape, 1.0, 12, W.F32), fmt, outputs=fq.FQ_COLWISE)


@pytest.mark.parametrize("shape", [(16, 16), (128, 128), (144, 272), (256, 384), (1040, 96), (32, 2064)])
@pytest.mark.parametrize("fmt", [fq.FQ_E4M3, fq.FQ_E5M2])
def test_colwise_tiles(shape, fmt):
    """Shapes with R % 16 == 0 and C % 16 == 0 take the vector tile path (edge
    tiles of 16 rows or columns included)."""
    x = W.normal(shape, 1.0, 31 + shape[1], W.BF16)
    check_current(x, fmt, outputs=fq.FQ_ROWWISE | fq.FQ_COLWISE)
    check_current(W.normal(shape, 2.0, 32, W.F32), fmt, outputs=fq.FQ_COLWISE)


def test_full_size_current_both_planes():
    w = W.BY_NAME["current_e4m3_act_8192x4096"]
    check_current(w.make(), fq.FQ_E4M3, outputs=fq.FQ_ROWWISE | fq.FQ_COLWISE)


def all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    return b[np.isfinite(f)]


@pytest.mark.parametrize("fmt", [fq.FQ_E4M3, fq.FQ_E5M2])
@pytest.mark.parametrize("amax", [448.0, 1000.0, 3.0, 1e-3, 57344.0, 2.0 ** -20, 1e30, 0.0])
def test_all_bf16_patterns_with_amax(fmt, amax):
    """Every finite bf16 value through the cast at a given amax (values above
    it saturate), through fq_quantize_with_amax."""
    x = all_finite_bf16()
    d = fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_BF16, fmt, 1, x.size)
    out = fq.alloc_quantized(d)
    a_dev = torch.tensor([amax], dtype=torch.float32, device="cuda")
    fq.fq_quantize_with_amax(d, dev(x), a_dev, out)
    torch.cuda.synchronize()
    want = orc.quantize_with_amax(x, FMTS[fmt], np.float32(amax))
    same_bytes(host(out.row_data), want["q_row"], f"codes at amax {amax}")
    same_bytes(host(out.tensor_scale), f32(want["s"]), "s")


@pytest.mark.parametrize("fmt", [fq.FQ_E4M3, fq.FQ_E5M2])
def test_random_fp32_bit_patterns(fmt):
    rng = np.random.default_rng(99)
    bits = rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = np.where(np.isfinite(x), x, np.float32(0)).astype(np.float32)
    d = fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_F32, fmt, 1, x.size)
    out = fq.alloc_quantized(d)
    for amax in (1.0, 3.0e38, 1e-30):
        a_dev = torch.tensor([amax], dtype=torch.float32, device="cuda")
        fq.fq_quantize_with_amax(d, dev(x), a_dev, out)
        torch.cuda.synchronize()
        want = orc.quantize_with_amax(x, FMTS[fmt], np.float32(amax))
        same_bytes(host(out.row_data), want["q_row"], f"codes at amax {amax}")


@pytest.mark.parametrize("recipe,fmt,block", [(fq.FQ_BLOCK_FP32, fq.FQ_E4M3, (1, 128)),
                                               (fq.FQ_MX, fq.FQ_E4M3, (1, 32)),
                                               (fq.FQ_NVFP4, fq.FQ_E2M1, (16, 16))])
def test_fq_amax_any_desc_with_reported_workspace(recipe, fmt, block):
    """fq_amax accepts any desc; the workspace fq_sizes reports for that desc
    is enough, and the amax equals the oracle's."""
    x = W.normal((256, 384), 1.0, 91, W.BF16)
    d = fq.desc(recipe, fq.FQ_IN_BF16, fmt, 256, 384, block)
    ws = torch.empty(fq.fq_sizes(d).workspace, dtype=torch.uint8, device="cuda")
    a = torch.empty(1, dtype=torch.float32, device="cuda")
    fq.fq_amax(d, dev(x), a, ws)
    torch.cuda.synchronize()
    same_bytes(host(a), f32(orc.amax(x)), "fq_amax")


def test_sharded_amax_allgather_example():
    """Shards quantized with the max of their amaxes equal the whole tensor
    quantized at once (fq_amax, a max across shards, fq_quantize_with_amax)."""
    g = golden("cs_allgather_example.json")
    shards = [np.array(s, np.float32) for s in g["shards"]]
    amaxes = []
    for s in shards:
        d = fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_F32, fq.FQ_E4M3, 1, s.size)
        a = torch.empty(1, dtype=torch.float32, device="cuda")
        fq.fq_amax(d, dev(s), a, fq.alloc_workspace(d))
        amaxes.append(a)
    torch.cuda.synchronize()
    assert [host(a)[0] for a in amaxes] == g["local_amax"]
    glob = torch.maximum(amaxes[0], amaxes[1])
    codes = []
    for s in shards:
        d = fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_F32, fq.FQ_E4M3, 1, s.size)
        out = fq.alloc_quantized(d)
        fq.fq_quantize_with_amax(d, dev(s), glob, out)
        torch.cuda.synchronize()
        codes.append(host(out.row_data).ravel())
    whole = orc.quantize_current(np.concatenate(shards), orc.E4M3)
    same_bytes(np.concatenate(codes), whole["q_row"], "sharded codes")


@pytest.mark.parametrize("shape", [(0, 0), (0, 128), (5, 0)])
def test_empty_tensor(shape):
    x = np.zeros(shape, np.float32)
    d = fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_F32, fq.FQ_E4M3, shape[0], shape[1])
    out = fq.alloc_quantized(d)
    ws = fq.alloc_workspace(d)
    xd = torch.empty(16, dtype=torch.float32, device="cuda")
    fq.fq_quantize(d, xd, out, ws)
    torch.cuda.synchronize()
    assert host(out.tensor_scale)[0] == 1.0 and host(out.amax)[0] == 0.0


@pytest.mark.parametrize("w", [w for w in W.LARGE if w.recipe == "current"], ids=lambda w: w.name)
def test_full_size_current(w):
    x = w.make()
    fmt = fq.FQ_E4M3 if w.fmt == "e4m3" else fq.FQ_E5M2
    out1 = check_current(x, fmt)
    # determinism: a second run gives identical bytes
    out2 = run_current(x, fmt)
    assert torch.equal(out1.row_data, out2.row_data) and torch.equal(out1.tensor_scale, out2.tensor_scale)


# ---------------------------------------------------------------- delayed
def check_state(st, ost, what):
    same_bytes(host(st.amax_history), ost.hist, f"{what} history")
    same_bytes(host(st.scale), f32(ost.alpha), f"{what} alpha")
    same_bytes(host(st.scale_inv), f32(ost.s), f"{what} s")


def delayed_steps(xs, fmt, H, outputs=fq.FQ_ROWWISE, check_every=1):
    """Steps on the GPU and in the oracle; at checked steps the codes, the s
    used, a_t, and (after fq_delayed_flush) the window and scales. Between
    checks the window update of each step runs inside the next step's cast."""
    R, C = shape2(xs[0])
    d = fq.desc(fq.FQ_PER_TENSOR_DELAYED, in_dtype(xs[0]), fmt, R, C, outputs=outputs)
    out = fq.alloc_quantized(d)
    st = fq.DelayedState(H)
    ost = orc.DelayedState(H)
    for t, x in enumerate(xs):
        s_before = ost.s
        fq.fq_quantize_delayed(d, dev(x), st, out)
        want = orc.quantize_delayed(x.reshape(-1), FMTS[fmt], ost, outputs=outputs, shape=(R, C))
        if t % check_every == 0 or t == len(xs) - 1:
            fq.fq_delayed_flush(d, st)
            torch.cuda.synchronize()
            if outputs & fq.FQ_ROWWISE:
                same_bytes(host(out.row_data), want["q_row"], f"step {t} codes")
            if outputs & fq.FQ_COLWISE:
                same_bytes(host(out.col_data), want["q_col"], f"step {t} colwise codes")
            same_bytes(host(out.tensor_scale), f32(s_before), f"step {t} s used")
            same_bytes(host(out.amax), f32(want["amax"]), f"step {t} amax")
            check_state(st, ost, f"step {t}")
    return st, ost


@pytest.mark.parametrize("fmt", [fq.FQ_E4M3, fq.FQ_E5M2])
def test_delayed_small_ring(fmt):
    rng = np.random.default_rng(4)
    xs = [(rng.standard_normal((37, 61)) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32) for _ in range(11)]
    delayed_steps(xs, fmt, 4)
    delayed_steps(xs, fmt, 4, check_every=5)
    delayed_steps([W.to_bf16_bits(x) for x in xs], fmt, 3, outputs=fq.FQ_ROWWISE | fq.FQ_COLWISE)
    delayed_steps(xs, fmt, 1, check_every=3)                       # a window of one step


def test_delayed_colwise_tiles():
    rng = np.random.default_rng(5)
    xs = [(rng.standard_normal((160, 272)) * 10.0 ** rng.uniform(-2, 2)).astype(np.float32) for _ in range(6)]
    delayed_steps([W.to_bf16_bits(x) for x in xs], fq.FQ_E4M3, 3, outputs=fq.FQ_ROWWISE | fq.FQ_COLWISE)
    delayed_steps(xs, fq.FQ_E5M2, 4, outputs=fq.FQ_COLWISE, check_every=4)


def test_delayed_window_wrap_1024():
    """1030 steps with an outlier at step 0: the window of 1024 wraps."""
    rng = np.random.default_rng(8)
    xs = [np.full((1, 16), 1000.0, np.float32)]
    xs += [(rng.standard_normal((1, 16)) * 2).astype(np.float32) for _ in range(1029)]
    st, ost = delayed_steps(xs, fq.FQ_E4M3, 1024, check_every=64)
    assert ost.alpha != orc.tensor_scales(1000.0, 448.0)[0]


def test_delayed_long_window_separate_finish():
    """A window longer than 1024 steps: each step's update runs as its own
    kernel in the same call, so the state is current after every call
    (checked here without a flush), and a flush changes nothing."""
    rng = np.random.default_rng(9)
    xs = [(rng.standard_normal((64, 96)) * 10.0 ** rng.uniform(-2, 2)).astype(np.float32) for _ in range(7)]
    H = 2048
    d = fq.desc(fq.FQ_PER_TENSOR_DELAYED, fq.FQ_IN_F32, fq.FQ_E5M2, 64, 96)
    out = fq.alloc_quantized(d)
    st, ost = fq.DelayedState(H), orc.DelayedState(H)
    for t, x in enumerate(xs):
        fq.fq_quantize_delayed(d, dev(x), st, out)
        want = orc.quantize_delayed(x, orc.E5M2, ost)
        torch.cuda.synchronize()
        same_bytes(host(out.row_data), want["q_row"], f"step {t} codes")
        check_state(st, ost, f"step {t} unflushed")
    fq.fq_delayed_flush(d, st)
    torch.cuda.synchronize()
    check_state(st, ost, "flushed")
    delayed_steps(xs, fq.FQ_E4M3, 1500, outputs=fq.FQ_ROWWISE | fq.FQ_COLWISE, check_every=3)


def test_delayed_state_lags_one_step_until_flushed():
    """Without a flush, the window and scales after the call for step t are
    those after step t-1 (step t's update runs in step t+1's cast); a flush
    brings them to step t, a second flush changes nothing, and the steps that
    follow are unaffected by the flushes."""
    rng = np.random.default_rng(10)
    xs = [W.to_bf16_bits((rng.standard_normal((128, 256)) * 3.0 ** t).astype(np.float32)) for t in range(6)]
    d = fq.desc(fq.FQ_PER_TENSOR_DELAYED, fq.FQ_IN_BF16, fq.FQ_E4M3, 128, 256)
    out = fq.alloc_quantized(d)
    out.amax = None                      # no amax output: the step is one kernel
    st, ost = fq.DelayedState(4), orc.DelayedState(4)
    prev = ost.copy()
    for t, x in enumerate(xs):
        fq.fq_quantize_delayed(d, dev(x), st, out)
        want = orc.quantize_delayed(x, orc.E4M3, ost)
        torch.cuda.synchronize()
        same_bytes(host(out.row_data), want["q_row"], f"step {t} codes")
        check_state(st, prev, f"step {t} before the flush")
        if t % 2:
            fq.fq_delayed_flush(d, st)
            fq.fq_delayed_flush(d, st)
            torch.cuda.synchronize()
            check_state(st, ost, f"step {t} after the flush")
        prev = ost.copy()


@pytest.mark.parametrize("flushed", [False, True], ids=["with-pending", "flushed"])
def test_delayed_checkpoint_resume(flushed):
    """Resume from a saved state: either everything including the pending
    records, or (after fq_delayed_flush) the window, scales and step with the
    pending records zero-filled."""
    rng = np.random.default_rng(6)
    xs = [W.to_bf16_bits((rng.standard_normal((64, 256)) * (t + 1)).astype(np.float32)) for t in range(12)]
    d = fq.desc(fq.FQ_PER_TENSOR_DELAYED, fq.FQ_IN_BF16, fq.FQ_E5M2, 64, 256)
    run = lambda st, x: (fq.fq_quantize_delayed(d, dev(x), st, out), host(out.row_data).copy())[1]
    out = fq.alloc_quantized(d)
    ref = fq.DelayedState(8)
    ref_bytes = [run(ref, x) for x in xs]
    a = fq.DelayedState(8)
    for x in xs[:5]:
        run(a, x)
    if flushed:
        fq.fq_delayed_flush(d, a)
    saved = a.state_dict()
    if flushed:
        del saved["pending"]
    b = fq.DelayedState(8)
    b.load_state_dict(saved)
    got = [run(b, x) for x in xs[5:]]
    for t, g in enumerate(got):
        assert np.array_equal(g, ref_bytes[5 + t])
    fq.fq_delayed_flush(d, b)
    fq.fq_delayed_flush(d, ref)
    torch.cuda.synchronize()
    assert torch.equal(b.amax_history, ref.amax_history) and torch.equal(b.scale, ref.scale)


def test_delayed_steps_in_a_graph():
    """One delayed step captured per parity (the step number selects the
    window slot and the record), replayed in order with new inputs copied in
    between, equals eager steps."""
    R, C = 256, 512
    d = fq.desc(fq.FQ_PER_TENSOR_DELAYED, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C)
    x = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    out = fq.alloc_quantized(d)
    out.amax = None
    st, ost = fq.DelayedState(4), orc.DelayedState(4)
    # steps 0 and 1 eagerly (warm-up), then steps 2 and 3 captured
    xs = [W.normal((R, C), 1.0 + t, 900 + t, W.BF16) for t in range(10)]
    for t in range(2):
        x.copy_(dev(xs[t]))
        fq.fq_quantize_delayed(d, x, st, out)
        orc.quantize_delayed(xs[t], orc.E4M3, ost)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graphs = []
    for t in (2, 3):
        g = torch.cuda.CUDAGraph()
        st.step = t
        with torch.cuda.graph(g, stream=s):
            fq.fq_quantize_delayed(d, x, st, out, advance=False)
        graphs.append(g)
    for t in range(2, 10):
        if t >= 4:
            st.step = t                   # slot t mod 4 and record t mod 2 repeat with period 4
        x.copy_(dev(xs[t]))
        torch.cuda.synchronize()
        if t % 4 in (2, 3):
            graphs[t % 2].replay()
        else:
            fq.fq_quantize_delayed(d, x, st, out, advance=False)
        want = orc.quantize_delayed(xs[t], orc.E4M3, ost)
        torch.cuda.synchronize()
        same_bytes(host(out.row_data), want["q_row"], f"step {t} codes")
    st.step = 10
    fq.fq_delayed_flush(d, st)
    torch.cuda.synchronize()
    check_state(st, ost, "after 10 steps")


@pytest.mark.parametrize("w", [w for w in W.LARGE if w.recipe == "delayed"], ids=lambda w: w.name)
def test_full_size_delayed(w):
    fmt = fq.FQ_E4M3 if w.fmt == "e4m3" else fq.FQ_E5M2
    xs = [w.make(w.seed + t) for t in range(3)]
    delayed_steps(xs, fmt, w.extra["history_len"])
