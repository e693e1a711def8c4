"""Host logic of the benchmark and of the profile summaries (CPU only).

- The benchmark's algorithmic bytes per workload equal the passes over the
  input plus the output planes that the library itself sizes (fq_sizes, a
  host call), plus the stated scalars: two independent derivations of the
  figure that value and the roofline divide by.
- The counter summaries scale FETCH_SIZE / WRITE_SIZE by what a 256 MiB
  device copy reads, average per dispatch over counter instances, and record
  the hash of the kernel's sources that the benchmark checks before it
  reports traffic.
"""
import csv
import json

import pytest

import bench
from fp8_fp4_tensor_amd import fq, profsum
from fp8_fp4_tensor_amd import workloads as W

RECIPES = {"current": fq.FQ_PER_TENSOR_CURRENT, "delayed": fq.FQ_PER_TENSOR_DELAYED,
           "block": fq.FQ_BLOCK_FP32, "mx": fq.FQ_MX, "nvfp4": fq.FQ_NVFP4}
FORMATS = {"e4m3": fq.FQ_E4M3, "e5m2": fq.FQ_E5M2, "e2m1": fq.FQ_E2M1}


@pytest.mark.parametrize("w", [W.SMALL_CURRENT, *W.LARGE], ids=lambda w: w.name)
def test_algorithmic_bytes_from_the_library_plane_sizes(w):
    R, C = w.shape
    d = fq.desc(RECIPES[w.recipe], fq.FQ_IN_BF16 if w.dtype == W.BF16 else fq.FQ_IN_F32, FORMATS[w.fmt], R, C,
                w.block or (0, 0), w.outputs)
    z = fq.fq_sizes(d)
    eb = 2 if w.dtype == W.BF16 else 4
    passes = {"current": 2, "nvfp4": 2}.get(w.recipe, 1)    # current scaling and NVFP4 read the input twice
    planes = z.row_data + z.row_scale + z.col_data + z.col_scale
    scalars = {"current": 4,                                  # s
               "nvfp4": 4,                                    # the tensor scale S
               "delayed": 2 * 4 * w.extra.get("history_len", 0) + 3 * 4}.get(w.recipe, 0)
    assert bench.algorithmic_bytes(w) == passes * R * C * eb + planes + scalars


def test_step_bytes_and_roofline_peak():
    total = sum(bench.algorithmic_bytes(w) for w in W.LARGE)
    assert total == 2362195496                                 # the step's figure in the bench line
    assert bench.HBM_PEAK_GBS == 8000.0


def test_kernel_source_maps_agree():
    """The benchmark reports traffic only while the hash over a kernel's
    sources matches the summary; both sides must hash the same files."""
    for key, kernel in bench.KERNEL_NAMES.items():
        recipe = next(r for r in bench.KERNEL_FILES if key.startswith(r))
        assert profsum.KERNEL_SOURCES[kernel] == bench.KERNEL_FILES[recipe], (key, kernel)


def write_counters(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for r in rows:
            wr.writerow(r)


def test_traffic_summary_scaling(tmp_path):
    """Two dispatches of a kernel, counters split over two instances each;
    the copy reads half its bytes through FETCH_SIZE (scale 2) and all of
    them through WRITE_SIZE (scale 1)."""
    copy = profsum.COPY_KERNEL
    kern = "void fq::(anonymous namespace)::k_block_128x128<unsigned short, false, 2>(...)"
    kib = profsum.COPY_BYTES / 1024
    fetch = [dict(Dispatch_Id=1, Kernel_Name=copy, Counter_Name="FETCH_SIZE", Counter_Value=kib / 4),
             dict(Dispatch_Id=1, Kernel_Name=copy, Counter_Name="FETCH_SIZE", Counter_Value=kib / 4),
             dict(Dispatch_Id=2, Kernel_Name=kern, Counter_Name="FETCH_SIZE", Counter_Value=600.0),
             dict(Dispatch_Id=2, Kernel_Name=kern, Counter_Name="FETCH_SIZE", Counter_Value=400.0),
             dict(Dispatch_Id=3, Kernel_Name=kern, Counter_Name="FETCH_SIZE", Counter_Value=1100.0),
             dict(Dispatch_Id=3, Kernel_Name=kern, Counter_Name="FETCH_SIZE", Counter_Value=900.0)]
    write = [dict(Dispatch_Id=1, Kernel_Name=copy, Counter_Name="WRITE_SIZE", Counter_Value=kib),
             dict(Dispatch_Id=2, Kernel_Name=kern, Counter_Name="WRITE_SIZE", Counter_Value=300.0),
             dict(Dispatch_Id=3, Kernel_Name=kern, Counter_Name="WRITE_SIZE", Counter_Value=500.0)]
    fc, wc, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    write_counters(fc, fetch)
    write_counters(wc, write)
    profsum.traffic(str(fc), str(wc), "k_block_128x128<unsigned short, false, 2>", "wl", "1x1", str(out), "cmd")
    t = json.loads(out.read_text())
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    assert t["fetch_kib_per_dispatch"] == pytest.approx(1500.0)          # (1000 + 2000) / 2
    assert t["hbm_read_bytes_per_launch"] == 1500 * 1024 * 2
    assert t["hbm_write_bytes_per_launch"] == 400 * 1024
    assert t["source_hash"] == profsum.source_hash(["k_block.hip", "codec.hpp"])


def test_traffic_for_ignores_a_stale_summary(tmp_path, monkeypatch):
    """bench.traffic_for returns the recorded bytes only while the hash of the
    kernel's sources is the one recorded."""
    w = W.BY_NAME["block128x128_wgt_7168x18432"]
    path = tmp_path / "traffic_block128x128_7168x18432.json"
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path.write_text(json.dumps({"source_hash": profsum.source_hash(bench.KERNEL_FILES["block"]),
                                "hbm_bytes_per_launch": 123}))
    assert bench.traffic_for(w, 0) == 123
    path.write_text(json.dumps({"source_hash": "0" * 16, "hbm_bytes_per_launch": 123}))
    assert bench.traffic_for(w, 0) is None


SMALL = [
    W.Workload("cur", (96, 256), W.BF16, "current", "e4m3", seed=11),
    W.Workload("del", (96, 256), W.BF16, "delayed", "e5m2", seed=12, std=1e-3, extra={"history_len": 8}),
    W.Workload("b1", (96, 256), W.BF16, "block", "e4m3", block=(1, 128), seed=13),
    W.Workload("b128", (384, 256), W.BF16, "block", "e4m3", block=(128, 128), seed=14, std=0.02),
    W.Workload("mx", (160, 128), W.BF16, "mx", "e4m3", block=(1, 32), outputs=3, seed=15, dist="student_t",
               extra={"nu": 3.0}),
    W.Workload("nv1", (96, 256), W.BF16, "nvfp4", "e2m1", block=(1, 16), seed=16),
    W.Workload("nv16", (96, 256), W.BF16, "nvfp4", "e2m1", block=(16, 16), seed=17, std=0.02),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_partitioned_oracle_equals_one_thread(w):
    """The all-core oracle baseline splits rows over threads (cut at block
    heights) and combines per-tensor amaxes with an exact max; its bytes,
    scales and delayed-scaling state equal one oracle call on the whole
    tensor."""
    import concurrent.futures

    import numpy as np

    import oracle as orc

    x = w.make()
    fmt = {"e4m3": orc.E4M3, "e5m2": orc.E5M2, "e2m1": orc.E2M1}[w.fmt]
    # one oracle call on the whole tensor
    if w.recipe == "current":
        whole = orc.quantize_current(x, fmt, outputs=w.outputs)
    elif w.recipe == "delayed":
        st = orc.DelayedState(w.extra["history_len"])
        whole = orc.quantize_delayed(x, fmt, st, outputs=w.outputs)
        whole.update(hist=st.hist, alpha=st.alpha, s=st.s)
    elif w.recipe == "block":
        whole = orc.quantize_block(x, w.block, outputs=w.outputs)
    elif w.recipe == "mx":
        whole = orc.quantize_mx(x, outputs=w.outputs, fmt=fmt)
    else:
        whole = orc.quantize_nvfp4(x, w.block, outputs=w.outputs)
    with concurrent.futures.ThreadPoolExecutor(max_workers=3) as pool:
        parts = bench.assemble(w, bench.oracle_partitioned(w, x, 3, pool))
        assert len(bench.row_parts(w.shape[0], bench.part_unit(w), 3)) == 3
    for k, v in parts.items():
        if v is None or k not in whole:
            continue
        a, b = np.atleast_1d(np.asarray(whole[k])), np.atleast_1d(np.asarray(v))
        assert a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8)), (w.name, k)
    assert {k for k, v in whole.items() if v is not None} <= set(parts)


def test_row_parts_cut_at_the_unit():
    assert bench.row_parts(384, 128, 3) == [(0, 128), (128, 256), (256, 384)]
    assert bench.row_parts(100, 1, 3) == [(0, 33), (33, 66), (66, 100)]
    assert bench.row_parts(96, 32, 5) == [(0, 32), (32, 64), (64, 96)]


def test_launches_per_call():
    """A delayed step with a window of at most 1024 slots is one kernel (its
    finish rides in the next step's cast); the two-pass recipes are two."""
    by = {w.name: bench.launches_per_call(w) for w in W.LARGE}
    assert by["delayed_e4m3_act_8192x4096"] == 1 and by["current_e4m3_act_8192x4096"] == 2
    assert by["nvfp4_1x16_act_8192x14336"] == 2 and by["block128x128_wgt_7168x18432"] == 1
    long = W.Workload("dl", (96, 256), W.BF16, "delayed", "e4m3", extra={"history_len": 2048})
    assert bench.launches_per_call(long) == 2


def test_fastest_step_from_a_trace():
    """The step table of the trace summaries: the library's dispatches cut
    after each final kernel of a step, the shortest full step kept; other
    kernels (torch's) and an incomplete tail are left out."""
    def row(name, s, e):
        return {"Kernel_Name": name, "Start_Timestamp": str(s), "End_Timestamp": str(e)}
    a = "void fq::(anonymous namespace)::k_amax_partial<unsigned short, 8>(x)"
    z = "void fq::(anonymous namespace)::k_nvfp4_16x16<unsigned short>(x)"
    rows = [row(a, 0, 10), row("at::native::copy(x)", 11, 12), row(z, 20, 40),    # span 40
            row(a, 100, 105), row(z, 105, 120),                                     # span 20
            row(a, 200, 230), row(z, 240, 300),                                     # span 100
            row(a, 400, 401)]                                                       # no final kernel
    step = profsum.fastest_step(rows)
    assert [r["Start_Timestamp"] for r in step] == ["100", "105"]
    assert profsum.fastest_step([row(a, 0, 1)]) == []
