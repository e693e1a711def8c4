"""Benchmark: FP8/FP4 quantization throughput on one MI355X.

One step quantizes every large workload once, each with its own recipe:
per-tensor current scaling (E4M3 activation, E5M2 gradient, 8192x4096 bf16),
delayed scaling with a 1024-entry window (same two tensors), blockwise 1x128
(16384x7168) and 128x128 (7168x18432), MXFP8 rowwise + colwise (8192x8192)
and NVFP4 1x16 (8192x14336) and 16x16 (14336x4096). Inputs are seeded,
synthetic and resident in HBM before timing; the step touches more than the
256 MB Infinity Cache, so each workload starts cold.

value = algorithmic bytes per step / time per step, in GB/s, over K steps
with nothing recorded between the calls. Algorithmic
bytes count one read of the input per pass the method makes (two for current
scaling and NVFP4, one otherwise) plus every byte written (codes, scales,
delayed-scaling window and scale).

Prints one JSON line. Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantize GB/s (bytes read+written) and % of HBM peak, per recipe"
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def launches_per_call(w):
    """Kernels one call enqueues: two passes for current scaling and NVFP4;
    one for delayed scaling while the window is short enough to be finished
    inside the next step's cast, else a separate finish kernel as well."""
    if w.recipe in ("current", "nvfp4"):
        return 2
    if w.recipe == "delayed" and w.extra["history_len"] > 1024:
        return 2
    return 1


def algorithmic_bytes(w) -> int:
    R, C = w.shape
    n = R * C
    eb = 2 if w.dtype == "bf16" else 4
    if w.recipe == "current":
        return 2 * n * eb + n + 4                      # amax read, cast read, codes, s
    if w.recipe == "delayed":
        H = w.extra["history_len"]
        return n * eb + n + 2 * 4 * H + 3 * 4          # one read, codes, window r/w, alpha, s, s_used
    if w.recipe == "block":
        br, bc = w.block
        return n * eb + n + (R // br) * (C // bc) * 4
    if w.recipe == "mx":
        return n * eb + 2 * n + 2 * (n // 32)          # rowwise + colwise codes and E8M0 scales
    if w.recipe == "nvfp4":
        br, bc = w.block
        return 2 * n * eb + n // 2 + (R // br) * (C // bc) + 4
    raise ValueError(w.recipe)


# which source files define each workload's kernels (for the traffic counters)
KERNEL_FILES = {"current": ["k_tensor.hip", "codec.hpp"], "delayed": ["k_tensor.hip", "codec.hpp"],
                "block": ["k_block.hip", "codec.hpp"], "mx": ["k_mx.hip", "codec.hpp"],
                "nvfp4": ["k_nvfp4.hip", "k_tensor.hip", "codec.hpp"]}
KERNEL_NAMES = {"current": "k_cast_tensor", "delayed": "k_cast_delayed", "block1x128": "k_block_1x128",
                "block128x128": "k_block_128x128", "mx": "k_mx_bf16", "nvfp4_1x16": "k_nvfp4_1x16",
                "nvfp4_16x16": "k_nvfp4_16x16"}


def kernel_key(w):
    if w.recipe == "block":
        return "block1x128" if w.block == (1, 128) else "block128x128"
    if w.recipe == "nvfp4":
        return "nvfp4_1x16" if w.block == (1, 16) else "nvfp4_16x16"
    return w.recipe


def traffic_for(w, per_launch_alg_bytes):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or the kernel's sources changed since."""
    path = os.path.join(PROFILES, f"traffic_{kernel_key(w)}_{w.shape[0]}x{w.shape[1]}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    from fp8_fp4_tensor_amd.profsum import source_hash
    if t.get("source_hash") != source_hash(KERNEL_FILES[w.recipe]):
        return None
    return t.get("hbm_bytes_per_launch")


def rocprof_duration(w, kernel, per_launch_alg_bytes):
    """The kernel's mean duration in the committed rocprofv3 kernel-trace
    summary of the step (profiles/kernels_bench_step_all_workloads.json),
    with the rate it gives, or None if there is none or the kernel's sources
    changed since it was taken."""
    path = os.path.join(PROFILES, "kernels_bench_step_all_workloads.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    from fp8_fp4_tensor_amd.profsum import source_hash
    found = [(n, k) for n, k in t.get("kernels", {}).items() if n.split("<")[0] == kernel]
    if len(found) != 1 or found[0][1].get("source_hash") != source_hash(KERNEL_FILES[w.recipe]):
        return None
    us = found[0][1]["mean_us"]
    gbs = per_launch_alg_bytes / (us * 1e-6) / 1e9
    return {"us_per_launch": us, "achieved": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
            "file": "profiles/kernels_bench_step_all_workloads.json"}


COPY_BYTES = 256 << 20


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence:
    recording it skips the system-scope fence (a cache write-back and
    invalidate on this GPU) that a default event adds between the kernels it
    brackets, which otherwise inflates a bracketed kernel's time by a few us.
    Same interface as torch.cuda.Event: record(stream), elapsed_time(end)."""
    _hip = None

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import torch
            # the HIP runtime torch already loaded (one runtime per process)
            path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
            hip = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        self.ev = ctypes.c_void_p()
        if self._lib().hipEventCreateWithFlags(ctypes.byref(self.ev), 0x20000000) != 0:  # DisableSystemFence
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream=None):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        if self._lib().hipEventRecord(self.ev, ctypes.c_void_p(s.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        ms = ctypes.c_float()
        if self._lib().hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


def plain_copy(torch, stream, reps):
    """Bandwidth of a plain device-to-device copy of 256 MiB (read + write)."""
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    del a, b
    return 2 * COPY_BYTES / t / 1e9


# rows of a partition are a multiple of this, so every block (and every
# colwise block down the columns) lies inside one partition
PART_UNIT = {"current": 1, "delayed": 1, "mx": 32}


def part_unit(w):
    if w.recipe in PART_UNIT:
        return PART_UNIT[w.recipe]
    br = w.block[0]
    if w.outputs & 2:                       # colwise blocks run down the columns
        return max(br, w.block[1])
    return br


def row_parts(R, unit, parts):
    """`parts` row ranges [r0, r1) of about equal size, cut at multiples of unit."""
    units = R // unit
    cuts = [unit * (units * k // parts) for k in range(parts + 1)]
    cuts[-1] = R
    return [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]


def oracle_partitioned(w, x, parts, pool):
    """The oracle on workload w's host input x, its rows split into `parts`
    ranges run on `pool`'s threads (each oracle call releases the GIL).
    Per-tensor amaxes are combined with an exact max before the cast, as the
    sharded flow does. Returns the raw per-partition results."""
    import oracle as orc

    fmt = {"e4m3": orc.E4M3, "e5m2": orc.E5M2, "e2m1": orc.E2M1}[w.fmt]
    rng = row_parts(x.shape[0], part_unit(w), parts)
    xs = [x[a:b] for a, b in rng]

    def amax_all():
        return max(pool.map(orc.amax, xs))

    if w.recipe == "current":
        A = amax_all()
        return [dict(r, amax=A) for r in pool.map(lambda xp: orc.quantize_with_amax(xp, fmt, A, outputs=w.outputs),
                                                  xs)]
    if w.recipe == "delayed":
        st = orc.DelayedState(w.extra["history_len"])

        def step(xp):
            # every partition casts with the same old scale; its own copy of
            # the state records its own amax
            mine = st.copy()
            return orc.quantize_delayed(xp, fmt, mine, outputs=w.outputs), mine
        return list(pool.map(step, xs))
    if w.recipe == "block":
        return list(pool.map(lambda xp: orc.quantize_block(xp, w.block, outputs=w.outputs), xs))
    if w.recipe == "mx":
        return list(pool.map(lambda xp: orc.quantize_mx(xp, outputs=w.outputs, fmt=fmt), xs))
    if w.recipe == "nvfp4":
        A = amax_all()
        return list(pool.map(lambda xp: orc.quantize_nvfp4(xp, w.block, outputs=w.outputs, amax=A), xs))
    raise ValueError(w.recipe)


def assemble(w, results):
    """One tensor's outputs from per-partition results (rowwise planes stack
    by rows; colwise planes, stored transposed, by columns)."""
    import numpy as np

    if w.recipe == "delayed":
        # the partition holding the largest amax made the whole tensor's update
        best = max(results, key=lambda r: r[0]["amax"])
        st = best[1]
        return {"q_row": np.concatenate([r[0]["q_row"] for r in results]), "amax": best[0]["amax"],
                "hist": st.hist, "alpha": st.alpha, "s": st.s}
    out = {}
    for k, v in results[0].items():
        if v is None or np.ndim(v) == 0:
            out[k] = v
        elif k.endswith("_col"):
            out[k] = np.concatenate([r[k] for r in results], axis=1)
        else:
            out[k] = np.concatenate([r[k] for r in results], axis=0)
    return out


def cpu_baseline(hosts, threads, one_thread_fraction):
    """The oracle on the host: every workload of the step on all `threads`
    (rows partitioned), and every workload on its first rows on one thread."""
    import concurrent.futures

    from fp8_fp4_tensor_amd import workloads as W

    def run(parts, fraction):
        total_bytes, total_t, per = 0, 0.0, {}
        with concurrent.futures.ThreadPoolExecutor(max_workers=parts) as pool:
            for w, x in hosts:
                R, C = w.shape
                unit = max(part_unit(w), 128 if w.recipe == "block" else 1)
                r = R if fraction >= 1 else max(unit, int(R * fraction) // unit * unit)
                xs = x[:r]
                sub = W.Workload(w.name, (r, C), w.dtype, w.recipe, w.fmt, w.block, w.outputs, w.seed, w.dist,
                                 w.std, w.extra)
                t0 = time.perf_counter()
                oracle_partitioned(w, xs, parts, pool)
                dt = time.perf_counter() - t0
                total_t += dt
                total_bytes += algorithmic_bytes(sub)
                per[w.name] = round(algorithmic_bytes(sub) / dt / 1e9, 3)
        return total_bytes, total_t, per

    nb, nt, nper = run(threads, 1.0)
    ob, ot, oper = run(1, one_thread_fraction)
    cpu = host_cpu()
    return {"value": round(nb / nt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"every workload of one step, all rows, split by rows over {threads} threads "
                      f"({nb / 1e9:.2f} GB algorithmic in {nt:.1f} s wall; {cpu})",
            "per_workload_GBps": nper,
            "one_thread": {"value": round(ob / ot / 1e9, 3), "cores": 1,
                           "sample": f"every workload on its first {one_thread_fraction:.0%} of rows "
                                     f"({ob / 1e9:.2f} GB in {ot:.1f} s)",
                           "per_workload_GBps": oper}}


def host_cpu():
    """The host CPU's model name and logical CPU count, for the baseline's record."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {os.cpu_count()} logical CPUs"


def plane_bytes(w, which):
    """Code and scale bytes of one plane of workload w (what a dequantize reads)."""
    R, C = w.shape
    n = R * C
    if w.recipe in ("current", "delayed"):
        return n + 4
    if w.recipe == "block":
        br, bc = w.block
        return n + 4 * n // (br * bc)
    if w.recipe == "mx":
        return n + n // 32
    br, bc = w.block
    return n // 2 + n // (br * bc) + 4


def time_extras(torch, fq, L, stream_p, jobs, steps, flush):
    """Dequantize (rowwise plane to bf16), MXFP8 and pow2 blockwise 1x128
    rowwise-to-colwise requantize, NVFP4 1x16 with stochastic rounding, the NVFP4 colwise copy with the RHT and
    stochastic rounding, stochastic rounding of the 8-bit elements (the E5M2
    gradient, blockwise 1x128 and MXFP8 workloads, `sr8`), MX with E5M2 and
    E2M1 elements, blockwise with power-of-two scales, and the rowwise-only
    recipes with both planes
    (rowcol) or the colwise plane alone (colwise), at the large workloads'
    shapes, each call bracketed by events and started cold (flush() runs
    before it, outside the events); not part of the step."""
    out = {}

    def time_requant(d_src, c_src, d_dst, nbytes, name, ev):
        """Colwise copy from the rowwise copy (c_src) into fresh planes of d_dst."""
        dst = fq.alloc_quantized(d_dst)
        cdst = dst.c()
        for k in range(-1, steps):
            flush()
            if k >= 0:
                ev[k][0].record()
            rc = L.fq_requantize_transpose(ctypes.byref(d_src), ctypes.byref(c_src), ctypes.byref(cdst), stream_p)
            if k >= 0:
                ev[k][1].record()
            if rc != fq.FQ_OK:
                raise fq.FqError(rc, "requantize " + name)
        torch.cuda.synchronize()
        us = 1e3 * sum(a.elapsed_time(b) for a, b in ev) / steps
        out["requant_colwise/" + name] = {"us_per_call": round(us, 2), "bytes": nbytes,
                                          "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}

    for j in jobs:
        w = j["w"]
        R, C = w.shape
        y = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
        ev = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
        for k in range(-1, steps):
            flush()
            if k >= 0:
                ev[k][0].record()
            rc = L.fq_dequantize(ctypes.byref(j["d"]), ctypes.byref(j["cq"]), fq.FQ_ROWWISE,
                                 ctypes.c_void_p(y.data_ptr()), fq.FQ_IN_BF16, stream_p)
            if k >= 0:
                ev[k][1].record()
            if rc != fq.FQ_OK:
                raise fq.FqError(rc, "dequantize " + w.name)
        torch.cuda.synchronize()
        us = 1e3 * sum(a.elapsed_time(b) for a, b in ev) / steps
        nbytes = plane_bytes(w, fq.FQ_ROWWISE) + 2 * R * C
        out["dequant_bf16/" + w.name] = {"us_per_call": round(us, 2), "bytes": nbytes,
                                         "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}
        del y
        if w.recipe == "nvfp4" and tuple(w.block) == (1, 16):
            # the same workload with stochastically rounded elements (a gradient)
            d = j["d"]
            dsr = fq.desc(d.recipe, d.in_dtype, d.format, R, C, (1, 16), d.outputs,
                          rounding=fq.FQ_ROUND_STOCHASTIC, seed=2024, offset=0)
            for k in range(-1, steps):
                flush()
                dsr.offset = k + 1
                if k >= 0:
                    ev[k][0].record()
                rc = L.fq_quantize(ctypes.byref(dsr), j["xp"], ctypes.byref(j["cq"]), j["wsp"], j["wsn"], stream_p)
                if k >= 0:
                    ev[k][1].record()
                if rc != fq.FQ_OK:
                    raise fq.FqError(rc, "stochastic rounding " + w.name)
            torch.cuda.synchronize()
            us = 1e3 * sum(a.elapsed_time(b) for a, b in ev) / steps
            out["nvfp4_1x16_sr/" + w.name] = {"us_per_call": round(us, 2), "bytes": j["bytes"],
                                              "GB/s": round(j["bytes"] / (us * 1e-6) / 1e9, 1)}
        variants = []
        if w.recipe == "mx":
            variants = [("mx_e5m2", fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E5M2, R, C, (1, 32), w.outputs),
                         j["bytes"]),
                        ("mxfp4", fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (1, 32), w.outputs),
                         2 * R * C + R * C + 2 * (R * C // 32))]
        if w.recipe == "block":
            variants = [("block_pow2", fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, w.block, w.outputs,
                                               scale_mode=fq.FQ_SCALE_POW2), j["bytes"])]
        if w.recipe == "nvfp4" and tuple(w.block) == (1, 16):
            # weight-gradient input: colwise copy with the RHT and stochastic rounding (two reads)
            variants = [("nvfp4_colwise_rht_sr",
                         fq.desc(fq.FQ_NVFP4, fq.FQ_IN_BF16, fq.FQ_E2M1, R, C, (1, 16), fq.FQ_COLWISE,
                                 rounding=fq.FQ_ROUND_STOCHASTIC, seed=2024, offset=1,
                                 transform=fq.FQ_TRANSFORM_RHT16, rht_signs=0xA5C3),
                         2 * 2 * R * C + R * C // 2 + R * C // 16 + 4)]
        d0 = j["d"]
        if ((w.recipe == "current" and d0.format == fq.FQ_E5M2) or (w.recipe == "block" and tuple(w.block) == (1, 128))
                or w.recipe == "mx"):
            # the same workload with stochastically rounded 8-bit elements
            variants.append(("sr8", fq.desc(d0.recipe, d0.in_dtype, d0.format, R, C, w.block or (0, 0), w.outputs,
                                            rounding=fq.FQ_ROUND_STOCHASTIC, seed=2024, offset=3), j["bytes"]))
        if w.recipe in ("current", "block", "nvfp4") and w.outputs == fq.FQ_ROWWISE:
            # the same recipe with both planes (the colwise copy for the
            # backward GEMMs): bytes from the library's own plane sizes
            d = j["d"]
            drc = fq.desc(d.recipe, d.in_dtype, d.format, R, C, w.block or (0, 0), fq.FQ_ROWWISE | fq.FQ_COLWISE)
            z = fq.fq_sizes(drc)
            two_pass = w.recipe in ("current", "nvfp4")
            variants.append(("rowcol", drc, (2 if two_pass else 1) * 2 * R * C + z.row_data + z.row_scale
                             + z.col_data + z.col_scale + (4 if two_pass else 0)))
            dco = fq.desc(d.recipe, d.in_dtype, d.format, R, C, w.block or (0, 0), fq.FQ_COLWISE)
            variants.append(("colwise", dco, (2 if two_pass else 1) * 2 * R * C + z.col_data + z.col_scale
                             + (4 if two_pass else 0)))
        for vname, dv, nbytes in variants:
            ov = fq.alloc_quantized(dv)
            cov = ov.c()
            wsv = fq.alloc_workspace(dv)
            wsp = None if wsv is None else ctypes.c_void_p(wsv.data_ptr())
            wsn = 0 if wsv is None else wsv.numel()
            for k in range(-1, steps):
                flush()
                if k >= 0:
                    ev[k][0].record()
                rc = L.fq_quantize(ctypes.byref(dv), j["xp"], ctypes.byref(cov), wsp, wsn, stream_p)
                if k >= 0:
                    ev[k][1].record()
                if rc != fq.FQ_OK:
                    raise fq.FqError(rc, vname + " " + w.name)
            torch.cuda.synchronize()
            us = 1e3 * sum(a.elapsed_time(b) for a, b in ev) / steps
            out[vname + "/" + w.name] = {"us_per_call": round(us, 2), "bytes": nbytes,
                                         "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}
            if vname == "block_pow2" and tuple(w.block) == (1, 128) and dv.outputs & fq.FQ_ROWWISE:
                # the blockwise requantize from this pow2 rowwise copy: codes and
                # fp32 tile scales read, the same written transposed
                dc = fq.desc(fq.FQ_BLOCK_FP32, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 128), fq.FQ_COLWISE,
                             scale_mode=fq.FQ_SCALE_POW2)
                time_requant(dv, cov, dc, 2 * (R * C + 4 * (R * C // 128)), "block_pow2_" + w.name, ev)
            del ov
        if w.recipe == "mx":
            d = fq.desc(fq.FQ_MX, fq.FQ_IN_BF16, fq.FQ_E4M3, R, C, (1, 32), fq.FQ_COLWISE)
            time_requant(j["d"], j["cq"], d, 2 * (R * C + R * C // 32), w.name, ev)
    return out


def time_clean_cold(torch, jobs, call, steps, flush):
    """Every workload's call from a clean cold cache (flush() outside the
    events, as for torch's cast reference), where in the step it follows
    kernels that have just written their outputs: the same call without the
    write-back of the previous workload's dirty lines."""
    out = {}
    for j in jobs:
        ev = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
        for k in range(-1, steps):
            flush()
            if k >= 0:
                ev[k][0].record()
            call(j)
            if k >= 0:
                ev[k][1].record()
        torch.cuda.synchronize()
        us = 1e3 * sum(a.elapsed_time(b) for a, b in ev) / steps
        out[j["w"].name] = {"us_per_call": round(us, 2), "GB/s": round(j["bytes"] / (us * 1e-6) / 1e9, 1)}
    return out


def time_second_read(torch, fq, L, stream_p, jobs, steps, flush):
    """The second read of the two-pass recipes (current scaling and NVFP4),
    with and without the memory-side cache: fq_amax (pass 1), then
    fq_quantize_with_amax (pass 2) either right after pass 1 (its input
    partly still in the 256 MB memory-side cache) or after a flush (its
    input cold, every byte from HBM). Events bracket each pass; the flush is
    outside them. No rocprofv3 counter on this chip separates
    memory-side-cache hits from HBM reads, so this timing split is the
    evidence of how much the cache serves."""
    out = {}
    for j in jobs:
        w = j["w"]
        if w.recipe not in ("current", "nvfp4"):
            continue
        d = j["d"]
        amax = torch.empty(1, dtype=torch.float32, device="cuda")
        ap = ctypes.c_void_p(amax.data_ptr())
        ev = [[TimingEvent() for _ in range(4)] for _ in range(steps)]
        for cold in (False, True):
            for k in range(-1, steps):
                flush()
                e = ev[max(k, 0)]
                if k >= 0:
                    e[0].record()
                rc = L.fq_amax(ctypes.byref(d), j["xp"], ap, j["wsp"], j["wsn"], stream_p)
                if k >= 0:
                    e[1].record()
                if cold:
                    flush()
                if k >= 0:
                    e[2].record()
                rc |= L.fq_quantize_with_amax(ctypes.byref(d), j["xp"], ap, ctypes.byref(j["cq"]), j["wsp"],
                                              j["wsn"], stream_p)
                if k >= 0:
                    e[3].record()
                if rc != fq.FQ_OK:
                    raise fq.FqError(rc, "second read " + w.name)
            torch.cuda.synchronize()
            p1 = 1e3 * sum(e[0].elapsed_time(e[1]) for e in ev) / steps
            p2 = 1e3 * sum(e[2].elapsed_time(e[3]) for e in ev) / steps
            key = "pass2_cold_us" if cold else "pass2_after_pass1_us"
            r = out.setdefault(w.name, {})
            r[key] = round(p2, 2)
            r.setdefault("pass1_us", round(p1, 2))
        r = out[w.name]
        R, C = w.shape
        r["two_pass_hbm_only_GB/s"] = round(j["bytes"] / ((r["pass1_us"] + r["pass2_cold_us"]) * 1e-6) / 1e9, 1)
        r["note"] = ("pass 1 = fq_amax (amax partials + their max), pass 2 = fq_quantize_with_amax; "
                     f"{2 * R * C} B read by pass 2 alone")
    return out


def torch_cast_reference(torch, stream, steps, flush):
    """torch's own bf16 -> float8_e4m3fn cast of an 8192x4096 tensor (2 bytes
    read, 1 written per element, no amax, no scale): a 2:1 stream reference
    from a library other than this one. Each cast starts cold."""
    x = torch.randn(8192, 4096, device="cuda").to(torch.bfloat16)
    y = torch.empty(8192, 4096, dtype=torch.float8_e4m3fn, device="cuda")
    ev = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
    for k in range(-2, steps):
        flush()
        if k >= 0:
            ev[k][0].record(stream)
        y.copy_(x)
        if k >= 0:
            ev[k][1].record(stream)
    torch.cuda.synchronize()
    us = 1e3 * sum(a.elapsed_time(b) for a, b in ev) / steps
    nbytes = 3 * x.numel()
    del x, y
    return {"what": "torch bf16 -> float8_e4m3fn copy_, 8192x4096, cold input", "us": round(us, 2),
            "bytes": nbytes, "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}


def time_small(torch, fq, L, stream_p, steps, flush):
    """The small per-tensor workload (2^20 fp32 with outliers, current
    scaling to E4M3): a few MiB, so launch latency bounds it; each call
    bracketed by events, not part of the step."""
    from fp8_fp4_tensor_amd import workloads as W
    w = W.SMALL_CURRENT
    R, C = w.shape
    x = torch.from_numpy(w.make()).cuda()
    d = fq.desc(fq.FQ_PER_TENSOR_CURRENT, fq.FQ_IN_F32, fq.FQ_E4M3, R, C, (0, 0), fq.FQ_ROWWISE)
    out = fq.alloc_quantized(d)
    ws = fq.alloc_workspace(d)
    cq = out.c()
    args = (ctypes.byref(d), ctypes.c_void_p(x.data_ptr()), ctypes.byref(cq), ctypes.c_void_p(ws.data_ptr()),
            ws.numel(), stream_p)
    ev = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
    for k in range(-3, steps):
        flush()
        if k >= 0:
            ev[k][0].record()
        rc = L.fq_quantize(*args)
        if k >= 0:
            ev[k][1].record()
        if rc != fq.FQ_OK:
            raise fq.FqError(rc, w.name)
    torch.cuda.synchronize()
    us = 1e3 * sum(a.elapsed_time(b) for a, b in ev) / steps
    nbytes = algorithmic_bytes(w)
    return {w.name: {"us_per_call": round(us, 2), "bytes": nbytes, "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads of the all-core oracle baseline (default: the host's CPUs, at most 16)")
    ap.add_argument("--cpu-rows", type=float, default=0.2,
                    help="row fraction of the one-thread oracle baseline")
    ap.add_argument("--repeats", type=int, default=5,
                    help="per-recipe figures: median over this many repeats of K calls")
    ap.add_argument("--only", default="", help="comma-separated workload names (profiling runs)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the dequantize / requantize timings reported beside the step")
    ap.add_argument("--copy-only", action="store_true",
                    help="time only a plain 256 MiB device copy (counter calibration and reference)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the sharded path is "
              "design-only, see the library's documentation)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from fp8_fp4_tensor_amd import fq
    from fp8_fp4_tensor_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    copy_gbs = plain_copy(torch, stream, args.steps if args.copy_only else 10)
    if args.copy_only:
        print(json.dumps({"copy_bytes": 2 * COPY_BYTES, "copy_GBps": round(copy_gbs, 1)}), flush=True)
        return

    recipes = {"current": fq.FQ_PER_TENSOR_CURRENT, "delayed": fq.FQ_PER_TENSOR_DELAYED,
               "block": fq.FQ_BLOCK_FP32, "mx": fq.FQ_MX, "nvfp4": fq.FQ_NVFP4}
    fmts = {"e4m3": fq.FQ_E4M3, "e5m2": fq.FQ_E5M2, "e2m1": fq.FQ_E2M1}
    wls = W.LARGE
    if args.only:
        keep = set(args.only.split(","))
        wls = [w for w in wls if w.name in keep]

    L = fq.lib()
    sp = ctypes.c_void_p(stream.cuda_stream)
    jobs = []
    for w in wls:
        R, C = w.shape
        x = w.make()
        xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
        d = fq.desc(recipes[w.recipe], fq.FQ_IN_BF16, fmts[w.fmt], R, C, w.block or (0, 0), w.outputs)
        out = fq.alloc_quantized(d)
        ws = fq.alloc_workspace(d)
        st = fq.DelayedState(w.extra["history_len"]) if w.recipe == "delayed" else None
        # the C arguments, built once: each call below is one ctypes call into libfq.so
        j = dict(w=w, x=xd, d=d, out=out, ws=ws, st=st, bytes=algorithmic_bytes(w), cq=out.c(),
                 xp=ctypes.c_void_p(xd.data_ptr()), wsp=ctypes.c_void_p(ws.data_ptr()) if ws is not None else None,
                 wsn=0 if ws is None else ws.numel(), cst=st.c() if st is not None else None,
                 xh=None if args.no_cpu_baseline else x)   # host copy for the oracle baseline
        if w.recipe == "delayed":
            # a step's outputs are its codes, the s used, the window and the
            # scales; the optional a_t output would add a kernel
            j["cq"].amax = None
        jobs.append(j)
        del x
    print(f"bench: {len(jobs)} workloads resident, {sum(j['x'].numel() * 2 for j in jobs) / 2**30:.2f} GiB input",
          file=sys.stderr, flush=True)

    def call(j):
        if j["cst"] is not None:
            rc = L.fq_quantize_delayed(ctypes.byref(j["d"]), j["xp"], ctypes.byref(j["cst"]), ctypes.byref(j["cq"]),
                                       j["wsp"], j["wsn"], sp)
            j["cst"].step += 1
        else:
            rc = L.fq_quantize(ctypes.byref(j["d"]), j["xp"], ctypes.byref(j["cq"]), j["wsp"], j["wsn"], sp)
        if rc != fq.FQ_OK:
            raise fq.FqError(rc, j["w"].name)

    for _ in range(args.warmup):
        for j in jobs:
            call(j)
    torch.cuda.synchronize()

    # per-recipe breakdown: `repeats` rounds of K instrumented steps, every
    # call bracketed by fence-free events (each call starts with its input
    # cold, as in the timed region below); each workload's figure is the
    # median over the rounds of its mean time per call
    rounds = {j["w"].name: [] for j in jobs}
    for _ in range(max(1, args.repeats)):
        for j in jobs:
            j["events"] = [(TimingEvent(), TimingEvent()) for _ in range(args.steps)]
        for k in range(args.steps):
            for j in jobs:
                j["events"][k][0].record(stream)
                call(j)
                j["events"][k][1].record(stream)
        torch.cuda.synchronize()
        for j in jobs:
            rounds[j["w"].name].append(1e3 * sum(a.elapsed_time(b) for a, b in j["events"]) / args.steps)
    per = {}
    for j in jobs:
        us = float(np.median(rounds[j["w"].name]))
        gbs = j["bytes"] / (us * 1e-6) / 1e9
        per[j["w"].name] = {"us_per_call": round(us, 2), "GB/s": round(gbs, 1),
                            "alg_pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 1), "bytes": j["bytes"],
                            "us_rounds": [round(v, 2) for v in rounds[j["w"].name]],
                            "kernels": launches_per_call(j["w"])}
    # the dominant kernel: the single-kernel workload with the largest time per call
    single = [j for j in jobs if per[j["w"].name]["kernels"] == 1]
    dom = max(single, key=lambda j: per[j["w"].name]["us_per_call"]) if single else None

    # timed region: K steps with nothing recorded between the calls (an event
    # record on the stream puts a gap of ~4 us before the next kernel)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(args.steps):
        for j in jobs:
            call(j)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    step_bytes = sum(j["bytes"] for j in jobs)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # the roofline kernel: K more steps, identical to the timed ones, with
    # fence-free events on the stream around the dominant kernel's launch
    dom_events = [(TimingEvent(), TimingEvent()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        for j in jobs:
            if j is dom:
                dom_events[k][0].record(stream)
                call(j)
                dom_events[k][1].record(stream)
            else:
                call(j)
    torch.cuda.synchronize()

    roofline = None
    if dom is not None:
        us = 1e3 * sum(a.elapsed_time(b) for a, b in dom_events) / args.steps
        gbs = dom["bytes"] / (us * 1e-6) / 1e9
        kname = KERNEL_NAMES[kernel_key(dom["w"])]
        roofline = {"kernel": kname, "workload": dom["w"].name, "bound": "hbm",
                    "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4),
                    "traffic": traffic_for(dom["w"], dom["bytes"]),
                    "alg_bytes_per_launch": dom["bytes"], "us_per_launch": round(us, 2),
                    "duration_source": "mean of fence-free HIP events around each launch, on the launch "
                                       "stream, in K steps identical to the timed ones",
                    "rocprof": rocprof_duration(dom["w"], kname, dom["bytes"])}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": "one step = every large workload once: " + ", ".join(j["w"].name for j in jobs),
                   "bytes_per_step": step_bytes, "input": "bf16",
                   "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1)},
        "per_recipe_basis": ("algorithmic bytes (one read of the input per pass the method makes, plus every "
                             "byte written) / median event time per call; a second read served by the "
                             "memory-side cache counts as a full read, so these are algorithmic-byte rates, "
                             "not measured HBM traffic"),
        "per_recipe": per,
        "roofline": roofline,
        "copy_reference_GBps": round(copy_gbs, 1),
    }
    # each reference or extra call starts cold, like the step's: 512 MiB read
    # between calls (outside the events) evicts the 256 MB memory-side cache
    # and L2 and leaves clean lines (a write would leave dirty ones for the
    # timed call to write back)
    scratch = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")

    def flush():
        torch.amax(scratch)

    result["torch_cast_reference"] = torch_cast_reference(torch, stream, args.steps, flush)
    if not args.no_extras:
        result["clean_cold"] = time_clean_cold(torch, jobs, call, args.steps, flush)
        result["second_read"] = time_second_read(torch, fq, L, sp, jobs, args.steps, flush)
        result["dequant_requant"] = time_extras(torch, fq, L, sp, jobs, args.steps, flush)
        result["small"] = time_small(torch, fq, L, sp, args.steps, flush)
    del scratch
    if not args.no_cpu_baseline:
        print("bench: timing the oracle on the host", file=sys.stderr, flush=True)
        threads = args.cpu_threads or min(os.cpu_count() or 1, 16)
        result["cpu_baseline"] = cpu_baseline([(j["w"], j["xh"]) for j in jobs], threads, args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
