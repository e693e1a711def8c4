"""Summaries of rocprofv3 runs of bench.py, for the profiles/ directory.

  python -m fp8_fp4_tensor_amd.profsum trace  STATS_CSV TRACE_CSV OUT.md "COMMAND"
      per-kernel durations (calls, mean, min, max) from a --kernel-trace --stats run,
      and the dispatches of the fastest complete step in order.

  python -m fp8_fp4_tensor_amd.profsum traffic FETCH_CSV WRITE_CSV KERNEL WORKLOAD ROWSxCOLS OUT.json "COMMANDS"
      HBM bytes per launch of KERNEL from two --pmc runs (FETCH_SIZE, then
      WRITE_SIZE; both in KiB per dispatch). Each counter is scaled by what it
      reads for the plain 256 MiB device copy that bench.py runs first
      (256 MiB read and 256 MiB written), so the result is in true bytes.
      The file records a hash of the kernel's sources; bench.py reports the
      traffic only while the sources are unchanged.

  python -m fp8_fp4_tensor_amd.profsum traffic-all FETCH_CSV WRITE_CSV OUT.md "COMMANDS"
      HBM bytes per dispatch of every kernel in the two --pmc runs, scaled
      like `traffic`.

  python -m fp8_fp4_tensor_amd.profsum insts OUT.md "COMMAND" WORKLOAD=CSV ...
      instruction counts per element from --pmc runs of bench.py --only
      WORKLOAD (SQ_INSTS_VALU, SQ_INSTS_SALU, SQ_INSTS_LDS, SQ_INSTS_VMEM_RD,
      SQ_INSTS_VMEM_WR, SQ_WAVES; wave-level counts summed over the chip).
      A wave instruction does the work of 64 lanes, so VALU x 64 / elements
      is the vector lane-operations per element.
"""
import collections
import csv
import json
import os
import sys

COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 256 << 20


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def short_name(name):
    """Kernel name without namespaces, parameter list or return type."""
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0].replace("fq::", "")


def trace(stats_csv, trace_csv, out_md, command):
    stats = _rows(stats_csv)
    lines = ["# Kernel durations (rocprofv3 --kernel-trace --stats)", "", f"Command: `{command}`", "",
             "| kernel | calls | mean us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in stats:
        name = r["Name"]
        short = short_name(name)
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    rows = sorted(_rows(trace_csv), key=lambda r: int(r["Start_Timestamp"]))
    step = fastest_step(rows)
    if step:
        span = (int(step[-1]["End_Timestamp"]) - int(step[0]["Start_Timestamp"])) / 1e3
        lines += ["", f"The fastest complete step of the library's kernels ({span:.1f} us from the first "
                  "start to the last end; a step of the timed region, where no event sits between calls), "
                  "dispatches in order with the gap after the previous kernel:", "",
                  "| kernel | grid (work-items) | us | gap us |", "|---|---|---|---|"]
        prev = None
        for r in step:
            s, e = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            gap = "" if prev is None else f"{(s - prev) / 1e3:.2f}"
            lines.append(f"| `{short_name(r['Kernel_Name'])}` | {r.get('Grid_Size_X', '')} | {(e - s) / 1e3:.2f} | {gap} |")
            prev = e
    # the end of the run in dispatch order: durations and gaps
    lines += ["", "Last dispatches in order (duration, gap after the previous kernel):", "",
              "| kernel | us | gap us |", "|---|---|---|"]
    prev = None
    for r in rows[-16:]:
        s, e = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        short = short_name(r["Kernel_Name"])
        gap = "" if prev is None else f"{(s - prev) / 1e3:.2f}"
        lines.append(f"| `{short}` | {(e - s) / 1e3:.2f} | {gap} |")
        prev = e
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    # the same mean durations as JSON, each with the hash of its kernel's
    # sources (bench.py quotes a duration only while they are unchanged)
    kernels = {}
    for r in stats:
        short = short_name(r["Name"])
        family = short.split("<")[0]
        entry = {"calls": int(r["Calls"]), "mean_us": round(float(r["AverageNs"]) / 1e3, 3)}
        if family in KERNEL_SOURCES:
            entry["source_hash"] = source_hash(KERNEL_SOURCES[family])
        kernels[short] = entry
    with open(os.path.splitext(out_md)[0] + ".json", "w") as f:
        json.dump({"command": command, "kernels": kernels}, f, indent=1)
        f.write("\n")


def fastest_step(rows, last="k_nvfp4_16x16"):
    """The library's dispatches of one bench step, from a time-ordered kernel
    trace: the library's kernels (names in namespace fq) are cut into steps
    after each dispatch of `last` (the step's final kernel); of the steps
    with the most common length, the one with the shortest span from its
    first start to its last end. Empty if `last` never ran."""
    ours = [r for r in rows if "fq::" in r["Kernel_Name"]]
    steps, cur = [], []
    for r in ours:
        cur.append(r)
        if short_name(r["Kernel_Name"]).split("<")[0] == last:
            steps.append(cur)
            cur = []
    if not steps:
        return []
    n = collections.Counter(len(st) for st in steps).most_common(1)[0][0]
    full = [st for st in steps if len(st) == n]
    return min(full, key=lambda st: int(st[-1]["End_Timestamp"]) - int(st[0]["Start_Timestamp"]))


def _mean_counter(rows, kernel_substr, counter):
    vals = [float(r["Counter_Value"]) for r in rows
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    # several rows per dispatch (one per counter instance) are summed per dispatch
    per = collections.defaultdict(float)
    for r in rows:
        if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for {kernel_substr}")
    return sum(per.values()) / len(per), len(per), len(vals)


def source_hash(files):
    import hashlib
    h = hashlib.sha256()
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    for f in files:
        with open(os.path.join(here, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {"k_block_128x128": ["k_block.hip", "codec.hpp"], "k_block_1x128": ["k_block.hip", "codec.hpp"],
                  "k_mx_bf16": ["k_mx.hip", "codec.hpp"], "k_cast_tensor": ["k_tensor.hip", "codec.hpp"],
                  "k_cast_delayed": ["k_tensor.hip", "codec.hpp"],
                  "k_nvfp4_1x16": ["k_nvfp4.hip", "k_tensor.hip", "codec.hpp"],
                  "k_nvfp4_16x16": ["k_nvfp4.hip", "k_tensor.hip", "codec.hpp"]}


def traffic(fetch_csv, write_csv, kernel, workload, shape, out_json, commands):
    fr, wr = _rows(fetch_csv), _rows(write_csv)
    f_k, nf, _ = _mean_counter(fr, kernel, "FETCH_SIZE")
    w_k, nw, _ = _mean_counter(wr, kernel, "WRITE_SIZE")
    f_c, _, _ = _mean_counter(fr, COPY_KERNEL, "FETCH_SIZE")
    w_c, _, _ = _mean_counter(wr, COPY_KERNEL, "WRITE_SIZE")
    f_scale = COPY_BYTES / (f_c * 1024.0)
    w_scale = COPY_BYTES / (w_c * 1024.0)
    read_b = f_k * 1024.0 * f_scale
    write_b = w_k * 1024.0 * w_scale
    family = kernel.split("<")[0].split("(")[0]
    out = {"kernel": kernel, "workload": workload, "shape": shape, "dispatches": {"fetch": nf, "write": nw},
           "fetch_kib_per_dispatch": f_k, "write_kib_per_dispatch": w_k,
           "copy_fetch_kib": f_c, "copy_write_kib": w_c,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_read_bytes_per_launch": int(read_b), "hbm_write_bytes_per_launch": int(write_b),
           "hbm_bytes_per_launch": int(read_b + write_b),
           "source_hash": source_hash(KERNEL_SOURCES[family]), "commands": commands}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def traffic_all(fetch_csv, write_csv, out_md, commands):
    fr, wr = _per_kernel_counters(_rows(fetch_csv)), _per_kernel_counters(_rows(write_csv))
    f_scale = COPY_BYTES / (fr[COPY_KERNEL]["FETCH_SIZE"] * 1024.0)
    w_scale = COPY_BYTES / (wr[COPY_KERNEL]["WRITE_SIZE"] * 1024.0)
    lines = ["# HBM traffic per dispatch, every kernel (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
             f"Commands: `{commands}`", "",
             f"Counters scaled by what they read for the plain 256 MiB device copy: FETCH_SIZE x {f_scale:.3f}, "
             f"WRITE_SIZE x {w_scale:.3f}. A kernel name that serves several workloads shows their mean.", "",
             "| kernel | dispatches | read MB | written MB |", "|---|---|---|---|"]
    for k in sorted(set(fr) & set(wr)):
        if not k.startswith("k_"):
            continue
        lines.append(f"| `{k}` | {fr[k]['dispatches']} | {fr[k]['FETCH_SIZE'] * 1024 * f_scale / 1e6:.2f} | "
                     f"{wr[k]['WRITE_SIZE'] * 1024 * w_scale / 1e6:.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


INST_COUNTERS = ["SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR",
                 "SQ_WAVES"]


def _per_kernel_counters(rows):
    """{short kernel name: {counter: mean per dispatch}} (instances summed per dispatch)."""
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in rows:
        acc[(r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = short_name(r["Kernel_Name"])
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for d, cs in acc.items():
        for c, v in cs.items():
            out[names[d]][c].append(v)
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} | {"dispatches": len(next(iter(cs.values())))}
            for k, cs in out.items()}


def insts(out_md, command, *pairs):
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from fp8_fp4_tensor_amd import workloads as W
    lines = ["# Instructions per element (rocprofv3 --pmc, SQ counters)", "",
             f"Command (per workload): `{command}`", "",
             "Wave-level instruction counts summed over the chip, per dispatch; a VALU",
             "instruction covers 64 lanes, so VALU x 64 / elements = vector lane-operations",
             "per element of the input tensor. (256 CUs x 64 lanes x 2.4 GHz = 39.3 T",
             "lane-ops/s; at 6.4 TB/s and 3 bytes per element the budget is ~18.)", "",
             "| workload | kernel | dispatches | VALU lane-ops / elem | SALU / 1K elem | LDS / 1K elem "
             "| VMEM rd / 1K elem | VMEM wr / 1K elem | waves |",
             "|---|---|---|---|---|---|---|---|---|"]
    for pair in pairs:
        wname, csv_path = pair.split("=", 1)
        w = W.BY_NAME[wname]
        n = w.shape[0] * w.shape[1]
        for k, cs in sorted(_per_kernel_counters(_rows(csv_path)).items()):
            if not k.startswith("k_"):
                continue
            g = cs.get
            lines.append(f"| {wname} | `{k}` | {cs['dispatches']} | {g('SQ_INSTS_VALU', 0) * 64 / n:.2f} | "
                         f"{g('SQ_INSTS_SALU', 0) * 1e3 / n:.2f} | {g('SQ_INSTS_LDS', 0) * 1e3 / n:.2f} | "
                         f"{g('SQ_INSTS_VMEM_RD', 0) * 1e3 / n:.2f} | {g('SQ_INSTS_VMEM_WR', 0) * 1e3 / n:.2f} | "
                         f"{g('SQ_WAVES', 0):.0f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        trace(*sys.argv[2:6])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:9])
    elif sys.argv[1] == "traffic-all":
        traffic_all(*sys.argv[2:6])
    elif sys.argv[1] == "insts":
        insts(*sys.argv[2:])
    else:
        raise SystemExit(__doc__)
