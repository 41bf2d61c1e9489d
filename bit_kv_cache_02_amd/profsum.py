"""Summaries of rocprofv3 runs of ``bench.py --profile-run`` for the kernels' rooflines.

Reads the CSV outputs of four rocprofv3 runs of the same command (kernel trace with --stats,
then FETCH_SIZE, WRITE_SIZE and the VALUBusy / MfmaUtil busy counters, each in a run of its own)
and the JSON line the kernel-trace run printed, and writes short text summaries: per-kernel
durations, per-leg HBM traffic (each counter scaled by what it reads for the bench's plain
1 GiB copy in the same run) and busy fractions.

    python -m bit_kv_cache_02_amd.profsum --stats DIR --fetch DIR --write DIR --busy DIR \
        --bench-json FILE --out profiles

Each traffic record carries a sha256 of the code of the kernel's sources (comment-only edits
leave it unchanged), so that a reader of the record can tell whether the kernel has changed
since the counters were taken.
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
DECODE_SRC = [os.path.join(CSRC, f) for f in ("kvq_decode.hip", "kvq_attn.h", "kvq_device.h")]
APPEND_SRC = [os.path.join(CSRC, f) for f in ("kvq_append.hip", "kvq_device.h")]
PREFILL_SRC = [os.path.join(CSRC, f) for f in ("kvq_prefill.hip", "kvq_device.h")]
DEQUANT_SRC = [os.path.join(CSRC, f) for f in ("kvq_dequant.hip", "kvq_device.h")]

PROFILE_CMD = "python3 $REPO/bench.py --profile-run"
STATS_CMD = ("cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d $REPO/gpurun_out/prof "
             "-o run -- " + PROFILE_CMD)
FETCH_CMD = ("cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d $REPO/gpurun_out/pmc_fetch "
             "-o run -- " + PROFILE_CMD)
WRITE_CMD = ("cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d $REPO/gpurun_out/pmc_write "
             "-o run -- " + PROFILE_CMD)
BUSY_CMD = ("cd /tmp && rocprofv3 --pmc VALUBusy MfmaUtil --output-format csv -d $REPO/gpurun_out/pmc_busy "
            "-o run -- " + PROFILE_CMD)
SUMMARY_CMD = ("python3 -m bit_kv_cache_02_amd.profsum --stats gpurun_out/prof --fetch gpurun_out/pmc_fetch "
               "--write gpurun_out/pmc_write --busy gpurun_out/pmc_busy --bench-json gpurun_out/prof.json "
               "--out profiles")


def code_sha256(paths):
    """sha256 of the code of the given source files: comment-only edits leave it unchanged."""
    lines = []
    for path in paths:
        for line in open(path, encoding="utf-8"):
            code = line.split("//", 1)[0].rstrip()
            if code:
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


# name: (substring of the kernel's name, bench JSON path of the algorithmic bytes, sources, sha key, what)
LEGS = {
    "decode_step_llama": (r"decode_kernel<0, 8, ", ("algorithmic_bytes", "step"), DECODE_SRC,
                          "decode_source_sha256", "fused decode step (kvq_decode_step: append + decode attention)"),
    "append_prefill": (r"append_kernel<true, 128, 0>", ("prefill_append", "algorithmic_bytes"), APPEND_SRC,
                       "append_source_sha256", "prefill append (kvq_append, Hadamard 128)"),
    "decode_long_ragged": (r"decode_kernel<0, 4, 2, ", ("long_ragged_decode", "algorithmic_bytes"), DECODE_SRC,
                           "decode_source_sha256", "long/ragged decode (kvq_decode_attn, balanced cut)"),
    "decode_mxfp4": (r"decode_kernel<1, ", ("mxfp4_decode", "algorithmic_bytes"), DECODE_SRC,
                     "decode_source_sha256", "MXFP4 decode, f16-tile q.K path (kvq_decode_attn)"),
    "decode_mxfp4_scaled": (r"decode_kernel<2, ", ("mxfp4_decode", "algorithmic_bytes"), DECODE_SRC,
                            "decode_source_sha256", "MXFP4 decode, both contractions on the scaled FP8 x FP4 "
                            "matrix cores (kvq_decode_attn, KVQ_MX_SCALED_MFMA)"),
    "dequant_rotated": (r"dequant_rot_i4_kernel<128>", ("dequant_pages", "algorithmic_bytes"), DEQUANT_SRC,
                        "dequant_source_sha256", "page dequantization rotated back, INT4 Hadamard 128 on the "
                        "matrix cores (kvq_dequant_page)"),
    "dequant_plain": (r"dequant_kernel<false>", ("dequant_pages", "algorithmic_bytes"), DEQUANT_SRC,
                      "dequant_source_sha256", "page dequantization, rotated basis (kvq_dequant_page)"),
    "prefill_attention": (r"prefill_kernel<0>", ("prefill_attention", "kv_bytes_once"), PREFILL_SRC,
                          "prefill_source_sha256", "chunked-prefill attention (kvq_prefill_attn); the "
                          "algorithmic bytes are the resident K/V read once"),
}
COPY_KERNEL = r"copy_kernel"


def _csvs(d, suffix):
    return sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))


def _rows(d, suffix):
    out = []
    for path in _csvs(d, suffix):
        with open(path, newline="") as f:
            out.extend(csv.DictReader(f))
    if not out:
        raise SystemExit(f"no *{suffix} under {d}")
    return out


def _grid(row):
    if "Grid_Size" in row:
        return int(float(row["Grid_Size"]))
    return tuple(int(float(row[k])) for k in ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z") if k in row)


def _launches(rows, pattern):
    """Rows of the kernel matching ``pattern`` with the most launches, restricted to its most
    frequent grid size (a leg runs its launches for ~0.3 s; cache builds and warm-ups differ)."""
    by_name = collections.Counter(r["Kernel_Name"] for r in rows if pattern in r["Kernel_Name"])
    if not by_name:
        return None, []
    name = by_name.most_common(1)[0][0]
    mine = [r for r in rows if r["Kernel_Name"] == name]
    grid = collections.Counter(_grid(r) for r in mine).most_common(1)[0][0]
    return name, [r for r in mine if _grid(r) == grid]


def _short(name, n=80):
    name = name.replace("|", "\\|")
    return name if len(name) <= n else name[:n]


def _counter_per_launch(rows, pattern, counter):
    rows = [r for r in rows if r["Counter_Name"] == counter]
    name, mine = _launches(rows, pattern)
    if not mine:
        return name, 0, None
    # one row per dispatch and counter (the _sum over the device's instances)
    per = collections.defaultdict(float)
    for r in mine:
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    vals = list(per.values())
    return name, len(vals), sum(vals) / len(vals)


def _bench_value(bench, path):
    v = bench
    for k in path:
        if not isinstance(v, dict) or k not in v:
            return None
        v = v[k]
    return v


def kernel_stats(stats_dir):
    rows = _rows(stats_dir, "kernel_stats.csv")
    out = []
    for r in rows:
        out.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                    float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return sorted(out, key=lambda t: -t[5])


def trace_avg_us(stats_dir, pattern):
    """(kernel name, launches, mean duration in us) from the kernel trace, for the leg's launches."""
    rows = _rows(stats_dir, "kernel_trace.csv")
    name, mine = _launches(rows, pattern)
    if not mine:
        return name, 0, None
    d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in mine]
    return name, len(d), sum(d) / len(d)


def write_stats_md(out_dir, stats, bench):
    step = _bench_value(bench, ("step_us",))
    lines = [
        "# decode_step_llama_kernel_stats", "",
        "Per-kernel durations of `bench.py --profile-run` under the rocprofv3 kernel trace ($REPO is the",
        "repository root on the MI355X box), summarized by the second command:", "",
        "```", STATS_CMD, "cd $REPO && " + SUMMARY_CMD, "```", "",
        "The run: 256 eager `kvq_decode_step` launches (clock warm-up), 800 warm-up and 800 timed fused",
        "steps replayed from HIP graphs (llama decode step: batch 32 x 4096, 32 q / 8 kv heads, INT4,",
        "Hadamard 128, 8 layer caches), the bandwidth probes (`copy_kernel`: 1 GiB copies; `read_kernel`:",
        "1 GiB reads and step-sized reads cycling over a 1 GiB buffer; `fold4_kernel`: the 4:1 read:write",
        "stream), the page dequantization (1024 pages x 8 kv heads to fp32, plain and rotated back), the",
        "prefill append (64 x 2048 tokens; Hadamard 128, 64, plain and the two quaternion rotations), the",
        "chunked-prefill attention (32 x 512-token chunks over a 3584-token prefix), the long/ragged",
        "decode (8 sequences of 1K-32K tokens, balanced cut), the tiny decode step and the MXFP4 decode",
        "(64 x 16K, e4m3 queries, f16 tiles and the scaled matrix cores).  Each leg first runs its",
        "launches for ~0.3 s so that clocks settle, which sets most launch counts.", "",
    ]
    if step is not None:
        lines += [f"In the same run bench.py measured the fused step at {step} us per launch (HIP events over",
                  "the timed region).", ""]
    lines += ["| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, pct in stats:
        lines.append(f"| `{_short(name)}` | {calls} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {pct:.1f} |")
    open(os.path.join(out_dir, "decode_step_llama_kernel_stats.md"), "w").write("\n".join(lines) + "\n")


def write_traffic(out_dir, leg, fetch_rows, write_rows, stats_dir, bench):
    pattern, bpath, src, key, what = LEGS[leg]
    _, _, copy_fetch = _counter_per_launch(fetch_rows, COPY_KERNEL, "FETCH_SIZE")
    _, _, copy_write = _counter_per_launch(write_rows, COPY_KERNEL, "WRITE_SIZE")
    name, n_f, fetch = _counter_per_launch(fetch_rows, pattern, "FETCH_SIZE")
    _, n_w, write = _counter_per_launch(write_rows, pattern, "WRITE_SIZE")
    tname, n_t, t_us = trace_avg_us(stats_dir, pattern)
    algo = _bench_value(bench, bpath)
    if fetch is None or write is None or copy_fetch is None or copy_write is None:
        return None
    # the bench's copy moves 1 GiB each way per launch: scale each counter to bytes by that copy
    gib_kib = float(1 << 20)
    fs, ws = gib_kib / copy_fetch, gib_kib / copy_write
    hbm = (fetch * fs + write * ws) * 1024.0
    rec = {
        "kernel": name, "leg": what,
        "workload": _bench_value(bench, (bpath[0], "workload")) if bpath[0] != "algorithmic_bytes"
        else bench.get("config", {}).get("workload"),
        "fetch_kib_per_launch": round(fetch, 1), "write_kib_per_launch": round(write, 1),
        "launches_fetch": n_f, "launches_write": n_w,
        "copy_fetch_kib_per_1GiB": round(copy_fetch, 1), "copy_write_kib_per_1GiB": round(copy_write, 1),
        "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
        "hbm_bytes_per_launch": int(round(hbm)),
        "algorithmic_bytes": algo,
        "ratio_to_algorithmic": round(hbm / algo, 4) if algo else None,
        "kernel_trace_launches": n_t,
        "kernel_trace_avg_us": round(t_us, 3) if t_us is not None else None,
        key: code_sha256(src),
        "commands": [STATS_CMD, FETCH_CMD, WRITE_CMD, "cd $REPO && " + SUMMARY_CMD],
    }
    json.dump(rec, open(os.path.join(out_dir, f"{leg}_traffic.json"), "w"), indent=1)
    lines = [
        f"# {leg}_traffic", "",
        f"HBM traffic of the {what}.", "",
        "Two rocprofv3 counter runs of the same command (FETCH_SIZE, then WRITE_SIZE), each counter scaled",
        "by what it reads for the bench's plain copy of 1 GiB (reads 1 GiB, writes 1 GiB) in the same run;",
        "the kernel-trace run gives the average duration of the same launches (the kernel's most frequent",
        "grid size, i.e. the leg's own launches).", "",
        "```", *rec["commands"], "```", "",
        "| quantity | value |", "|---|---|",
        f"| kernel | `{_short(name, 120)}` |",
        f"| launches counted (fetch / write / trace) | {n_f} / {n_w} / {n_t} |",
        f"| FETCH_SIZE per launch (KiB, raw) | {fetch:.1f} |",
        f"| WRITE_SIZE per launch (KiB, raw) | {write:.1f} |",
        f"| FETCH_SIZE / WRITE_SIZE per 1 GiB copy (KiB, raw) | {copy_fetch:.1f} / {copy_write:.1f} |",
        f"| scale factors fetch / write | {fs:.4f} / {ws:.4f} |",
        f"| HBM bytes per launch (scaled) | {hbm / 1e6:.2f} MB |",
    ]
    if algo:
        lines += [f"| algorithmic bytes per launch | {algo / 1e6:.2f} MB |",
                  f"| ratio | {hbm / algo:.4f} |"]
    if t_us is not None:
        lines += [f"| kernel-trace average duration | {t_us:.2f} us |"]
        if algo:
            lines += [f"| algorithmic GB/s at that duration | {algo / t_us / 1e3:.1f} |",
                      f"| fraction of the 8 TB/s HBM peak | {algo / t_us / 8e6:.4f} |"]
    open(os.path.join(out_dir, f"{leg}_traffic.md"), "w").write("\n".join(lines) + "\n")
    return rec


def write_busy(out_dir, busy_dir):
    rows = _rows(busy_dir, "counter_collection.csv")
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in rows:
        acc[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    table = []
    for name, cs in acc.items():
        n = max(len(v) for v in cs.values())
        vb = cs.get("VALUBusy", [])
        mu = cs.get("MfmaUtil", [])
        table.append((name, n, sum(vb) / len(vb) if vb else float("nan"), sum(mu) / len(mu) if mu else float("nan")))
    table.sort(key=lambda t: -t[1])
    lines = [
        "# kernel_busy", "",
        "VALU and matrix-core busy fractions per kernel (rocprofv3 derived counters, averaged over the",
        "launches of `bench.py --profile-run`; the workloads are those of the kernel-stats summary):", "",
        "```", BUSY_CMD, "cd $REPO && " + SUMMARY_CMD, "```", "",
        "VALUBusy = 100 * SQ_ACTIVE_INST_VALU / CU_NUM / GRBM_GUI_ACTIVE;",
        "MfmaUtil = 100 * SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * SIMD_NUM).", "",
        "| kernel | launches | VALUBusy % | MfmaUtil % |", "|---|---|---|---|",
    ]
    for name, n, vb, mu in table:
        if name.startswith(("void at::", "at::", "void (anonymous")):
            continue
        lines.append(f"| `{_short(name)}` | {n} | {vb:.1f} | {mu:.1f} |")
    open(os.path.join(out_dir, "kernel_busy.md"), "w").write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--stats", required=True, help="rocprofv3 --kernel-trace --stats output directory")
    ap.add_argument("--fetch", help="rocprofv3 --pmc FETCH_SIZE output directory")
    ap.add_argument("--write", help="rocprofv3 --pmc WRITE_SIZE output directory")
    ap.add_argument("--busy", help="rocprofv3 --pmc VALUBusy MfmaUtil output directory")
    ap.add_argument("--bench-json", required=True, help="file whose last line is bench.py's JSON line")
    ap.add_argument("--out", default="profiles")
    args = ap.parse_args()
    bench = json.loads(open(args.bench_json).read().strip().splitlines()[-1])
    os.makedirs(args.out, exist_ok=True)
    write_stats_md(args.out, kernel_stats(args.stats), bench)
    if args.fetch and args.write:
        fetch_rows = _rows(args.fetch, "counter_collection.csv")
        write_rows = _rows(args.write, "counter_collection.csv")
        for leg in LEGS:
            rec = write_traffic(args.out, leg, fetch_rows, write_rows, args.stats, bench)
            print(leg, "->", None if rec is None else (rec["kernel"], rec["ratio_to_algorithmic"],
                                                       rec["kernel_trace_avg_us"]))
    if args.busy:
        write_busy(args.out, args.busy)


if __name__ == "__main__":
    main()
