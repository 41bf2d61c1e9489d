"""The rocprofv3 summarizer on small hand-made CSVs (host logic only)."""
import csv
import json
import os

from bit_kv_cache_02_amd import profsum

TRACE_HDR = ["Kind", "Agent_Id", "Queue_Id", "Kernel_Id", "Kernel_Name", "Correlation_Id", "Start_Timestamp",
             "End_Timestamp", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
PMC_HDR = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
           "Kernel_Id", "Kernel_Name", "Workgroup_Size", "Counter_Name", "Counter_Value", "Start_Timestamp",
           "End_Timestamp"]
STEP = "void kvq::decode_kernel<0, 8, 3, 1>(kvq::DecodeParams)"
COPY = "kvq::copy_kernel(unsigned int __vector(4) const*, unsigned int __vector(4)*, long, long)"


def _write(path, hdr, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(hdr)
        w.writerows(rows)


def test_traffic_and_trace_average(tmp_path):
    d = str(tmp_path)
    # trace: 3 step launches of 20 us at the leg's grid, 1 of 100 us at another grid (ignored)
    trace = [["KERNEL_DISPATCH", 1, 1, 5, STEP, i, 1000 * i, 1000 * i + 20000, 256, 1, 1] for i in range(3)]
    trace.append(["KERNEL_DISPATCH", 1, 1, 5, STEP, 9, 0, 100000, 512, 1, 1])
    _write(f"{d}/prof/h/1/run_kernel_trace.csv", TRACE_HDR, trace)
    _write(f"{d}/prof/h/1/run_kernel_stats.csv",
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
           [[STEP, 4, 160000, 40000, 100.0, 20000, 100000, 1]])
    # counters: copy reads 2^19 KiB and writes 2^20 KiB per 1 GiB; two step dispatches, each
    # counter split over two rows (instances) that are summed per dispatch
    fetch = [[1, 1, 1, 1, 1, 1, 512, 6, COPY, 512, "FETCH_SIZE", 2 ** 19, 0, 1]]
    write = [[1, 1, 1, 1, 1, 1, 512, 6, COPY, 512, "WRITE_SIZE", 2 ** 20, 0, 1]]
    for disp in (2, 3):
        fetch += [[disp, disp, 1, 1, 1, 1, 256, 5, STEP, 512, "FETCH_SIZE", 25.0, 0, 1]] * 2
        write += [[disp, disp, 1, 1, 1, 1, 256, 5, STEP, 512, "WRITE_SIZE", 10.0, 0, 1]] * 2
    _write(f"{d}/f/run_counter_collection.csv", PMC_HDR, fetch)
    _write(f"{d}/w/run_counter_collection.csv", PMC_HDR, write)
    bench = {"algorithmic_bytes": {"step": 100 * 1024}, "step_us": 21.0, "config": {"workload": "w"}}
    out = f"{d}/out"
    os.makedirs(out)
    fr = profsum._rows(f"{d}/f", "counter_collection.csv")
    wr = profsum._rows(f"{d}/w", "counter_collection.csv")
    rec = profsum.write_traffic(out, "decode_step_llama", fr, wr, f"{d}/prof", bench)
    assert rec["fetch_kib_per_launch"] == 50.0 and rec["write_kib_per_launch"] == 20.0
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["hbm_bytes_per_launch"] == (2 * 50 + 20) * 1024
    assert rec["ratio_to_algorithmic"] == 1.2
    assert rec["kernel_trace_launches"] == 3 and rec["kernel_trace_avg_us"] == 20.0
    assert rec["decode_source_sha256"] == profsum.code_sha256(profsum.DECODE_SRC)
    assert json.load(open(f"{out}/decode_step_llama_traffic.json"))["kernel"] == STEP
    profsum.write_stats_md(out, profsum.kernel_stats(f"{d}/prof"), bench)
    md = open(f"{out}/decode_step_llama_kernel_stats.md").read()
    assert "| 4 | 40.00 | 20.00 | 100.00 | 100.0 |" in md


def test_code_sha_ignores_comments(tmp_path):
    a, b = tmp_path / "a.hip", tmp_path / "b.hip"
    a.write_text("int x = 1;  // one\n// note\nint y;\n")
    b.write_text("int x = 1;\nint y;  // other\n")
    assert profsum.code_sha256([str(a)]) == profsum.code_sha256([str(b)])
