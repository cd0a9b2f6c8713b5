"""The profile summariser's arithmetic on hand-made rocprofv3 files: counter
rows summed per dispatch, the copy calibration, and the JSON that bench.py
reads back (only while the kernel sources are the measured ones)."""
import csv
import json
import os

from persistent_megakernel_decode_02_amd import profile_summary as ps

HDR = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
       "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
       "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HDR)
        for disp, name, counter, value in rows:
            w.writerow([disp, disp, "Agent 1", 1, 1, 1, 1, 1, name, 512, 0, 0, 0, 0, 0, counter, value, 0, 1])


def _bench(path, alg):
    with open(path, "w") as f:
        f.write("[bench] noise\n")
        f.write(json.dumps({"roofline": {"algorithmic_bytes_per_launch": alg, "kernel_ms_mean": 1.0},
                            "config": {"decode_tokens_per_step": 4, "n_wg": 8, "n_chunks": 1},
                            "us_per_token": 250.0}) + "\n")


def test_traffic_summary(tmp_path):
    t = str(tmp_path)
    # the megakernel's FETCH_SIZE arrives in two rows per dispatch (summed)
    _counters(t + "/f", [(1, "mkd_reset", "FETCH_SIZE", 5), (2, "mkd_megakernel", "FETCH_SIZE", 300),
                         (2, "mkd_megakernel", "FETCH_SIZE", 200), (4, "mkd_megakernel", "FETCH_SIZE", 500)])
    _counters(t + "/w", [(2, "mkd_megakernel", "WRITE_SIZE", 40), (4, "mkd_megakernel", "WRITE_SIZE", 60)])
    # a 1 MiB copy: FETCH_SIZE reports half of its reads, WRITE_SIZE all of its writes
    _counters(t + "/cf", [(1, "fill", "FETCH_SIZE", 3), (2, "copy", "FETCH_SIZE", 512)])
    _counters(t + "/cw", [(1, "fill", "WRITE_SIZE", 1024), (2, "copy", "WRITE_SIZE", 1024)])
    _bench(t + "/b.json", 1.0e6)
    out = t + "/prof/k_w_traffic.md"
    ps.main(["traffic", "--kernel", "mkd_megakernel", "--workload", "w", "--fetch", t + "/f", "--write", t + "/w",
             "--calib-fetch", t + "/cf", "--calib-write", t + "/cw", "--calib-bytes", str(1 << 20),
             "--bench", t + "/b.json", "--command", "rocprofv3 ...", "--out", out])
    d = json.load(open(t + "/prof/k_w_traffic.json"))
    assert abs(d["fetch_scale"] - 2.0) < 1e-12 and abs(d["write_scale"] - 1.0) < 1e-12
    assert abs(d["fetch_bytes_per_launch"] - 500 * 1024 * 2.0) < 1e-6     # (300+200, 500) per dispatch
    assert abs(d["write_bytes_per_launch"] - 50 * 1024) < 1e-6
    assert d["hbm_bytes_per_launch"] == d["fetch_bytes_per_launch"] + d["write_bytes_per_launch"]
    assert d["kernel_sha256_16"] == ps.kernel_digest()
    text = open(out).read()
    assert "rocprofv3 ..." in text and "measured / algorithmic" in text


def test_kernel_trace_summary(tmp_path):
    t = str(tmp_path)
    os.makedirs(t + "/s")
    with open(t + "/s/run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow(["mkd_megakernel", 3, 300e6, 100e6, 99.0, 99e6, 101e6, 1e6])
        w.writerow(["mkd_reset", 3, 9e3, 3e3, 0.0, 2e3, 4e3, 1e3])
        w.writerow(["other", 1, 1e3, 1e3, 0.0, 1e3, 1e3, 0])
    _bench(t + "/b.json", 1.0e6)
    out = t + "/k_w_kernel_trace.md"
    ps.main(["kernel-trace", "--kernel", "mkd_megakernel", "--workload", "w", "--stats", t + "/s",
             "--bench", t + "/b.json", "--command", "rocprofv3 --kernel-trace --stats ...", "--out", out])
    text = open(out).read()
    assert "| mkd_megakernel | 3 | 100.000 | 99.000 | 101.000 |" in text
    assert "| mkd_reset | 3 | 0.0030 |" in text and "other" not in text
