"""CPU test of bench.py's profile summariser on synthetic rocprofv3 outputs:
segment launches are attributed to arms by the launch schedule the profiled
bench run printed, and the counters are scaled by the calibration copy."""
import csv
import json
import os

import bench

KT_COLS = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
PMC_COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
SEG = "void skv::(anonymous namespace)::seg_mfma_kernel<2, false, 4, false, 4>(skv::SegParams)"
RED = "void skv::(anonymous namespace)::reduce_kernel<false, 128>(float const*)"
PLAN = "void skv::(anonymous namespace)::plan_kernel(int const*)"


def _write(path, cols, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _line(schedule, kvb=1_000_000):
    return {"metric": "m", "value": 1.0, "us_per_call": 10.0,
            "config": {"workload": "wl_x: note"},
            "roofline": {"kernel_source_hash": "abc", "algorithmic_bytes_per_launch": kvb},
            "segment_launch_schedule": schedule}


def test_summarize_attributes_arms_and_scales_counters(tmp_path):
    d = tmp_path / "p_wl_x"
    c = tmp_path / "p_copy"
    # trace: planned launches take 100 us, fixed 300 us, graph 90 us
    sched = [["precondition", "planned", 3], ["timed", "planned", 1], ["timed", "fixed", 1],
             ["timed", "graph", 1], ["timed", "fixed", 1], ["timed", "graph", 1],
             ["timed", "planned", 1]]
    dur = {"planned": 100_000, "fixed": 300_000, "graph": 90_000}
    rows, t, i = [], 1000, 0
    for ph, arm, n in sched:
        for _ in range(n):
            if arm == "planned":
                rows.append(dict(Kind="K", Dispatch_Id=i, Kernel_Name=PLAN, Start_Timestamp=t,
                                 End_Timestamp=t + 5000))
                i += 1
                t += 6000
            rows.append(dict(Kind="K", Dispatch_Id=i, Kernel_Name=SEG, Start_Timestamp=t,
                             End_Timestamp=t + dur[arm]))
            i += 1
            t += dur[arm] + 1000
            rows.append(dict(Kind="K", Dispatch_Id=i, Kernel_Name=RED, Start_Timestamp=t,
                             End_Timestamp=t + 4000))
            i += 1
            t += 5000
    _write(str(d / "trace" / "trace_kernel_trace.csv"), KT_COLS, rows)
    (d / "trace.json").write_text("noise\n" + json.dumps(_line(sched)) + "\n")
    # counters: planned segment dispatches read 500 KiB raw, fixed ones 999
    fsched = [["timed", "planned", 1], ["timed", "fixed", 1], ["timed", "planned", 1]]
    for kind, val in (("fetch", {"planned": 500.0, "fixed": 999.0}),
                      ("write", {"planned": 2.0, "fixed": 7.0})):
        prow, k = [], 0
        for ph, arm, n in fsched:
            prow.append(dict(Dispatch_Id=k, Kernel_Name=SEG, Counter_Name=kind,
                             Counter_Value=val[arm]))
            prow.append(dict(Dispatch_Id=k + 1, Kernel_Name=RED, Counter_Name=kind,
                             Counter_Value=1.0))
            k += 2
        _write(str(d / kind / f"{kind}_counter_collection.csv"), PMC_COLS, prow)
        (d / f"{kind}.json").write_text(json.dumps(_line(fsched)) + "\n")
    # calibration copy: FETCH_SIZE reads half the true KiB, WRITE_SIZE all of it
    _write(str(c / "fetch" / "cf_counter_collection.csv"), PMC_COLS,
           [dict(Dispatch_Id=0, Kernel_Name="__amd_rocclr_copyBuffer", Counter_Name="F",
                 Counter_Value=524288.0)])
    _write(str(c / "write" / "cw_counter_collection.csv"), PMC_COLS,
           [dict(Dispatch_Id=0, Kernel_Name="__amd_rocclr_copyBuffer", Counter_Name="W",
                 Counter_Value=1048576.0)])
    out = tmp_path / "profiles"
    traffic = bench.summarize(str(d), out_dir=str(out))
    e = traffic["wl_x"]
    assert e["read_bytes"] == 500 * 1024 * 2 and e["write_bytes"] == 2 * 1024
    assert e["hbm_bytes_per_launch"] == 500 * 1024 * 2 + 2 * 1024
    md = (out / "wl_x_kernel_trace.md").read_text()
    assert "| timed | planned | 2 | 100.0 |" in md
    assert "| timed | fixed | 2 | 300.0 |" in md
    assert "| timed | graph | 2 | 90.0 |" in md
    assert "| precondition | planned | 3 | 100.0 |" in md
    assert json.loads((out / "segment_traffic.json").read_text())["wl_x"]["kernel"] == \
        "seg_mfma_kernel<2, false, 4, false, 4>"
