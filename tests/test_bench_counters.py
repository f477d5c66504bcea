"""Host logic of the bench's counter bookkeeping: the per-kernel reduction of a
rocprofv3 --pmc run (--summarize-sq) and the rule that the headline traffic
record is used only while it was taken on the current kernel source."""
import csv
import hashlib
import json
import os

import bench

K1 = "void moe::ffn_stage1<0, true, 128, 1, 2>(moe::FfnArgs, unsigned short*)"
K2 = "void moe::align_kernel<2, 0, 0>(moe::AlignArgs)"
PROBE = "copy_probe_kernel(float4 const*, float4*, long)"
OTHER = "void at::native::vectorized_elementwise_kernel<4>(int)"


def write_run(d, rows, trace=None):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)
    if trace is not None:
        with open(os.path.join(d, "run_kernel_trace.csv"), "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
            w.writerows(trace)


def test_summarize_sq_sums_instances_and_takes_medians(tmp_path):
    rows = []
    # three dispatches of the GEMM: GRBM_GUI_ACTIVE has one instance per XCD
    for did, per_xcd, mfma in (("1", 1000, 10), ("2", 3000, 30), ("5", 2000, 20)):
        rows += [[did, K1, "GRBM_GUI_ACTIVE", per_xcd] for _ in range(bench.NUM_XCD)]
        rows += [[did, K1, "SQ_INSTS_MFMA", mfma / 4] for _ in range(4)]    # four instances
    rows += [["3", K2, "SQ_INSTS_MFMA", 0]]
    rows += [["4", PROBE, "FETCH_SIZE", 7.0], ["4", PROBE, "FETCH_SIZE", 5.0]]
    rows += [["6", OTHER, "SQ_INSTS_MFMA", 99]]                              # not the library's
    trace = [["1", K1, 1000, 3000], ["2", K1, 1000, 7000], ["5", K1, 0, 4000]]
    d = str(tmp_path / "pmc")
    write_run(d, rows, trace)
    out = str(tmp_path / "o.json")
    bench.summarize_sq(d, out)
    got = json.load(open(out))
    assert set(got) == {"moe::ffn_stage1<0, true, 128, 1, 2>", "moe::align_kernel<2, 0, 0>", "copy_probe_kernel"}
    g = got["moe::ffn_stage1<0, true, 128, 1, 2>"]
    assert g["dispatches"] == 3
    assert g["GRBM_GUI_ACTIVE"] == 2000 * bench.NUM_XCD          # median of the summed dispatches
    assert g["SQ_INSTS_MFMA"] == 20
    assert g["us_median"] == 4.0                                # durations 2, 6, 4 us
    assert sorted(map(tuple, g["per_dispatch_us_cycles"])) == [(2.0, 1000.0), (4.0, 2000.0), (6.0, 3000.0)]
    assert got["copy_probe_kernel"]["FETCH_SIZE"] == 12.0
    assert "us_median" not in got["copy_probe_kernel"]          # no trace row for it


def test_summarize_sq_without_trace(tmp_path):
    d = str(tmp_path / "pmc")
    write_run(d, [["1", K1, "FETCH_SIZE", 4], ["1", K1, "FETCH_SIZE", 6]])
    out = str(tmp_path / "o.json")
    bench.summarize_sq(d, out)
    g = json.load(open(out))["moe::ffn_stage1<0, true, 128, 1, 2>"]
    assert g == {"dispatches": 1, "FETCH_SIZE": 10.0}


def test_traffic_record_only_on_its_kernel_source(tmp_path, monkeypatch):
    src = os.path.join(bench.ROOT, "routing_align_sort_amd", "csrc", "ffn_mfma.hip")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    path = tmp_path / "ffn_stage1_prefill_bf16_B64_counters.json"
    assert bench.measured_traffic("prefill_bf16", 64) is None          # no record
    path.write_text(json.dumps({"hbm_bytes_per_launch": 123, "kernel_source_sha256": digest}))
    assert bench.measured_traffic("prefill_bf16", 64) == 123
    path.write_text(json.dumps({"hbm_bytes_per_launch": 123, "kernel_source_sha256": "0" * 64}))
    assert bench.measured_traffic("prefill_bf16", 64) is None          # taken on another source

