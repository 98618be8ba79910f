"""The rocprofv3 summaries that feed `profiles/` read dispatches in the order
bench.py launches them, and derive clock and MFMA busy from the counters."""
import csv

import bench
import hidden_decoding_stream_amd.profile_summary as PS


def test_orders_match_bench():
    assert PS.ORDER == bench.PROFILE_PREFILL_ORDER and PS.REPS == bench.PROFILE_PREFILL_REPS
    assert PS.DATA_ORDER == bench.PREFILL_DATA_ORDER and PS.DATA_REPS == bench.PREFILL_DATA_REPS


def test_data_summary_from_counters(tmp_path):
    # one warm-up dispatch, then DATA_REPS per data set; data set i runs (i + 1) ms at 1.5 GHz with
    # the matrix core busy (50 + 10 i)% of SIMD cycles and every CU busy
    n = 1 + len(PS.DATA_ORDER) * PS.DATA_REPS
    with open(tmp_path / "x_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        for did in range(n):
            i = max(0, (did - 1) // PS.DATA_REPS)
            ns = (i + 1) * 1_000_000
            gx = 1.5 * ns                                      # one XCD's active cycles
            vals = {"GRBM_GUI_ACTIVE": gx * PS.XCDS, "SQ_VALU_MFMA_BUSY_CYCLES": (0.5 + 0.1 * i) * gx * PS.SIMDS,
                    "SQ_BUSY_CU_CYCLES": gx * PS.CUS}
            for k, v in vals.items():
                w.writerow([did, "void sfa::attn_fwd128_kernel<1>(P)", k, v, 10 ** 9 * did, 10 ** 9 * did + ns])
    out = PS.data([tmp_path]).splitlines()
    for i, name in enumerate(PS.DATA_ORDER):
        row = next(r.split() for r in out if r.startswith(name + " "))
        assert float(row[1]) == (i + 1) * 1000.0
        assert float(row[3]) == 1.5
        assert abs(float(row[4]) - (50 + 10 * i)) < 1e-9
        assert float(row[5]) == 100.0
