"""bench_counters.py on hand-made rocprofv3 CSVs (no GPU): the marker
split, init kernels counted with their case, the copy calibration, and the
per-kernel figures bench.py's roofline reads."""
import csv
import json
import os

import bench_counters as bc

HDR = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
       "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size",
       "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value",
       "Start_Timestamp", "End_Timestamp"]
FILL = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float> >()"
GEMM_A = "void baim::addmm_kernel<baim::Tile<128, 128, 32, 2, 4, 1, 2> >(baim::AddmmArgs)"
INIT = "void baim::conv_init_kernel(float*, float const*)"
CONV = "void baim::conv_window_kernel<baim::WinCfg<3, 3> >(baim::WinArgs)"


def write(path, dispatches):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HDR)
        for i, (name, counters) in enumerate(dispatches, 1):
            for cn, cv in counters.items():
                w.writerow([i, i, "Agent 1", 1, 1, 1, 64, 1, name, 64, 0, 0, 8, 0, 8, cn, cv, 0, 1])


def trace(counter_of):
    # set-up launches (one per case), marker, case 0 x2, marker, case 1 x2 (init + conv), marker
    d = [("__amd_rocclr_copyBuffer", counter_of("copy")), (GEMM_A, counter_of("a")),
         (INIT, counter_of("init")), (CONV, counter_of("conv")), (FILL, counter_of("fill"))]
    d += [(GEMM_A, counter_of("a"))] * 2 + [(FILL, counter_of("fill"))]
    d += [(INIT, counter_of("init")), (CONV, counter_of("conv"))] * 2 + [(FILL, counter_of("fill"))]
    return d


def test_counters_split_scale_and_average(tmp_path):
    d = str(tmp_path)
    fetch = {"a": 1000.0, "init": 10.0, "conv": 300.0, "fill": 1.0, "copy": 0.0}
    write_ = {"a": 500.0, "init": 20.0, "conv": 100.0, "fill": 1.0, "copy": 0.0}
    busy = {"a": 800.0, "init": 5.0, "conv": 600.0, "fill": 0.0, "copy": 0.0}
    write(os.path.join(d, "f_counter_collection.csv"), trace(lambda k: {"FETCH_SIZE": fetch[k]}))
    write(os.path.join(d, "w_counter_collection.csv"), trace(lambda k: {"WRITE_SIZE": write_[k]}))
    write(os.path.join(d, "b_counter_collection.csv"),
          trace(lambda k: {"SQ_VALU_MFMA_BUSY_CYCLES": busy[k] * 1024, "GRBM_GUI_ACTIVE": 8 * 1000.0,
                           "SQ_INSTS_MFMA": 7.0}))
    # copies of 256 MiB: FETCH reads half the bytes, WRITE all of them
    write(os.path.join(d, "cf_counter_collection.csv"),
          [("__amd_rocclr_copyBuffer", {"FETCH_SIZE": 131072.0})] * 3)
    write(os.path.join(d, "cw_counter_collection.csv"),
          [("__amd_rocclr_copyBuffer", {"WRITE_SIZE": 262144.0})] * 3)
    seq = {"profile_cases": ["up", "c4a"], "kernels": ["kA", "kW"], "algorithmic_bytes": [4096, 2048],
           "flops": [1, 1], "launches": 2, "marker": "FillFunctor", "step_cases": ["c4a", "up"],
           "kernel_source_sha": "abc"}
    with open(os.path.join(d, "seq.json"), "w") as f:
        f.write("some log line\n" + json.dumps(seq) + "\n")
    out = os.path.join(d, "traffic.json")
    md = os.path.join(d, "t.md")
    bc.main(["counters", "--seq", os.path.join(d, "seq.json"), "--dir", d, "--json", out, "--md", md])
    doc = json.load(open(out))
    assert doc["fetch_scale"] == 2.0 and doc["write_scale"] == 1.0
    up, conv = doc["per_case"]["up"], doc["per_case"]["c4a"]
    assert up["hbm_bytes"] == (1000 * 2 + 500) * 1024
    # the init kernel's bytes count with the case, its MFMA cycles do not
    assert conv["hbm_bytes"] == ((300 + 10) * 2 + 100 + 20) * 1024
    assert conv["dispatches_per_call"] == 2 and up["dispatches_per_call"] == 1
    assert abs(conv["mfma_busy"] - 0.6) < 1e-9 and abs(up["mfma_busy"] - 0.8) < 1e-9
    assert set(doc["kernels"]) == {"kA", "kW"}
    assert doc["kernels"]["kW"]["bytes_per_launch"] == conv["hbm_bytes"]
    assert doc["kernels"]["kW"]["algorithmic_bytes_per_launch"] == 2048
    assert "| c4a | kW |" in open(md).read()


def test_a_foreign_dispatch_inside_a_case_is_refused(tmp_path):
    d = [(GEMM_A, {"FETCH_SIZE": 1.0}), (FILL, {"FETCH_SIZE": 1.0}),
         ("void some_other_kernel()", {"FETCH_SIZE": 1.0}), (FILL, {"FETCH_SIZE": 1.0})]
    p = os.path.join(str(tmp_path), "x.csv")
    write(p, d)
    seq = {"profile_cases": ["up"], "marker": "FillFunctor"}
    import pytest
    with pytest.raises(SystemExit):
        bc.split_cases(bc.read_dispatches(p), seq)
