"""bench.py --record-traffic on synthetic rocprofv3 counter files (CPU): the per-call bytes of the
chunk kernels (two dispatches per prefill call, the main pass and the launch that holds the
transition and rerun passes; or three, the rerun pass being the one instantiation with rerun code,
where those two run as launches of their own) and of the decode kernel, each scaled by the
plain-copy calibration."""
import csv
import json
import os

import pytest

import bench

HEADER = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
MAIN = "void gdn::(anonymous namespace)::chunk_bf16_kernel<128, 128, false, false, true, false>(gdn::Params<128>)"
TRANS = "void gdn::(anonymous namespace)::chunk_bf16_kernel<128, 128, false, false, true, true>(gdn::Params<128>)"
RERUN = "void gdn::(anonymous namespace)::chunk_bf16_kernel<128, 128, false, false, false, false>(gdn::Params<128>)"
TAIL = ("void gdn::(anonymous namespace)::chunk_bf16_tail_kernel<128, 128, false, false>(gdn::Params<128>, "
        "gdn::Params<128>)")
STEP = "void gdn::step_kernel<128, 128, gdn::bf16, false, false>(gdn::bf16 const*)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, counter, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HEADER)
        for d, (name, kib) in enumerate(rows):
            # two dimensions of one dispatch: the parser sums them
            for part in (0.25, 0.75):
                w.writerow([d, d, 1, 1, 1, 1, 64, 1, name, 256, 0, 0, 0, 0, 0, counter, kib * part, 0, 1])


@pytest.mark.parametrize("fused", [True, False])
def test_record_traffic(tmp_path, fused):
    d = str(tmp_path)
    # calibration: a 1 GiB copy that FETCH_SIZE reports as half its bytes, WRITE_SIZE exactly
    _write(os.path.join(d, "cfetch", "run_counter_collection.csv"), "FETCH_SIZE", [(COPY, 524288.0)] * 3)
    _write(os.path.join(d, "cwrite", "run_counter_collection.csv"), "WRITE_SIZE", [(COPY, 1048576.0)] * 3)
    # two prefill calls (main, then transition + rerun in one launch or in two) and one decode step,
    # KiB per dispatch
    tail = [(TAIL, 11.0)] if fused else [(TRANS, 1.0), (RERUN, 10.0)]
    calls = ([(MAIN, 100.0)] + tail) * 2 + [(STEP, 50.0)]
    _write(os.path.join(d, "fetch", "run_counter_collection.csv"), "FETCH_SIZE", calls)
    _write(os.path.join(d, "write", "run_counter_collection.csv"), "WRITE_SIZE",
           [(n, k / 2) for n, k in calls])
    out = bench.record_traffic(d, out_path=os.path.join(d, "traffic.json"))
    c = out["chunk_bf16_kernel"]
    assert c["calls"] == [2, 2]
    assert c["counter_scale"]["FETCH_SIZE"] == pytest.approx(2.0)
    assert c["counter_scale"]["WRITE_SIZE"] == pytest.approx(1.0)
    assert c["fetch_bytes"] == pytest.approx(111.0 * 1024 * 2.0)
    assert c["write_bytes"] == pytest.approx(55.5 * 1024)
    assert c["bytes_per_launch"] == pytest.approx(c["fetch_bytes"] + c["write_bytes"])
    assert c["source_sha"] == bench.source_sha("chunk_bf16.hip")
    s = out["step_kernel"]
    assert s["fetch_bytes"] == pytest.approx(50.0 * 1024 * 2.0)
    assert s["write_bytes"] == pytest.approx(25.0 * 1024)
    assert json.load(open(os.path.join(d, "traffic.json")))["step_kernel"]["calls"] == [1, 1]
