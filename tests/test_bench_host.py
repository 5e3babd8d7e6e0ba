"""Host logic of bench.py (no GPU): the algorithmic byte / flop counts and the
rocprofv3 summaries, on small synthetic inputs whose answers are known."""
import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, counter, value, dur_ns) in enumerate(rows):
            r = {k: 0 for k in FIELDS}
            r.update(Dispatch_Id=i + 1, Kernel_Name=name, Counter_Name=counter,
                     Counter_Value=value, Start_Timestamp=1000, End_Timestamp=1000 + dur_ns)
            w.writerow(r)


def test_flop_and_byte_counts_at_v3_shape():
    import moe_inputs
    c = moe_inputs.CONFIGS["v3_bf16"]
    # 6*T*k*d*I + 6*T*d*Is: the routed and shared SwiGLU FFNs
    assert bench.ffn_flops(c) == 6 * 8192 * 8 * 7168 * 2048 + 6 * 8192 * 7168 * 2048
    # bf16 weights: 256 experts x 3 matrices of 2048 x 7168 plus the shared ones
    assert bench.ffn_weight_bytes(c) == (256 + 1) * 3 * 2048 * 7168 * 2


def test_counter_summary_calibrates_mfma_and_bytes(tmp_path):
    probe = "void moe::(anonymous namespace)::probe_mfma_kernel<1>(int, float*)"
    probe8 = "void moe::(anonymous namespace)::probe_mfma_kernel<2>(int, float*)"
    gemm = "void moe::ffn_gemm_bf16_kernel<0, 64, 2>(moe::GemmParamsV2)"
    copy = "__amd_rocclr_copyBuffer"
    m = tmp_path / "m.csv"
    _csv(m, [(probe, "SQ_VALU_MFMA_BUSY_CYCLES", 400.0, 10), (probe, "GRBM_GUI_ACTIVE", 4.0, 10),
             (probe8, "SQ_VALU_MFMA_BUSY_CYCLES", 800.0, 10), (probe8, "GRBM_GUI_ACTIVE", 8.0, 10),
             (gemm, "SQ_VALU_MFMA_BUSY_CYCLES", 50.0, 2000), (gemm, "GRBM_GUI_ACTIVE", 1.0, 2000)])
    # the copy reads 2 * 1 GiB by the counter (so the scale is 1/2), writes 1 GiB
    f = tmp_path / "f.csv"
    _csv(f, [(copy, "FETCH_SIZE", 2.0 * (1 << 20), 5)] * 3 + [(gemm, "FETCH_SIZE", 2.0 * 1000, 2000)])
    w = tmp_path / "w.csv"
    _csv(w, [(copy, "WRITE_SIZE", 1.0 * (1 << 20), 5)] * 3 + [(gemm, "WRITE_SIZE", 500.0, 2000)])
    out = bench.counter_summary(str(m), str(f), str(w), "v3_bf16")
    row = [l for l in out.splitlines() if "ffn_gemm_bf16_kernel" in l][0].split()
    # busy 50/1 against the probe's 400/4 = 100: 50%; 2 us per dispatch;
    # read 1000 KiB = 1.024 MB, write 500 KiB = 0.512 MB
    assert row[-6] == "2.0" and row[-5] == "50.0%"
    assert row[-4] == "1.0" and row[-3] == "0.5"


def test_counter_summary_needs_calibration(tmp_path):
    gemm = "void moe::ffn_gemm_bf16_kernel<0, 64, 2>(moe::GemmParamsV2)"
    p = tmp_path / "x.csv"
    _csv(p, [(gemm, "SQ_VALU_MFMA_BUSY_CYCLES", 1.0, 1), (gemm, "GRBM_GUI_ACTIVE", 1.0, 1)])
    with pytest.raises(SystemExit):
        bench.counter_summary(str(p), str(p), str(p), "v3_bf16")
