"""Host logic of bench.py (CPU only): the one-GPU refusal and the arithmetic that turns a
rocprofv3 counter pass into MFMA utilisation and clock."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_touching_a_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_mfma_counter_arithmetic(tmp_path):
    # Two XCDs, 8 SIMDs, 2 GHz maximum. Dispatch 1 is a warmup that must be dropped
    # (last=2); dispatches 2 and 3 are the attention kernel, 4 is another kernel.
    _write(tmp_path / "m_agent_info.csv",
           ["Name", "Num_Xcc", "Simd_Count", "Max_Engine_Clk_Fcompute"],
           [["AMD EPYC", "0", "0", "0"], ["gfx950", "2", "8", "2000"]])
    cc = []
    for did, gui, busy, mops in ((1, 1, 1, 1), (2, 2000, 8000, 1000), (3, 6000, 8000, 3000)):
        for name, val in (("GRBM_GUI_ACTIVE", gui), ("SQ_VALU_MFMA_BUSY_CYCLES", busy),
                          ("SQ_INSTS_VALU_MFMA_MOPS_BF16", mops)):
            cc.append([did, "void attn::attn_fwd_pp_kernel<128, false>(attn::FwdParams)", name,
                       val])
    cc.append([4, "void at::native::reduce_kernel<>", "GRBM_GUI_ACTIVE", 99999])
    _write(tmp_path / "m_counter_collection.csv",
           ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], cc)
    _write(tmp_path / "m_kernel_trace.csv",
           ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [[1, "attn_fwd_pp_kernel", 0, 5], [2, "attn_fwd_pp_kernel", 100, 1100],
            [3, "attn_fwd_pp_kernel", 2000, 4000], [4, "reduce_kernel", 0, 10]])
    m = bench.mfma_from_dir(str(tmp_path), algorithmic_flop=123, last=2)
    # per XCD: mean GUI (2000 + 6000) / 2 / 2 XCDs = 2000 cycles over a mean 1500 ns
    assert m["dispatches"] == 2
    assert m["cycles_per_xcd"] == 2000
    assert m["clock_ghz"] == pytest.approx(2000 / 1500, abs=1e-3)
    # busy 8000 / (2000 cycles x 8 SIMDs) = 0.5
    assert m["mfma_util"] == pytest.approx(0.5)
    assert m["mfma_flop_counted"] == 2000 * 512
    assert m["algorithmic_flop"] == 123
    assert m["max_clock_ghz"] == 2.0
    assert m["peak_at_measured_clock_tflops"] == pytest.approx(
        bench.PEAK_BF16_TFLOPS * (2000 / 1500) / 2.0, abs=0.1)


def test_counter_readings_are_dropped_when_sources_change(tmp_path, monkeypatch):
    import json
    import synth
    f = tmp_path / "counters.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    w = synth.workload("dense_b1_n4096_h32_d128")
    f.write_text(json.dumps({"workloads": {w.name: {
        "kernel_source_hash": "0" * 16, "hbm_bytes_per_launch": 1,
        "mfma": {"mfma_util": 0.5, "clock_ghz": 2.0, "profiled_duration_us": 200}}}}))
    assert bench.counters_for(w) == {} and bench.traffic_for(w) is None
    bench._update_entry(w.name, {"hbm_bytes_per_launch": 7})
    e = bench.counters_for(w)
    assert e["hbm_bytes_per_launch"] == 7 and "mfma" not in e
    assert e["kernel_source_hash"] == bench.kernel_source_hash(w.kind)


def test_output_check_applies_the_acceptance_rule():
    """The bench's check of its timed output: the oracle's own rows rounded to BF16 pass,
    the same rows with one element off by 0.5 fail (the per-element cap)."""
    import numpy as np

    import synth
    w = synth.small("dense", 1, 64, 2, 64, 950, sigma_qk=2.0)
    ts = w.tensors()
    cpu, ref = bench.cpu_baseline(w, 0.0, ts)
    assert ref.shape == (w.B * w.Nq * w.H, w.D) and cpu["kind"] == "oracle"
    bits = synth.f32_to_bf16_bits(ref.astype(np.float32))
    good = bench.check_output(bits, ref, w.D)
    assert good["ok"] and good["rows_checked"] == good["rows_total"] == 128
    bad = synth.bf16_bits_to_f32(bits).copy()
    bad[7, 3] += 0.5
    res = bench.check_output(synth.f32_to_bf16_bits(bad), ref, w.D)
    assert not res["ok"] and res["max_abs_err"] > 0.4


def test_output_check_covers_only_the_rows_the_oracle_computed():
    import numpy as np
    ref = np.zeros((3, 64))
    out = np.zeros((10, 64), np.uint16)
    out[5:] = 0x4000  # 2.0 in BF16, beyond the checked rows
    res = bench.check_output(out, ref, 64)
    assert res["ok"] and res["rows_checked"] == 3 and res["rows_total"] == 10


def test_kernel_names_follow_the_library_instantiation():
    """The bench names the kernel a plan runs as rocprofv3 reports it."""
    assert bench.kernel_name(128, {"waves": 8, "splits": 1}, 4096) == "attn_fwd_pp_kernel<128, false>"
    assert bench.kernel_name(64, {"waves": 2, "splits": 1}, 64) == "attn_fwd_kernel<64, 2, 64, 1>"
    assert bench.kernel_name(64, {"waves": 2, "splits": 1}, 256) == "attn_fwd_kernel<64, 2, 64, 3>"
    assert bench.kernel_name(128, {"waves": 2, "splits": 1}, 100) == "attn_fwd_kernel<128, 2, 32, 3>"
    assert (bench.kernel_name(128, {"waves": 4, "splits": 4}, 256)
            == "attn_fwd_kernel<128, 4, 64, 1> + attn_combine_kernel<128>")
