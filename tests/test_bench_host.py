"""Host logic of bench.py on synthetic rocprofv3 CSVs (no GPU): the copy calibration
scales FETCH_SIZE / WRITE_SIZE into bytes, the clock run gives clock and peak
fractions, both land in the traffic table keyed by the GEMM source hash, and the
bench reads them back only while that hash matches."""
import csv
import json

import bench


def write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                                          "End_Timestamp"])
        w.writeheader()
        for kernel, counter, value, dur_ns in rows:
            w.writerow({"Kernel_Name": f"void gl::gemm::{kernel}(gl::gemm::Params)", "Counter_Name": counter,
                        "Counter_Value": value, "Start_Timestamp": 1000, "End_Timestamp": 1000 + dur_ns})


def test_summaries_round_trip(tmp_path, monkeypatch):
    table = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(table))
    fwd = bench.PASS_KERNELS["forward"]
    # copy of 1 GiB: FETCH_SIZE reads half the bytes in KiB, WRITE_SIZE all of them
    write_csv(tmp_path / "cf.csv", [("copy_kernel", "FETCH_SIZE", (1 << 30) / 2048, 10)])
    write_csv(tmp_path / "cw.csv", [("copy_kernel", "WRITE_SIZE", (1 << 30) / 1024, 10)])
    write_csv(tmp_path / "f.csv", [(fwd, "FETCH_SIZE", 1000.0, 10), (fwd, "FETCH_SIZE", 3000.0, 10)])
    write_csv(tmp_path / "w.csv", [(fwd, "WRITE_SIZE", 500.0, 10)])
    bench.summarize_pmc(tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "cf.csv", tmp_path / "cw.csv")
    rec = json.loads(table.read_text())["bf16_train_g8_k4096_n14336:forward"]
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["fetch_bytes"] == 2000 * 1024 * 2 and rec["write_bytes"] == 500 * 1024
    assert bench.traffic_for("forward", "bf16_train_g8_k4096_n14336") == rec["bytes_per_launch"]

    # clock run: 2.0 GHz over 1 ms, MFMA busy half of the SIMD-cycles
    cycles = 2.0e6
    write_csv(tmp_path / "c.csv", [(fwd, "GRBM_GUI_ACTIVE", 8 * cycles, 1_000_000),
                                   (fwd, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cycles * 256 * 4, 1_000_000),
                                   (fwd, "SQ_LDS_BANK_CONFLICT", 10.0, 1_000_000),
                                   (fwd, "SQ_LDS_IDX_ACTIVE", 1000.0, 1_000_000)])
    bench.summarize_clock(tmp_path / "c.csv")
    rec = bench.clock_for("forward", "bf16_train_g8_k4096_n14336")
    assert rec["sclk_ghz"] == 2.0 and rec["mfma_busy_frac"] == 0.5 and rec["lds_bank_conflict_per_active"] == 0.01
    flops = 2.0 * 16384 * 14336 * 4096
    assert abs(rec["frac_of_peak_at_sclk"] - flops / 1e-3 / (256 * 4096 * 2.0e9)) < 1e-4
    assert rec["bytes_per_launch"] == 2000 * 1024 * 2 + 500 * 1024  # the traffic fields survive

    # another source hash: nothing is reported
    data = json.loads(table.read_text())
    data["bf16_train_g8_k4096_n14336:forward"]["source_sha"] = "0" * 16
    table.write_text(json.dumps(data))
    assert bench.traffic_for("forward", "bf16_train_g8_k4096_n14336") is None
    assert bench.clock_for("forward", "bf16_train_g8_k4096_n14336") is None


def test_gpus_above_one_exits_with_a_message(monkeypatch, capsys):
    import pytest
    import sys

    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2 and "one GPU" in capsys.readouterr().err
