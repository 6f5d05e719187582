"""Host-side logic of bench.py (no GPU): the algorithmic byte count, tactic
strings, the HBM traffic record built from rocprofv3 counter files, the
counter summary, and the refusal of more than one GPU.  The counter files
here are small synthetic CSVs in rocprofv3's column layout."""
from __future__ import annotations

import csv
import json
import subprocess
import sys
from pathlib import Path

import pytest

import bench
from split_bf16_gemm_amd import binding

ROOT = Path(__file__).resolve().parents[1]


def test_algorithmic_bytes():
    # the headline: W 2KN, A 2MK, C 2MN and the split-K partials 4MN(2S-1)
    M, N, K, S = 4, 6144, 4096, 2
    assert bench.algorithmic_bytes(M, N, K, S) == 2 * K * N + 2 * M * K + 2 * M * N + 4 * M * N * 3
    assert bench.algorithmic_bytes(M, N, K, S) == 50_708_480
    # no workspace traffic without split-K
    assert bench.algorithmic_bytes(M, N, K, 1) == 2 * K * N + 2 * M * K + 2 * M * N


@pytest.mark.parametrize("text", ["line:16:2:4", "quarter:32:2:3", "qrows:48:2:3", "panel:64:2:4",
                                  "reg:16:8:2", "lds:32:4:3"])
def test_tactic_strings_round_trip(text):
    t = bench.parse_tactic(text)
    assert bench.tactic_text(t) == text
    assert bench.parse_tactic("") is None


def _counter_csv(path: Path, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


GEMM = "void lowm::lowm_line_kernel<1, 1, 4, __bf16>(lowm::Args, lowm::Batch)"
COPY = "copy_kernel(uint4 const*, uint4*, unsigned long)"


def test_summarize_pmc_scales_by_the_copy(tmp_path):
    """FETCH_SIZE reads half the copy's bytes here, WRITE_SIZE all of them:
    the GEMM's counts are scaled by the same factors, from medians."""
    kib = bench.COPY_BYTES / 1024
    _counter_csv(tmp_path / "f" / "run_counter_collection.csv",
                 [(GEMM, "FETCH_SIZE", 24000.0), (GEMM, "FETCH_SIZE", 25000.0),
                  (GEMM, "FETCH_SIZE", 26000.0), ("other_kernel", "FETCH_SIZE", 1.0)])
    _counter_csv(tmp_path / "w" / "run_counter_collection.csv",
                 [(GEMM, "WRITE_SIZE", 250.0), (GEMM, "WRITE_SIZE", 270.0),
                  (GEMM, "WRITE_SIZE", 260.0)])
    _counter_csv(tmp_path / "cf" / "run_counter_collection.csv", [(COPY, "FETCH_SIZE", kib / 2)])
    _counter_csv(tmp_path / "cw" / "run_counter_collection.csv", [(COPY, "WRITE_SIZE", kib)])
    out = tmp_path / "traffic.json"
    before = bench.PMC_FILE.read_bytes() if bench.PMC_FILE.exists() else None
    rec = bench.summarize_pmc("m4_n6144_k4096_s2", None, tmp_path / "f", tmp_path / "w",
                              tmp_path / "cf", tmp_path / "cw", out=out)
    assert json.loads(out.read_text()) == rec
    assert (bench.PMC_FILE.read_bytes() if bench.PMC_FILE.exists() else None) == before
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_kib_per_dispatch"] == 25000.0 and rec["write_kib_per_dispatch"] == 260.0
    assert rec["traffic_bytes_per_launch"] == round(25000.0 * 1024 * 2 + 260.0 * 1024)
    assert rec["algorithmic_bytes_per_launch"] == 50_708_480
    assert rec["kernel"] == GEMM
    assert rec["source_sha"] == bench.source_hash()
    assert rec["tactic"]["stage"] == binding.LOWM_STAGE_LINE


def test_traffic_is_reported_only_for_its_sources(tmp_path, monkeypatch):
    import workloads
    wl = workloads.by_name("m4_n6144_k4096_s2")
    tac = {"stage": 3, "rows": 16, "waves": 4, "unroll": 2, "stages": 4}
    rec = {"source_sha": bench.source_hash(), "workload": wl.name, "tactic": tac,
           "traffic_bytes_per_launch": 123}
    f = tmp_path / "pmc.json"
    monkeypatch.setattr(bench, "PMC_FILE", f)
    f.write_text(json.dumps(rec))
    assert bench.pmc_traffic(wl, tac, 0) == 123
    assert bench.pmc_traffic(wl, dict(tac, stages=2), 0) is None          # another tactic
    f.write_text(json.dumps(dict(rec, source_sha="0" * 16)))
    assert bench.pmc_traffic(wl, tac, 0) is None                          # other sources
    f.write_text(json.dumps(dict(rec, workload="m4_n2304_k12288_s4")))
    assert bench.pmc_traffic(wl, tac, 0) is None                          # other workload
    f.write_text("not json")
    assert bench.pmc_traffic(wl, tac, 0) is None


def test_counter_summary_table(tmp_path, capsys):
    _counter_csv(tmp_path / "p1" / "a_counter_collection.csv",
                 [(GEMM, "SQ_WAVES", 3072.0), (GEMM, "SQ_WAVES", 3072.0),
                  (GEMM, "GRBM_GUI_ACTIVE", 10.0), (GEMM, "GRBM_GUI_ACTIVE", 30.0),
                  (GEMM, "GRBM_GUI_ACTIVE", 20.0), (COPY, "SQ_WAVES", 1.0)])
    bench.counter_summary([tmp_path / "p1"])
    out = capsys.readouterr().out
    assert "void lowm::lowm_line_kernel<1, 1, 4, __bf16>" in out and "copy_kernel" not in out
    assert "| GRBM_GUI_ACTIVE | 20 | 3 |" in out
    assert "| SQ_WAVES | 3,072 | 2 |" in out


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
