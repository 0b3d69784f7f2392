"""Host logic of bench.py that runs without a GPU: the one-GPU refusal, the
traffic record's source check, and the CPU baseline's record."""
import json
import os
import shutil
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_traffic_record_is_used_only_while_the_kernel_sources_match(tmp_path, monkeypatch):
    rec_path = os.path.join(ROOT, "profiles", "attn_fwd_bf16_video.traffic.json")
    rec = json.load(open(rec_path))
    assert bench.recorded_traffic("attn_fwd_bf16", "video") == rec["traffic_bytes_per_launch"]
    assert bench.recorded_traffic("attn_fwd_bf16", "no_such_workload") is None
    # a copy of the tree with one kernel source changed by a byte: the record no longer applies
    os.makedirs(tmp_path / "profiles")
    shutil.copy(rec_path, tmp_path / "profiles")
    for src in rec["sources"]:
        os.makedirs(tmp_path / os.path.dirname(src), exist_ok=True)
        shutil.copy(os.path.join(ROOT, src), tmp_path / src)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("attn_fwd_bf16", "video") == rec["traffic_bytes_per_launch"]
    with open(tmp_path / rec["sources"][0], "ab") as f:
        f.write(b"\n")
    assert bench.recorded_traffic("attn_fwd_bf16", "video") is None


def test_cpu_baseline_record():
    w = workloads.WORKLOADS["tiny"]
    inp = workloads.make_inputs(w)
    cb = bench.cpu_baseline(w, inp, 0.2)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    n = int(cb["sample"].split(" of ")[0])
    assert 1 <= n <= w.B * w.S * w.H and n % cb["cores"] == 0 or n == w.B * w.S * w.H


SMI_TEXT = """GPU: 0
    POWER:
        SOCKET_POWER: 1331 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 1760 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 1772 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        MEM_0:
            CLK: 2000 MHz
"""


def test_amd_smi_text_parsed():
    # socket power and the mean of the GFX clocks only (not the memory clock, not the limits)
    assert bench.smi_parse(SMI_TEXT) == (1331.0, 1766.0)
    assert bench.smi_parse("GPU: 0\n    POWER:\n        SOCKET_POWER: N/A\n") is None


def test_live_clock_pairs_samples_by_compute_unit():
    # constant counter 100 MHz (100000 kHz), 1 ms between the samples.  XCC 0: CUs
    # 0x01 and 0x02 ran 1.7e6 and 1.9e6 cycles (median 1.8 GHz); XCC 5: CU 0x01 2.0e6;
    # hw_id bits outside 8-15 do not matter; CU 0x03 of XCC 0 appears in one sample
    # only and is skipped; later records of a CU already seen are ignored.  The
    # counters of different CUs are not synchronised.
    a = [[1000, 500, 0, 0x0107], [9_000_000, 500, 0, 0x0200], [7000, 510, 5, 0x0100],
         [1, 1, 0, 0x0300], [9, 9, 0, 0x0100]]
    b = [[1000 + 1_700_000, 500 + 100_000, 0, 0x0155], [9_000_000 + 1_900_000, 500 + 100_000, 0, 0x0200],
         [7000 + 2_000_000, 510 + 100_000, 5, 0x0100]]
    ghz = bench.live_clock(a, b, 100000)
    assert set(ghz) == {0, 5}
    assert abs(ghz[0] - 1.8) < 1e-9 and abs(ghz[5] - 2.0) < 1e-9
    rec = bench.run_clock(ghz, 1200.0, 1190.0, 2500.0, None)
    assert rec["sclk_ghz"] == 1.9
    assert abs(rec["peak_at_that_clock"] - 2500.0 * 1.9 / 2.4) < 0.1
    assert bench.run_clock({}, 1.0, 1.0, 2500.0, None)["sclk_ghz"] is None
