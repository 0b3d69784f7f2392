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
