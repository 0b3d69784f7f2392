"""The matrix-core ceiling probes (xs_mfma_ceiling) run through the C ABI on the GPU."""
import ctypes

import pytest
import torch

import bench
from sequence_attention_amd import _lib

pytestmark = pytest.mark.gpu


def test_every_probe_mode_runs():
    L = _lib.lib()
    sentinel = 12345.678
    sink = torch.empty((1024, 512), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    for waves in (1, 2):
        for mode in range(len(bench.CEILING_MODES)):
            print(f"ceiling probe mode={mode} waves={waves}", flush=True)
            sink.fill_(sentinel)
            rc = L.xs_mfma_ceiling(mode, waves, 8, ctypes.c_void_p(sink.data_ptr()), sink.numel() * 4,
                                   ctypes.c_void_p(stream.cuda_stream))
            assert rc == 0
            torch.cuda.synchronize()
            # every thread of the 1024 workgroups stored its float (its value carries no
            # meaning: the operands are arbitrary bit patterns), and no thread wrote elsewhere
            written = sink[:, :256 * waves]
            assert bool((written != sentinel).all())
            assert bool((sink[:, 256 * waves:] == sentinel).all())


def test_ceiling_rates_are_rates():
    res = bench.ceilings(64, reps=2)
    for waves in ("1_waves_per_simd", "2_waves_per_simd"):
        r = res[waves]
        assert 0.5 < r["mfma_only_clock_ghz"] < 3.5
        for row in r["modes"]:
            assert row["ms"] > 0 and 0.1 < row["mfma_rate_vs_mfma_only"] < 1.5


def test_clock_sample_reads_a_plausible_shader_clock():
    L = _lib.lib()
    stream = torch.cuda.current_stream()
    a = torch.zeros(1024 * 4, dtype=torch.int64, device="cuda:0")
    b = torch.zeros_like(a)
    sink = torch.empty((1024, 512), dtype=torch.float32, device="cuda:0")
    khz = bench.clock_sample(L, a, stream)
    # about 10 ms of matrix work between the two samples
    for _ in range(3):
        assert L.xs_mfma_ceiling(0, 2, 2048, ctypes.c_void_p(sink.data_ptr()), sink.numel() * 4,
                                 ctypes.c_void_p(stream.cuda_stream)) == 0
    bench.clock_sample(L, b, stream)
    torch.cuda.synchronize()
    ra, rb = a.cpu().numpy().reshape(-1, 4), b.cpu().numpy().reshape(-1, 4)
    print(f"wall clock {khz} kHz; xcc ids {sorted(set(ra[:, 2].tolist()))}", flush=True)
    assert khz > 0
    assert (ra[:, 0] > 0).all() and (ra[:, 1] > 0).all()
    assert set(ra[:, 2].tolist()) <= set(range(16))
    ghz = bench.live_clock(ra, rb, khz)
    print("per-XCC clock GHz", {k: round(v, 3) for k, v in ghz.items()}, flush=True)
    # every compute unit seen in both samples, for the record of the spread
    first = lambda r: {(int(x), (int(h) >> 8) & 0xFF): (int(t), int(q)) for t, q, x, h in r[::-1]}
    fa, fb = first(ra), first(rb)
    cu = [(fb[k][0] - fa[k][0]) / ((fb[k][1] - fa[k][1]) / (khz * 1e3)) / 1e9 for k in set(fa) & set(fb)]
    print(f"{len(cu)} compute units paired; per-CU clock min {min(cu):.3f} median "
          f"{sorted(cu)[len(cu) // 2]:.3f} max {max(cu):.3f} GHz", flush=True)
    assert ghz and all(0.5 < g < 3.5 for g in ghz.values())
