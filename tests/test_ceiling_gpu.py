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
