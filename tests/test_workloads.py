"""Host-side checks of the seeded input generators (no attention arithmetic)."""
import numpy as np
import torch

import workloads


def test_named_workloads_have_the_stated_shapes():
    w = workloads.WORKLOADS
    assert (w["tiny"].B, w["tiny"].H, w["tiny"].S, w["tiny"].D, w["tiny"].P) == (1, 2, 256, 64, 2)
    assert (w["image"].H, w["image"].S, w["image"].P) == (3, 4608, 8)
    assert (w["video"].H, w["video"].S, w["video"].D) == (5, 32768, 128)
    assert (w["long"].S, w["long"].sigma) == (131072, 0.5)
    assert (w["fp8"].B, w["fp8"].H, w["fp8"].dtype) == (2, 4, "fp8")
    for x in w.values():
        assert x.S % x.P == 0


def test_inputs_are_deterministic_and_bf16():
    w = workloads.custom(1, 96, 2, 64, 2)
    a, b = workloads.make_inputs(w), workloads.make_inputs(w)
    for n in "qkv":
        assert a[n].dtype == torch.bfloat16 and a[n].shape == (1, 96, 2, 64)
        assert torch.equal(a[n].view(torch.int16), b[n].view(torch.int16))
    assert not torch.equal(a["q"], a["k"])
    assert a["scale"] == float(np.float32(1 / 8))


def test_fp8_quantisation_stays_in_range_and_round_trips():
    w = workloads.custom(1, 128, 2, 64, 2, dtype="fp8")
    inp = workloads.make_inputs(w)
    for n, d in zip("qkv", inp["descales"]):
        x = inp[n]
        assert x.dtype == torch.float8_e4m3fn
        f = x.to(torch.float32)
        assert torch.isfinite(f).all() and f.abs().max() <= 448
        assert f.abs().max() >= 400  # amax maps to (near) the top of the range
        assert d > 0 and np.float32(d) == d


def test_long_sigma_is_applied():
    w = workloads.custom(1, 4096, 1, 64, 8, sigma=0.5)
    x = workloads.make_inputs(w)["q"].float()
    assert 0.45 < float(x.std()) < 0.55


def test_sample_rows_touch_every_slice():
    w = workloads.WORKLOADS["video"]
    rows = workloads.sample_rows(w, 64)
    T = w.S // w.P
    assert set((rows[:, 1] // T).tolist()) == set(range(w.P))
    assert rows[:, 0].max() < w.B and rows[:, 1].max() < w.S and rows[:, 2].max() < w.H
