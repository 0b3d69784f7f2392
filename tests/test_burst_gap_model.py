"""The Burst-Gap model code (sequence_attention_amd.burst_gap) on the CPU:
hand-computed predictions, and the fit recovering known parameters from
measurements synthesised with the model (plus noise)."""
import numpy as np
import pytest

from sequence_attention_amd import burst_gap as bg

P = bg.Params(a=2e-6, c=4e-10, R=50e9, Q=8e6)


def test_predictions_by_hand():
    # t0 = 2e-6 + 4e-10 * 65536 = 2.62144e-5 s; V/R = 256*65536/50e9 = 3.3554432e-4 s
    K, V = 256, 256 * 65536
    t0 = 2e-6 + 4e-10 * 65536
    assert bg.predict(P, K, V, 0.0) == pytest.approx(V / 50e9, rel=1e-12)        # drain-dominated
    assert bg.predict(P, K, V, 1e-4) == pytest.approx(V / 50e9 - 1e-4, rel=1e-12)
    assert bg.predict(P, K, V, 1e-3) == pytest.approx(t0, rel=1e-12)            # backpressure-free
    # a single burst stalls only beyond Q outstanding bytes
    assert bg.predict_first(P, K, 4e6) == pytest.approx(2e-6 + 4e-10 * 4e6 / 256, rel=1e-12)
    assert bg.predict_first(P, K, V) == pytest.approx((V - 8e6) / 50e9, rel=1e-12)


def _synthetic(p, noise, seed=0):
    rng = np.random.default_rng(seed)
    K, V, G = [], [], []
    for k in (64, 256):
        for b in (16384, 65536, 262144):
            for g in (0.0, 5e-6, 2e-5, 5e-5, 1e-4, 2e-4, 5e-4, 2e-3):
                K.append(k), V.append(k * b), G.append(g)
    K, V, G = (np.array(x, dtype=np.float64) for x in (K, V, G))
    ts = bg.predict(p, K, V, G) * (1 + noise * rng.standard_normal(len(K)))
    tf = bg.predict_first(p, K, V) * (1 + noise * rng.standard_normal(len(K)))
    return K, V, G, ts, tf


@pytest.mark.parametrize("noise", [0.0, 0.02])
def test_fit_recovers_known_parameters(noise):
    K, V, G, ts, tf = _synthetic(P, noise)
    f = bg.fit(K, V, G, ts, tf)
    tol = 1e-9 if noise == 0 else 0.06
    assert f.a == pytest.approx(P.a, rel=10 * tol if noise else 1e-6, abs=2e-7 if noise else 1e-12)
    assert f.c == pytest.approx(P.c, rel=tol if noise else 1e-6)
    assert f.R == pytest.approx(P.R, rel=tol if noise else 1e-9)
    # Q is bracketed by the sweep's burst volumes: 4 MiB bursts are absorbed,
    # 16 MiB bursts stall (true Q = 8e6)
    lo, hi = f.Q_bracket
    assert (lo, hi) == (4 * 2**20, 16 * 2**20)
    assert lo <= P.Q < hi and lo <= f.Q < hi


def test_fit_without_stalled_first_bursts_reports_unbounded_capacity():
    p = bg.Params(a=2e-6, c=4e-10, R=50e9, Q=1e12)
    K, V, G, ts, tf = _synthetic(p, 0.0)
    f = bg.fit(K, V, G, ts, tf)
    assert f.Q == float("inf") and f.Q_bracket[1] == float("inf")


def test_fit_needs_backpressure_free_runs():
    K = np.array([64, 64, 64.0])
    V = np.array([1e6, 2e6, 4e6])
    G = np.zeros(3)
    ts = V / 50e9
    with pytest.raises(ValueError):
        bg.fit(K, V, G, ts, ts)


def test_completion_coupled_prediction_sums_every_round():
    # T_c(V) = a + V / R for each round's burst of min(tiles, CUs) tiles
    pc = bg.Coupled(a=2e-6, R=100e9, runs=[])
    tile = 65536
    # 640 tiles on 256 CUs: rounds of 256, 256 and 128 tiles
    want = 3 * 2e-6 + (256 + 256 + 128) * tile / 100e9
    assert abs(bg.predict_attention_coupled(pc, 640, 256, tile) - want) < 1e-12
    # fewer tiles than CUs: one round
    assert abs(bg.predict_attention_coupled(pc, 54, 256, tile) - (2e-6 + 54 * tile / 100e9)) < 1e-12


def test_end_drain_prediction_by_hand():
    end = bg.Linear(a=5e-6, R=50e9)
    stretch = bg.Linear(a=0.0, R=600e9)
    tile = 65536
    # 640 tiles on 256 CUs: two full rounds stretch the loads after them, the
    # last (128 tiles) drains at the end
    want = 2 * (256 * tile / 600e9) + 5e-6 + 128 * tile / 50e9
    assert bg.predict_attention_end(end, stretch, 640, 256, tile) == pytest.approx(want, rel=1e-12)
    assert bg.predict_attention_end(end, stretch, 54, 256, tile) == pytest.approx(5e-6 + 54 * tile / 50e9)
    f = bg.fit_linear([1e6, 2e6, 4e6], [5e-6 + 1e6 / 50e9, 5e-6 + 2e6 / 50e9, 5e-6 + 4e6 / 50e9])
    assert f.a == pytest.approx(5e-6, rel=1e-6) and f.R == pytest.approx(50e9, rel=1e-6)
    g = bg.fit_linear([1e6, 2e6], [1e6 / 600e9, 2e6 / 600e9], through_origin=True)
    assert g.a == 0.0 and g.R == pytest.approx(600e9, rel=1e-9)
