"""One-GPU characterisation of the Burst-Gap model with the library's
microbenchmark (include/xs_burst_gap.h).

The model (X-Stage paper, gist.science explainer, "Methodik: Die
X-Stage-Abstraktion und das Burst-Gap-Modell"): a burst of aggregate volume V
issued by K producers that leave a computation gap G between bursts has the
sender-visible issue time

    T_iss(G; K, V) = max(T0_iss(K, V), V/R - G)

where T0_iss is the backpressure-free issue time, R the effective drain rate and
Q the outstanding capacity.  A single burst after an idle period is not limited
by earlier bursts; it stalls only once more than Q bytes are outstanding:
T_first(K, V) = max(T0_iss(K, V), (V - Q)/R).  On one GPU the producers'
stores go to fine-grained host memory, standing in for a remote link.

This module runs the microbenchmark (``measure``), fits T0_iss, R and Q to the
measurements (``fit``: T0_iss(K, V) = a + c*V/K from backpressure-free points,
R from drain-dominated steady-state points, Q from stalled first bursts) and
predicts issue times from the fitted parameters (``predict``).  Host memory is
allocated with the HIP runtime (hipHostMalloc, coherent and mapped); the
measurement itself runs in the library's HIP kernel.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from ._lib import lib

HIP_HOST_MALLOC_MAPPED = 0x2
HIP_HOST_MALLOC_COHERENT = 0x40000000
WAVES = 4          # per producer (include/xs_burst_gap.h)
STEP_BYTES = 4096  # bytes per producer must be a multiple of this


# ---------------------------------------------------------------- model
@dataclass
class Params:
    a: float  # s, fixed part of the backpressure-free issue time of a burst
    c: float  # s per byte per producer (1 / per-producer issue rate)
    R: float  # bytes/s, effective drain rate
    Q: float  # bytes, outstanding capacity
    Q_bracket: tuple = (0.0, float("inf"))  # bytes: largest absorbed, smallest stalled burst

    def t0(self, K, V):
        return self.a + self.c * np.asarray(V, dtype=np.float64) / np.asarray(K, dtype=np.float64)


def predict(p: Params, K, V, G):
    """Steady-state issue time T_iss(G; K, V) = max(T0(K, V), V/R - G)."""
    V = np.asarray(V, dtype=np.float64)
    return np.maximum(p.t0(K, V), V / p.R - np.asarray(G, dtype=np.float64))


def predict_first(p: Params, K, V):
    """Issue time of a single burst after idle: max(T0(K, V), (V - Q)/R)."""
    V = np.asarray(V, dtype=np.float64)
    return np.maximum(p.t0(K, V), (V - p.Q) / p.R)


def fit(K, V, G, t_steady, t_first) -> Params:
    """Fit T0 = a + c V/K, R and Q to measurements (arrays of one entry per run).

    1. R0 = median V / (T_steady + G) over the runs with the smallest gap
       (drain-dominated when G is small and the bursts fill the outstanding
       capacity) -- a first estimate of R.
    2. T0: least squares of T_steady on V/K over runs with G >= 2 V / R0
       (the gap covers the drain: backpressure-free), weighted by 1/T_steady
       so that small bursts count as much as large ones.
    3. R: median V / (T_steady + G) over runs whose steady issue time exceeds
       both 1.25 T0 and a quarter of V/R0 (drain-dominated).
    4. Q: a single burst after idle issues at the backpressure-free rate until
       Q bytes are outstanding.  Runs whose first burst took more than half of
       V/R are stalled; Q lies between the largest burst that was not and the
       smallest that was (Q_lo, Q_hi).  The point value is the geometric mean
       of the bracket (Q_hi alone if no burst was absorbed, +inf if none
       stalled).
    """
    K, V, G, ts, tf = (np.asarray(x, dtype=np.float64) for x in (K, V, G, t_steady, t_first))
    small = G <= np.min(G) + 1e-12
    R0 = float(np.median(V[small] / (ts[small] + G[small])))
    free = G >= 2.0 * V / R0
    if free.sum() < 2:
        raise ValueError("need at least two backpressure-free runs (G >= 2 V / R)")
    x = V[free] / K[free]
    wgt = 1.0 / ts[free]
    A = np.stack([np.ones_like(x), x], axis=1) * wgt[:, None]
    (a, c), *_ = np.linalg.lstsq(A, ts[free] * wgt, rcond=None)
    t0 = a + c * V / K
    drained = (ts > 1.25 * t0) & (ts > 0.25 * V / R0)
    R = float(np.median(V[drained] / (ts[drained] + G[drained]))) if drained.any() else R0
    stalled = tf > 0.5 * V / R
    if not stalled.any():
        Q, lo, hi = float("inf"), float(V.max()), float("inf")
    else:
        hi = float(V[stalled].min())
        absorbed = ~stalled & (V < hi)
        lo = float(V[absorbed].max()) if absorbed.any() else 0.0
        Q = float(np.sqrt(lo * hi)) if lo > 0 else hi
    return Params(float(a), float(c), R, Q, (lo, hi))


# ---------------------------------------------------------------- measurement
class HostBuffer:
    """Fine-grained (coherent), mapped host memory from the HIP runtime."""

    def __init__(self, nbytes: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t,
                                            ctypes.c_uint]
        self._hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                      ctypes.c_void_p, ctypes.c_uint]
        self._hip.hipHostFree.argtypes = [ctypes.c_void_p]
        p = ctypes.c_void_p()
        rc = self._hip.hipHostMalloc(ctypes.byref(p), nbytes,
                                     HIP_HOST_MALLOC_COHERENT | HIP_HOST_MALLOC_MAPPED)
        if rc != 0 or not p.value:
            raise RuntimeError(f"hipHostMalloc({nbytes}) failed with {rc}")
        self.host = p.value
        d = ctypes.c_void_p()
        rc = self._hip.hipHostGetDevicePointer(ctypes.byref(d), p, 0)
        if rc != 0:
            self._hip.hipHostFree(p)
            raise RuntimeError(f"hipHostGetDevicePointer failed with {rc}")
        self.ptr = d.value
        self.nbytes = nbytes

    def view(self, dtype=np.uint8, count=None):
        n = self.nbytes // np.dtype(dtype).itemsize if count is None else count
        buf = (ctypes.c_char * (n * np.dtype(dtype).itemsize)).from_address(self.host)
        return np.frombuffer(buf, dtype=dtype, count=n)

    def free(self):
        if self.host:
            self._hip.hipHostFree(ctypes.c_void_p(self.host))
            self.host = self.ptr = 0


@dataclass
class Run:
    K: int
    V: float          # bytes, all producers
    G: float          # s
    t_first: float    # s, issue time of the first burst (slowest wave, median producer)
    t_steady: float   # s, median over the later half of the bursts of the same
    drain: float      # s, completion of the last burst's stores after its gap
    clock_hz: float


def measure(dst_ptr: int, dst_bytes: int, producers: int, bytes_per_producer: int, nburst: int,
            gap_cycles: int, torch_device) -> Run:
    """One launch of the microbenchmark; times converted with the run's own clock."""
    import torch

    n = producers * WAVES * (nburst + 3)
    times = torch.zeros(n, dtype=torch.int64, device=torch_device)
    stream = torch.cuda.current_stream(torch_device)
    rc = lib().xs_burst_gap(dst_ptr, dst_bytes, producers, bytes_per_producer, nburst, gap_cycles,
                            times.data_ptr(), stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"xs_burst_gap failed with {rc}")
    torch.cuda.synchronize(torch_device)
    t = times.cpu().numpy().astype(np.float64).reshape(producers, WAVES, nburst + 3)
    clock_hz = float(np.median(t[:, :, nburst + 1] / (t[:, :, nburst + 2] * 1e-8)))
    issue = t[:, :, :nburst].max(axis=1) / clock_hz          # [producer][burst], slowest wave
    first = float(np.median(issue[:, 0]))
    steady = float(np.median(issue[:, nburst // 2:])) if nburst > 1 else first  # later half
    drain = float(np.median(t[:, :, nburst].max(axis=1))) / clock_hz
    return Run(producers, float(producers) * bytes_per_producer, gap_cycles / clock_hz, first,
               steady, drain, clock_hz)


# ---------------------------------------------------------------- the characterisation run
SWEEP_PRODUCERS = (64, 256)
SWEEP_BYTES = (16384, 65536, 262144, 1048576)              # per producer and burst
SWEEP_GAPS_US = (0.0, 5.0, 20.0, 50.0, 100.0, 200.0, 500.0, 2000.0)
NOMINAL_CLOCK_HZ = 2.1e9                                    # only to turn gaps into cycles
RING_BYTES = 512 << 20                                      # fresh addresses for every burst
RUN_BUDGET_S = 0.05                                         # rough time budget per run
DRAIN_GUESS = 40e9                                          # bytes/s, only to size the runs


def bursts_for(V: float, gap_s: float) -> int:
    """Enough bursts to fill a few hundred MiB of outstanding stores at G = 0 (so
    the later bursts are in steady state), within the run's time budget and
    the ring (every burst writes fresh addresses)."""
    n = max(4, min(512, int(RING_BYTES // V)))
    return max(4, min(n, int(RUN_BUDGET_S / (gap_s + V / DRAIN_GUESS))))


def sweep(torch_device, log=None):
    """Runs the microbenchmark over the grid into fine-grained host memory."""
    buf = HostBuffer(RING_BYTES)
    runs = []
    try:
        measure(buf.ptr, buf.nbytes, 16, STEP_BYTES, 2, 0, torch_device)  # warm-up
        for K in SWEEP_PRODUCERS:
            for b in SWEEP_BYTES:
                for g_us in SWEEP_GAPS_US:
                    r = measure(buf.ptr, buf.nbytes, K, b, bursts_for(K * b, g_us * 1e-6),
                                int(g_us * 1e-6 * NOMINAL_CLOCK_HZ), torch_device)
                    runs.append(r)
                    if log:
                        log(f"K={K} V={r.V / 2**20:.2f} MiB G={r.G * 1e6:.1f} us: "
                            f"first {r.t_first * 1e6:.2f} us, steady {r.t_steady * 1e6:.2f} us")
    finally:
        buf.free()
    return runs


def fit_runs(runs) -> Params:
    return fit([r.K for r in runs], [r.V for r in runs], [r.G for r in runs],
               [r.t_steady for r in runs], [r.t_first for r in runs])


def prediction_errors(p: Params, runs):
    """Relative errors of the model on the runs' steady and first-burst issue times."""
    K = np.array([r.K for r in runs], dtype=np.float64)
    V = np.array([r.V for r in runs])
    G = np.array([r.G for r in runs])
    ts = np.array([r.t_steady for r in runs])
    tf = np.array([r.t_first for r in runs])
    es = np.abs(predict(p, K, V, G) - ts) / ts
    ef = np.abs(predict_first(p, K, V) - tf) / tf
    return es, ef


# ---------------------------------------------------------------- the attention epilogue as bursts
def attention_overhead(w, inp, p: Params, torch_device, reps: int = 9) -> dict:
    """The attention call with out_packed in fine-grained host memory (the
    stand-in remote link) against out_packed in HBM, for a workload `w` (sizes
    B, S, H, D, P, name) with inputs `inp` (q, k, v, scale on the CPU), with the
    uncut schedule (no workspace).  Every tile owner's O
    tile (256 rows x D bf16) is one producer's burst; a round of resident
    workgroups is K = min(tiles, CUs) producers issuing V = K tile bytes, and the
    next round's key loop is their gap.  The model predicts the extra time as
    the drain the gaps do not cover plus what is still outstanding when the
    computation ends -- at most the last round's bursts, at most Q -- drained at
    R before the kernel completes:
        (rounds - 1) * max(0, V/R - G) + min(V_last + backlog, Q) / R."""
    import torch

    import sequence_attention_amd as xs

    q, k, v = (inp[n].to(torch_device) for n in "qkv")
    nbytes = w.P * w.B * (w.S // w.P) * w.H * w.D * 2
    out_dev = torch.empty(nbytes, dtype=torch.uint8, device=torch_device)
    host = HostBuffer(nbytes)
    stream = torch.cuda.current_stream(torch_device)

    def call(ptr):
        rc = xs.xs_attn_fwd_ex(q, k, v, 0, ptr, None, w.B, w.S, w.H, w.D, w.P, inp["scale"], None, 0,
                               stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"xs_attn_fwd_ex failed with {rc}")

    def timed(ptr):
        for _ in range(2):
            call(ptr)
        torch.cuda.synchronize(torch_device)
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call(ptr)
            e1.record(stream)
            torch.cuda.synchronize(torch_device)
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms)) * 1e-3

    try:
        t_dev = timed(out_dev.data_ptr())
        t_host = timed(host.ptr)
        same = bool(np.array_equal(host.view(np.uint8), out_dev.cpu().numpy()))
    finally:
        host.free()
    cus = torch.cuda.get_device_properties(torch_device).multi_processor_count
    tiles = w.B * w.H * -(-w.S // 256)
    tile_bytes = 256 * w.D * 2  # one O tile: 256 rows of one head
    rounds = -(-tiles // cus)
    V = min(tiles, cus) * tile_bytes
    V_last = (tiles - (rounds - 1) * cus) * tile_bytes
    G = t_dev / rounds
    backlog = V * (rounds - 1) - p.R * G * (rounds - 1) if rounds > 1 else 0.0
    tail = min(V_last + max(0.0, backlog), p.Q if np.isfinite(p.Q) else float("inf"))
    pred = (rounds - 1) * max(0.0, V / p.R - G) + tail / p.R
    return {"workload": w.name, "tiles": tiles, "rounds": rounds, "burst_bytes": V,
            "reps": reps,
            "gap_us": round(G * 1e6, 2), "t_hbm_ms": round(t_dev * 1e3, 4),
            "t_host_ms": round(t_host * 1e3, 4),
            "overhead_us": round((t_host - t_dev) * 1e6, 2),
            "predicted_overhead_us": round(pred * 1e6, 2), "host_output_bit_exact": same}


def characterise(torch_device, cases, log=None) -> dict:
    """The sweep, the fit with its errors and a hold-out check, and the
    attention epilogue check on `cases` = [(workload, inputs), ...]."""
    runs = sweep(torch_device, log=log)
    p = fit_runs(runs)
    es, ef = prediction_errors(p, runs)
    # hold-out check: fit on the gaps at even positions of the sweep, predict the others
    ng = len(SWEEP_GAPS_US)
    train = [r for i, r in enumerate(runs) if (i % ng) % 2 == 0]
    test = [r for i, r in enumerate(runs) if (i % ng) % 2 == 1]
    ph = fit_runs(train)
    es_h, _ = prediction_errors(ph, test)
    att = [attention_overhead(w, inp, p, torch_device) for w, inp in cases]
    return {
        "T0_iss": {"a_us": round(p.a * 1e6, 3), "ns_per_KiB_per_producer": round(p.c * 1024 * 1e9, 3)},
        "R_GBps": round(p.R / 1e9, 2),
        "Q_MiB": None if not np.isfinite(p.Q) else round(p.Q / 2**20, 2),
        "Q_bracket_MiB": [round(q / 2**20, 2) if np.isfinite(q) else None for q in p.Q_bracket],
        "steady_rel_err": {"median": round(float(np.median(es)), 4), "max": round(float(es.max()), 4)},
        "first_burst_rel_err": {"median": round(float(np.median(ef)), 4),
                                "max": round(float(ef.max()), 4)},
        "holdout_steady_rel_err": {"median": round(float(np.median(es_h)), 4),
                                   "max": round(float(es_h.max()), 4)},
        "runs": [{"K": r.K, "V_MiB": round(r.V / 2**20, 3), "G_us": round(r.G * 1e6, 2),
                  "first_us": round(r.t_first * 1e6, 3), "steady_us": round(r.t_steady * 1e6, 3),
                  "model_us": round(float(predict(p, r.K, r.V, r.G)) * 1e6, 3)} for r in runs],
        "attention": att,
    }
