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


TILE_ROWS, TILE_WAVES = 256, 8  # xs_burst_gap_tiles: one 256-row output tile per producer


def measure_tiles(dst_ptr: int, dst_bytes: int, producers: int, row_bytes: int, row_pitch: int,
                  nburst: int, gap_cycles: int, torch_device, coupled: bool = False,
                  gap_src=None, gap_loads: int = 0) -> Run:
    """One launch of the tile-pattern microbenchmark (the attention epilogue's
    stores); V counts the bytes written (producers x 256 rows x row_bytes).  With
    `coupled` the times run to the completion of each burst's stores; with
    `gap_src` (a device tensor of a power-of-two size) the gap is gap_loads loads
    of 1 KiB per wave, and Run.G is the median measured gap (slowest wave,
    later half of the bursts)."""
    import torch

    n = producers * TILE_WAVES * (2 * nburst + 3)
    times = torch.zeros(n, dtype=torch.int64, device=torch_device)
    stream = torch.cuda.current_stream(torch_device)
    src_ptr = gap_src.data_ptr() if gap_src is not None else None
    src_bytes = gap_src.numel() * gap_src.element_size() if gap_src is not None else 0
    rc = lib().xs_burst_gap_tiles(dst_ptr, dst_bytes, producers, row_bytes, row_pitch, nburst,
                                  gap_cycles, int(coupled), src_ptr, src_bytes, gap_loads,
                                  times.data_ptr(), stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"xs_burst_gap_tiles failed with {rc}")
    torch.cuda.synchronize(torch_device)
    t = times.cpu().numpy().astype(np.float64).reshape(producers, TILE_WAVES, 2 * nburst + 3)
    clock_hz = float(np.median(t[:, :, 2 * nburst + 1] / (t[:, :, 2 * nburst + 2] * 1e-8)))
    issue = t[:, :, :nburst].max(axis=1) / clock_hz
    gaps = t[:, :, nburst:2 * nburst].max(axis=1) / clock_hz
    first = float(np.median(issue[:, 0]))
    steady = float(np.median(issue[:, nburst // 2:])) if nburst > 1 else first
    drain = float(np.median(t[:, :, 2 * nburst].max(axis=1))) / clock_hz
    G = float(np.median(gaps[:, nburst // 2:])) if gap_src is not None else gap_cycles / clock_hz
    return Run(producers, float(producers) * TILE_ROWS * row_bytes, G, first, steady, drain,
               clock_hz)


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
        warm_ring(buf, torch_device)
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


TILE_SWEEP_PRODUCERS = (16, 64, 256)
TILE_SWEEP_GAPS_US = (0.0, 5.0, 20.0, 50.0, 100.0, 200.0, 500.0, 1000.0, 2000.0)


def warm_ring(buf, torch_device):
    """Writes every byte of the host ring once from the GPU, so that no measured
    burst is the first to touch its pages."""
    per = buf.nbytes // 256
    measure(buf.ptr, buf.nbytes, 256, per - per % STEP_BYTES, 1, 0, torch_device)


def sweep_tiles(torch_device, row_bytes: int, row_pitch: int, log=None):
    """The tile-pattern microbenchmark over producers and gaps into fine-grained
    host memory: K producers each store one 256-row tile per burst (rows
    row_pitch bytes apart, as in the destination-ordered buffer of a share with
    H_local = row_pitch / row_bytes heads)."""
    buf = HostBuffer(RING_BYTES)
    runs = []
    try:
        warm_ring(buf, torch_device)
        for K in TILE_SWEEP_PRODUCERS:
            span = K * TILE_ROWS * row_pitch  # address range of one burst
            for g_us in TILE_SWEEP_GAPS_US:
                V = K * TILE_ROWS * row_bytes
                n = max(4, min(256, int(RUN_BUDGET_S / (g_us * 1e-6 + V / 30e9))))
                n = max(4, min(n, 4 * int(RING_BYTES // span)))
                r = measure_tiles(buf.ptr, buf.nbytes, K, row_bytes, row_pitch, n,
                                  int(g_us * 1e-6 * NOMINAL_CLOCK_HZ), torch_device)
                runs.append(r)
                if log:
                    log(f"tiles K={K} V={r.V / 2**20:.2f} MiB G={r.G * 1e6:.1f} us: "
                        f"first {r.t_first * 1e6:.2f} us, steady {r.t_steady * 1e6:.2f} us")
    finally:
        buf.free()
    return runs


COUPLED_PRODUCERS = (8, 16, 32, 54, 64, 128, 192, 256)
COUPLED_GAP_US = 2000.0  # bursts far apart: each one's completion time on its own


@dataclass
class Coupled:
    a: float  # s, fixed part of a burst's completion time
    R: float  # bytes/s, completion rate of a burst's stores
    runs: list

    def t(self, V):
        return self.a + np.asarray(V, dtype=np.float64) / self.R


def sweep_coupled(torch_device, row_bytes: int, row_pitch: int, log=None) -> Coupled:
    """Completion time of one tile burst from K producers that wait for their
    stores before the gap (what the attention kernels' waves do), isolated by a
    long gap; fitted as T_c(V) = a + V / R_c (least squares, weighted 1/T_c)."""
    buf = HostBuffer(RING_BYTES)
    runs = []
    try:
        warm_ring(buf, torch_device)
        for K in COUPLED_PRODUCERS:
            span = K * TILE_ROWS * row_pitch
            n = max(4, min(12, 4 * int(RING_BYTES // span)))
            r = measure_tiles(buf.ptr, buf.nbytes, K, row_bytes, row_pitch, n,
                              int(COUPLED_GAP_US * 1e-6 * NOMINAL_CLOCK_HZ), torch_device,
                              coupled=True)
            runs.append(r)
            if log:
                log(f"coupled tiles K={K} V={r.V / 2**20:.2f} MiB: completion {r.t_steady * 1e6:.2f} us")
    finally:
        buf.free()
    V = np.array([r.V for r in runs])
    t = np.array([r.t_steady for r in runs])
    w = 1.0 / t
    A = np.stack([np.ones_like(V), V], axis=1) * w[:, None]
    (a, inv_r), *_ = np.linalg.lstsq(A, t * w, rcond=None)
    return Coupled(float(a), float(1.0 / inv_r), runs)


LOADGAP_PRODUCERS = (54, 128, 256)
LOADGAP_LOADS = 128        # 1 KiB loads per wave per gap (128 KiB per wave)
LOADGAP_SRC_BYTES = 1 << 30


def sweep_loadgap(torch_device, row_bytes: int, row_pitch: int, log=None) -> list:
    """The gap as the next tile's key loop sees it -- loads from device memory --
    after a burst of output tiles into host memory, against the same run with
    the burst into device memory: the difference is the time the burst's drain
    takes away from the loads that follow it (per burst, median of the later
    half of 8 bursts)."""
    import torch

    buf = HostBuffer(RING_BYTES)
    src = torch.ones(LOADGAP_SRC_BYTES // 4, dtype=torch.int32, device=torch_device)
    res = []
    try:
        warm_ring(buf, torch_device)
        for K in LOADGAP_PRODUCERS:
            span = K * TILE_ROWS * row_pitch
            dev = torch.empty(span, dtype=torch.uint8, device=torch_device)
            runs = {}
            for name, ptr, nbytes in (("hbm", dev.data_ptr(), span), ("host", buf.ptr, buf.nbytes),
                                      ("hbm2", dev.data_ptr(), span)):
                runs[name] = measure_tiles(ptr, nbytes, K, row_bytes, row_pitch, 8, 0, torch_device,
                                           gap_src=src, gap_loads=LOADGAP_LOADS)
            g_dev = 0.5 * (runs["hbm"].G + runs["hbm2"].G)
            r = {"K": K, "V_MiB": round(runs["host"].V / 2**20, 3),
                 "gap_after_hbm_burst_us": round(g_dev * 1e6, 2),
                 "gap_after_host_burst_us": round(runs["host"].G * 1e6, 2),
                 "stretch_us": round((runs["host"].G - g_dev) * 1e6, 2)}
            res.append(r)
            if log:
                log(f"load gap K={K}: {r}")
            del dev
    finally:
        buf.free()
    return res


END_PRODUCERS = (8, 32, 54, 128, 256)


def sweep_end_drain(torch_device, row_bytes: int, row_pitch: int, log=None, reps: int = 7) -> list:
    """What a kernel's end adds after its last burst into host memory: a launch
    of one tile burst (K producers, no gap), timed with events around the launch,
    against the kernel's own walk (first store to the drain of its last store,
    s_memrealtime) -- the kernel completes only once its writes are visible to
    the host.  The same launch into device memory gives the fixed launch cost;
    end_us is the host launch's excess over it (median of reps launches)."""
    import torch

    buf = HostBuffer(RING_BYTES)
    res = []
    try:
        warm_ring(buf, torch_device)
        stream = torch.cuda.current_stream(torch_device)
        for K in END_PRODUCERS:
            span = K * TILE_ROWS * row_pitch
            dev = torch.empty(span, dtype=torch.uint8, device=torch_device)
            out = {}
            for name, ptr, nbytes in (("hbm", dev.data_ptr(), span), ("host", buf.ptr, buf.nbytes)):
                ms = []
                for _ in range(reps):
                    times = torch.zeros(K * TILE_WAVES * 5, dtype=torch.int64, device=torch_device)
                    torch.cuda.synchronize(torch_device)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    rc = lib().xs_burst_gap_tiles(ptr, nbytes, K, row_bytes, row_pitch, 1, 0, 0, None,
                                                  0, 0, times.data_ptr(), stream.cuda_stream)
                    e1.record(stream)
                    torch.cuda.synchronize(torch_device)
                    if rc != 0:
                        raise RuntimeError(f"xs_burst_gap_tiles failed with {rc}")
                    ms.append(e0.elapsed_time(e1) * 1e-3)
                out[name] = float(np.median(ms))
            r = {"K": K, "V_MiB": round(K * TILE_ROWS * row_bytes / 2**20, 3),
                 "launch_hbm_us": round(out["hbm"] * 1e6, 2), "launch_host_us": round(out["host"] * 1e6, 2),
                 "end_us": round((out["host"] - out["hbm"]) * 1e6, 2)}
            res.append(r)
            if log:
                log(f"end drain K={K}: {r}")
            del dev
    finally:
        buf.free()
    return res


@dataclass
class Linear:
    """y(V) = a + V / R, fitted by least squares (weighted 1/y)."""
    a: float
    R: float

    def __call__(self, V):
        return self.a + np.asarray(V, dtype=np.float64) / self.R


def fit_linear(V, y, through_origin: bool = False) -> Linear:
    V, y = np.asarray(V, dtype=np.float64), np.asarray(y, dtype=np.float64)
    if through_origin:
        return Linear(0.0, float(np.sum(V * V) / max(np.sum(V * y), 1e-30)))
    w = 1.0 / np.maximum(np.abs(y), 1e-9)
    A = np.stack([np.ones_like(V), V], axis=1) * w[:, None]
    (a, inv_r), *_ = np.linalg.lstsq(A, y * w, rcond=None)
    return Linear(float(a), float(1.0 / inv_r))


def predict_attention_end(end: Linear, stretch: Linear, tiles: int, cus: int,
                          tile_bytes: float) -> float:
    """The extra time of an attention call whose output tiles go to host memory,
    from what the microbenchmark measures for the epilogue's store pattern: each
    round's burst of min(tiles, CUs) tiles slows the loads of the next round's
    key loop by stretch(V) (the loads share the memory pipeline with the
    draining writes), and the kernel cannot end before its last round's burst
    has drained to the host: end(V_last)."""
    rounds = -(-tiles // cus)
    t = 0.0
    for r in range(rounds - 1):
        t += max(0.0, float(stretch(cus * tile_bytes)))
    return t + float(end((tiles - (rounds - 1) * cus) * tile_bytes))


def predict_attention_coupled(pc: Coupled, tiles: int, cus: int, tile_bytes: float) -> float:
    """Completion-coupled prediction: every round's output tiles are waited for
    (before the next tile's first barrier, or at the kernel's end), so each
    round of min(tiles, CUs) producers adds the completion time of its burst."""
    rounds = -(-tiles // cus)
    total = 0.0
    for r in range(rounds):
        k = min(cus, tiles - r * cus)
        total += float(pc.t(k * tile_bytes))
    return total


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
def predict_attention(p: Params, tiles: int, cus: int, tile_bytes: float, t_dev: float) -> float:
    """The model's extra time of the attention call when its output tiles cross
    the link: rounds of min(tiles, CUs) producers issue V bytes each, the next
    round's key loop (t_dev / rounds) is their gap; the drain the gaps do not
    cover accumulates, and what is outstanding when the computation ends -- at
    most the last round's bursts plus that backlog, at most Q -- drains at R
    before the kernel completes."""
    rounds = -(-tiles // cus)
    V = min(tiles, cus) * tile_bytes
    V_last = (tiles - (rounds - 1) * cus) * tile_bytes
    G = t_dev / rounds
    backlog = V * (rounds - 1) - p.R * G * (rounds - 1) if rounds > 1 else 0.0
    tail = min(V_last + max(0.0, backlog), p.Q if np.isfinite(p.Q) else float("inf"))
    return (rounds - 1) * max(0.0, V / p.R - G) + tail / p.R


def attention_overhead(w, inp, p: Params, torch_device, reps: int = 21, p_tiles: Params = None,
                       p_coupled: Coupled = None, p_end: tuple = None) -> dict:
    """The attention call with out_packed in fine-grained host memory (the
    stand-in remote link) against out_packed in HBM, for a workload `w` (sizes
    B, S, H, D, P, name) with inputs `inp` (q, k, v, scale on the CPU), with the
    uncut schedule in one launch (no workspace, XS_ONE_LAUNCH).  Every tile owner's O
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

    # both outputs under the same schedule: an output behind a link never takes the
    # second, half-tile launch, so the device-memory run is held to one launch too
    def call(ptr):
        rc = xs.xs_attn_fwd_ex(q, k, v, xs.LAYOUT_BSHD | xs.ONE_LAUNCH, ptr, None, w.B, w.S, w.H,
                               w.D, w.P, inp["scale"], None, 0, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"xs_attn_fwd_ex failed with {rc}")

    def once(ptr):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call(ptr)
        e1.record(stream)
        torch.cuda.synchronize(torch_device)
        return e0.elapsed_time(e1) * 1e-3

    try:
        for _ in range(2):
            call(out_dev.data_ptr())
            call(host.ptr)
        torch.cuda.synchronize(torch_device)
        # interleaved pairs, so that clock and power drift hit both alike
        td, th = [], []
        for i in range(reps):
            if i % 2:
                th.append(once(host.ptr))
                td.append(once(out_dev.data_ptr()))
            else:
                td.append(once(out_dev.data_ptr()))
                th.append(once(host.ptr))
        t_dev, t_host = float(np.median(td)), float(np.median(th))
        diff = np.array(th) - np.array(td)
        same = bool(np.array_equal(host.view(np.uint8), out_dev.cpu().numpy()))
    finally:
        host.free()
    cus = torch.cuda.get_device_properties(torch_device).multi_processor_count
    tiles = w.B * w.H * -(-w.S // 256)
    tile_bytes = 256 * w.D * 2  # one O tile: 256 rows of one head
    rounds = -(-tiles // cus)
    pred = predict_attention(p, tiles, cus, tile_bytes, t_dev)
    res = {"workload": w.name, "tiles": tiles, "rounds": rounds,
           "burst_bytes": min(tiles, cus) * tile_bytes, "reps": reps,
           "gap_us": round(t_dev / rounds * 1e6, 2), "t_hbm_ms": round(t_dev * 1e3, 4),
           "t_host_ms": round(t_host * 1e3, 4),
           "overhead_us": round(float(np.median(diff)) * 1e6, 2),
           "overhead_iqr_us": [round(float(np.percentile(diff, 25)) * 1e6, 2),
                               round(float(np.percentile(diff, 75)) * 1e6, 2)],
           "predicted_overhead_us": round(pred * 1e6, 2), "host_output_bit_exact": same}
    if p_tiles is not None:
        res["predicted_overhead_tiles_fit_us"] = round(
            predict_attention(p_tiles, tiles, cus, tile_bytes, t_dev) * 1e6, 2)
    if p_coupled is not None:
        res["predicted_overhead_coupled_us"] = round(
            predict_attention_coupled(p_coupled, tiles, cus, tile_bytes) * 1e6, 2)
    if p_end is not None:
        res["predicted_overhead_end_drain_us"] = round(
            predict_attention_end(p_end[0], p_end[1], tiles, cus, tile_bytes) * 1e6, 2)
    return res


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
    # the epilogue's own store pattern: 16 bytes into each of 32 rows per store
    # instruction, rows H*D*2 bytes apart -- fitted per head count of the cases
    tiles_fit = {}
    for w, _ in cases:
        key = (w.D * 2, w.H * w.D * 2)
        if key not in tiles_fit:
            truns = sweep_tiles(torch_device, key[0], key[1], log=log)
            pt = fit_runs(truns)
            ets, etf = prediction_errors(pt, truns)
            pc = sweep_coupled(torch_device, key[0], key[1], log=log)
            lg = sweep_loadgap(torch_device, key[0], key[1], log=log)
            ed = sweep_end_drain(torch_device, key[0], key[1], log=log)
            end = fit_linear([r["V_MiB"] * 2**20 for r in ed], [r["end_us"] * 1e-6 for r in ed])
            stretch = fit_linear([r["V_MiB"] * 2**20 for r in lg],
                                 [max(0.0, r["stretch_us"]) * 1e-6 for r in lg], through_origin=True)
            tiles_fit[key] = (pt, ets, etf, truns, pc, lg, ed, end, stretch)
    att = []
    for w, inp in cases:
        f = tiles_fit[(w.D * 2, w.H * w.D * 2)]
        att.append(attention_overhead(w, inp, p, torch_device, p_tiles=f[0], p_coupled=f[4],
                                      p_end=(f[7], f[8])))
    tile_report = []
    for (rb, pitch), (pt, ets, etf, truns, pc, lg, ed, end, stretch) in tiles_fit.items():
        tile_report.append({
            "row_bytes": rb, "row_pitch": pitch, "load_gap": lg, "end_drain": ed,
            "end_fit": {"a_us": round(end.a * 1e6, 2), "R_GBps": round(end.R / 1e9, 2)},
            "stretch_fit": {"R_GBps": round(stretch.R / 1e9, 2)},
            "coupled": {"a_us": round(pc.a * 1e6, 3), "R_GBps": round(pc.R / 1e9, 2),
                        "runs": [{"K": r.K, "V_MiB": round(r.V / 2**20, 3),
                                  "completion_us": round(r.t_steady * 1e6, 3),
                                  "model_us": round(float(pc.t(r.V)) * 1e6, 3)}
                                 for r in pc.runs]},
            "T0_iss": {"a_us": round(pt.a * 1e6, 3),
                       "ns_per_KiB_per_producer": round(pt.c * 1024 * 1e9, 3)},
            "R_GBps": round(pt.R / 1e9, 2),
            "Q_MiB": None if not np.isfinite(pt.Q) else round(pt.Q / 2**20, 2),
            "Q_bracket_MiB": [round(q / 2**20, 2) if np.isfinite(q) else None for q in pt.Q_bracket],
            "steady_rel_err": {"median": round(float(np.median(ets)), 4),
                               "max": round(float(ets.max()), 4)},
            "first_burst_rel_err": {"median": round(float(np.median(etf)), 4),
                                    "max": round(float(etf.max()), 4)},
            "runs": [{"K": r.K, "V_MiB": round(r.V / 2**20, 3), "G_us": round(r.G * 1e6, 2),
                      "first_us": round(r.t_first * 1e6, 3), "steady_us": round(r.t_steady * 1e6, 3),
                      "model_us": round(float(predict(pt, r.K, r.V, r.G)) * 1e6, 3)}
                     for r in truns]})
    return {
        "tile_pattern": tile_report,
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
