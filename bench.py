"""Benchmark: fused Ulysses-share attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload video|image|long|fp8|tiny]

One step is one call of the whole path -- attention over the full sequence for
every head of the share plus the destination-ordered epilogue -- on inputs
already resident in HBM.  Prints one JSON line.  The default workload is the
S=32768, D=128 video share (B=1, H_local=5, P=8), bf16.

The line carries the roofline of the (single) kernel -- algorithmic flops per
launch over the mean launch time measured with HIP events on the launch stream
-- and a CPU baseline: the fp64 oracle timed on a bounded sample of query rows
of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads  # noqa: E402

METRIC = "attention TFLOP/s (4·B·H·S²·D) + % MFMA peak, S=32768 D=128 bf16"
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}  # MI355X published dense MFMA peaks


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="video", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=25.0,
                    help="target wall time of the CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--samples", type=int, default=20,
                    help="timed launches also bracketed by their own events (roofline launch "
                         "time): every max(4, K/samples)-th call")
    ap.add_argument("--in-layout", default="bshd", choices=["bshd", "chunked"],
                    help="input layout: [B][S][H][D] or the pre-attention All-to-All chunk layout "
                         "[P][B][S/P][H][D] (converted once, before timing)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step (the attention kernel and, when the plan splits, the "
                         "merge kernel) in a HIP graph and replay it per step: removes the host "
                         "launch cost that bounds the short workloads")
    ap.add_argument("--cold", action="store_true",
                    help="write a 512 MiB buffer before every timed call (evicts L2 and MALL) and "
                         "report the per-call event times instead of the back-to-back step time")
    ap.add_argument("--no-check", action="store_true", help="skip the sampled parity check")
    ap.add_argument("--no-plain-entry", action="store_true",
                    help="skip the extra timing of xs_attn_fwd / xs_attn_fwd_fp8 without workspace "
                         "(for profiling runs whose dispatches should be the timed calls only)")
    ap.add_argument("--burst-gap", action="store_true",
                    help="characterise the Burst-Gap model with the microbenchmark (fine-grained "
                         "host memory as the remote link) and check it on the attention epilogue")
    ap.add_argument("--epilogue-overhead", action="store_true",
                    help="time the fused destination-ordered epilogue against a plain [B][S][H][D] "
                         "epilogue and against attention followed by a separate relayout")
    ap.add_argument("--torch-sdpa", action="store_true",
                    help="context: time torch's own fused attention (scaled_dot_product_attention, "
                         "flash backend only) on the same inputs next to this library's call")
    ap.add_argument("--power", type=float, default=0.0, metavar="SECONDS",
                    help="instead of the timed steps, run back-to-back steps for SECONDS while "
                         "sampling the socket power and GFX clocks with amd-smi; report the "
                         "energy per step")
    ap.add_argument("--ceilings", action="store_true",
                    help="instead of the benchmark, run the matrix-core ceiling probes "
                         "(xs_mfma_ceiling: MFMA rate next to LDS operand reads and softmax "
                         "vector work, one and two waves per SIMD); with --power, the socket "
                         "power and matrix work per joule of probe modes 0, 5 and 7-12 instead")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run a plain device copy of MIB MiB (the "
                         "reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def copy_calibration(mib, steps):
    """A plain device-to-device copy of a known size, for counter calibration."""
    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n * 4, "bytes_written": n * 4,
                                           "launches": steps}}), flush=True)


CEILING_MODES = ["mfma only", "1 KiB ds_read_b128 per MFMA", "0.5 KiB ds_read_b128 per MFMA",
                 "1 KiB ds_read_b64_tr_b16 per MFMA",
                 "softmax work per MFMA (fma, exp, add, half a bf16 pack)",
                 "softmax work + 1 KiB ds_read_b128 per MFMA (32 query rows per wave)",
                 "softmax work + 0.5 KiB ds_read_b128 per MFMA (64 query rows per wave)",
                 "mfma only, N(0, 1) bf16 operands",
                 "softmax work + 1 KiB ds_read_b128 per MFMA, N(0, 1) bf16 data",
                 "mfma only, N(0, 1) bf16 operands, as two 16x16x32 MFMAs",
                 "mode 8 with two 16x16x32 MFMAs sharing the LDS fragment",
                 "fp8 MFMAs (32x32x64, 64 clocks) only, e4m3 operands like the fp8 share's",
                 "fp8 kernel's mix: 2 KiB LDS operand + codes (4 FMA, 2 pknorm, perm, 2 max3) per MFMA, e4m3 data"]
# modes whose MFMA is the fp8 32x32x64 one (four times the multiply-adds of a bf16
# 32x32x16, in twice the clocks)
CEILING_FP8_MODES = (11, 12)


def ceilings(iters, reps=5):
    """MFMA issue rate of each xs_mfma_ceiling mode against MFMA-only issue with the same
    number of waves per SIMD (minimum time over `reps` launches after one warm-up)."""
    from sequence_attention_amd import _lib

    L = _lib.lib()
    stream = torch.cuda.current_stream()
    sink = torch.empty(1024 * 512, dtype=torch.float32, device="cuda:0")

    def run(mode, waves):
        best = None
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            _lib.check(L.xs_mfma_ceiling(mode, waves, iters, ctypes.c_void_p(sink.data_ptr()),
                                          sink.numel() * 4, ctypes.c_void_p(stream.cuda_stream)))
            e1.record(stream)
            e1.synchronize()
            t = e0.elapsed_time(e1)
            if r and (best is None or t < best):
                best = t
        return best

    res = {}
    for waves in (2, 1):
        base = run(0, waves)
        mfma_per_simd = 1024 / 256 * waves * 16 * iters
        rows = []
        for mode, name in enumerate(CEILING_MODES):
            t = base if mode == 0 else run(mode, waves)
            rows.append({"mode": mode, "stream": name, "ms": round(t, 4),
                         "mfma_rate_vs_mfma_only": round(base / t, 4)})
        res[f"{waves}_waves_per_simd"] = {
            "mfma_only_clock_ghz": round(mfma_per_simd * 32 / (base * 1e-3) / 1e9, 3), "modes": rows}
    return res


def ceiling_power(seconds, modes=(0, 5, 7, 8, 9, 10, 11, 12), iters=2048):
    """Socket power, GFX clock and matrix work per joule of probe modes run back to back
    (two waves per SIMD) for `seconds` each, sampled as in power_run."""
    from sequence_attention_amd import _lib

    L = _lib.lib()
    stream = torch.cuda.current_stream()
    sink = torch.empty(1024 * 512, dtype=torch.float32, device="cuda:0")
    flops = 1024 * 8 * 16 * iters * 32 * 32 * 16 * 2.0
    out = []
    for mode in modes:
        def step(mode=mode):
            _lib.check(L.xs_mfma_ceiling(mode, 2, iters, ctypes.c_void_p(sink.data_ptr()),
                                          sink.numel() * 4, ctypes.c_void_p(stream.cuda_stream)))
        step()
        torch.cuda.synchronize()
        f = flops * (4 if mode in CEILING_FP8_MODES else 1)
        out.append({"mode": mode, "stream": CEILING_MODES[mode], **power_run(step, seconds, f)})
        print(f"ceiling power mode {mode} done", file=sys.stderr, flush=True)
    return out


def smi_parse(text):
    """(socket power in W, mean GFX clock in MHz over the XCDs) from the text of
    `amd-smi metric -p -c`, or None when a field is missing."""
    import re

    m = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", text)
    clocks, in_gfx = [], False
    for line in text.splitlines():
        if re.match(r"\s*GFX_\d+:", line):
            in_gfx = True
        elif in_gfx and re.match(r"\s*CLK:", line):
            clocks.append(float(re.findall(r"[0-9.]+", line)[0]))
            in_gfx = False
    if not m or not clocks:
        return None
    return float(m.group(1)), sum(clocks) / len(clocks)


def smi_sample():
    """One amd-smi sample (see smi_parse), or None when the tool is not there."""
    import subprocess

    try:
        out = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True,
                             timeout=10).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    return smi_parse(out)


def power_run(step, seconds, flops):
    """Back-to-back steps for `seconds` while a thread samples amd-smi every 0.25 s;
    samples of the first second (clock ramp) are dropped."""
    import threading

    idle = smi_sample()
    samples, stop = [], threading.Event()
    t0 = time.time()

    def sampler():
        while not stop.is_set():
            v = smi_sample()
            if v is not None:
                samples.append((time.time() - t0, *v))
            stop.wait(0.25)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    n = 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    while time.time() - t0 < seconds:
        for _ in range(20):
            step()
        n += 20
        torch.cuda.current_stream().synchronize()
    e1.record()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    ms = e0.elapsed_time(e1) / n
    steady = [s for s in samples if s[0] >= 1.0] or samples
    if not steady:
        return {"available": False}
    watts = sum(s[1] for s in steady) / len(steady)
    mhz = sum(s[2] for s in steady) / len(steady)
    return {"available": True, "steps": n, "ms_per_step": round(ms, 4),
            "value_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "socket_w_mean": round(watts, 1), "gfx_mhz_mean": round(mhz, 1),
            "samples": len(steady), "idle_socket_w": idle[0] if idle else None,
            "joules_per_step": round(watts * ms * 1e-3, 4),
            "tflop_per_joule": round(flops / (watts * ms * 1e-3) / 1e12, 4)}


def recorded_traffic(kernel_tag, workload):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, or
    None when there is none for this workload or the kernel sources changed since it was taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256(b"".join(open(os.path.join(ROOT, s), "rb").read() for s in rec["sources"]))
    if h.hexdigest() != rec["kernel_sources_sha256"]:
        return None
    return rec["traffic_bytes_per_launch"]


def profile_clock(kernel_tag, workload, achieved, peak):
    """The shader clock the kernel ran at in its committed rocprofv3 profile
    (SQ_BUSY_CYCLES per shader engine over the dispatch time), when the record
    still matches the kernel sources; the published peak assumes 2.4 GHz."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256(b"".join(open(os.path.join(ROOT, s), "rb").read() for s in rec["sources"]))
    ghz = rec.get("shader_clock_ghz_from_counters")
    if h.hexdigest() != rec["kernel_sources_sha256"] or ghz is None:
        return None
    return {"sclk_ghz": round(ghz, 3),
            "source": f"profiles/{kernel_tag}_{workload}.md: SQ_BUSY_CYCLES / 32 shader engines over "
                      "the mean dispatch time of that profile's counter runs (another run of this "
                      "kernel, not this one)",
            "peak_at_that_clock": round(peak * ghz / 2.4, 1),
            "frac_at_that_clock": round(achieved / (peak * ghz / 2.4), 4)}


def clock_sample(L, buf, stream):
    """Queue one xs_clock_sample on `stream` into the device buffer `buf`; returns the
    constant counter's rate in kHz."""
    khz = ctypes.c_int(0)
    from sequence_attention_amd import _lib
    _lib.check(L.xs_clock_sample(ctypes.c_void_p(buf.data_ptr()), buf.numel() * 8, ctypes.byref(khz),
                                 ctypes.c_void_p(stream.cuda_stream)))
    return khz.value


def live_clock(before, after, wall_khz):
    """Mean shader clock (GHz) of each XCC between two xs_clock_sample records (rows
    [memtime, realtime, xcc, hw_id]): per compute unit (xcc, hw_id bits 8-15) seen in
    both, memtime cycles over the constant counter's elapsed time; the median over an
    XCC's compute units."""
    def first_by_cu(rec):
        out = {}
        for t, r, x, hw in np.asarray(rec, dtype=np.int64).reshape(-1, 4):
            out.setdefault((int(x), (int(hw) >> 8) & 0xFF), (int(t), int(r)))
        return out
    a, b = first_by_cu(before), first_by_cu(after)
    per = {}
    for key in set(a) & set(b):
        dt, dr = b[key][0] - a[key][0], b[key][1] - a[key][1]
        if dt > 0 and dr > 0 and wall_khz > 0:
            per.setdefault(key[0], []).append(dt / (dr / (wall_khz * 1e3)) / 1e9)
    return {x: float(np.median(v)) for x, v in sorted(per.items())}


def run_clock(xcc_ghz, value, achieved, peak, profile):
    """The bench line's clock record: the live per-XCC shader clock of the timed
    launches, the published peak scaled to its mean, and the profile's figure."""
    if not xcc_ghz:
        return {"sclk_ghz": None, "profile": profile}
    mean = float(np.mean(list(xcc_ghz.values())))
    at = peak * mean / 2.4
    return {"sclk_ghz": round(mean, 3),
            "per_xcc_ghz": {str(k): round(v, 3) for k, v in xcc_ghz.items()},
            "source": "xs_clock_sample before and after the timed launches on their stream: "
                      "s_memtime cycles over s_memrealtime time per compute unit, median per XCC",
            "peak_at_that_clock": round(at, 1),
            "value_frac_at_that_clock": round(value / at, 4),
            "frac_at_that_clock": round(achieved / at, 4),
            "profile": profile}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, inp, target_s):
    """Time the fp64 oracle on a deterministic sample of rows; scale to TFLOP/s."""
    from oracle import oracle

    threads = oracle.default_threads()
    per_row = 4.0 * w.S * w.D  # algorithmic flops of one query row
    total = w.B * w.S * w.H

    def probe(n, seed):
        rows = workloads.sample_rows(w, n, seed=seed)
        t0 = time.perf_counter()
        oracle.attention_rows(inp["q"], inp["k"], inp["v"], rows, inp["scale"], inp["descales"],
                              threads)
        return time.perf_counter() - t0

    # Each oracle call first decodes the whole of q, k and v once, a fixed cost
    # that a small probe would take for per-row time: two probe sizes separate
    # the two, and the sample is sized so that the timed call lasts target_s.
    n1 = min(max(threads, 8), total)
    n2 = min(4 * n1, total)
    t1 = probe(n1, 11)
    t2 = probe(n2, 11)
    per = (t2 - t1) / (n2 - n1) if n2 > n1 and t2 > t1 else t2 / n2
    fixed = max(0.0, t2 - per * n2)
    n = int(min(max(n1, (target_s - fixed) / max(per, 1e-9)), total))
    n = max(min(threads, total), (n // threads) * threads)
    rows = workloads.sample_rows(w, n, seed=12)
    t0 = time.perf_counter()
    oracle.attention_rows(inp["q"], inp["k"], inp["v"], rows, inp["scale"], inp["descales"], threads)
    dt = time.perf_counter() - t0
    return {
        "value": per_row * len(rows) / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "extrapolated": len(rows) < total,
        "sample": f"{len(rows)} of {total} query rows ({100.0 * len(rows) / total:.2f} %) of the "
                  f"{w.name} workload (all {w.S} keys each), {dt:.1f} s wall, fp64; the rate is "
                  f"extrapolated linearly to the whole workload (rows are independent)",
    }


def epilogue_overhead(args):
    """The fused epilogue's cost: the same kernel and schedule writing
    (a) a plain [B][S][H][D] output (P = 1, the identity relayout),
    (b) the P-way destination-ordered buffer (the product path), and
    (c) (a) followed by a separate relayout pass into the P-way buffer (torch
        copy of a permuted view) -- the serial analogue;
    on the video share (B = 1: the P-way buffer is byte-identical to [B][S][H][D])
    and on a B = 2 share (the relayout moves data).  Results must agree bit for bit."""
    import sequence_attention_amd as xs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    cases = [workloads.WORKLOADS["video"],
             workloads.custom(2, 32768, 4, 128, 8, index=4, name="video_b2")]
    results = []
    for w in cases:
        inp = workloads.make_inputs(w)
        q, k, v = (inp[n].to(dev) for n in "qkv")
        ws_bytes = xs.workspace_size(w.B, w.S, w.H, w.D)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
        plain = torch.empty((1, w.B, w.S, w.H, w.D), dtype=torch.bfloat16, device=dev)
        packed = torch.empty((w.P, w.B, w.S // w.P, w.H, w.D), dtype=torch.bfloat16, device=dev)
        serial = torch.empty_like(packed)

        def run_plain():
            xs.fwd(q, k, v, 1, inp["scale"], out=plain, stream=stream, workspace=ws)

        def run_packed():
            xs.fwd(q, k, v, w.P, inp["scale"], out=packed, stream=stream, workspace=ws)

        def run_serial():
            run_plain()
            serial.copy_(plain[0].view(w.B, w.P, w.S // w.P, w.H, w.D).permute(1, 0, 2, 3, 4))

        fns = (("plain", run_plain), ("packed", run_packed), ("serial", run_serial))
        for _ in range(args.warmup):
            for _, fn in fns:
                fn()
        torch.cuda.synchronize()
        # interleaved, so clock and power drift hit the three variants alike
        samples = {name: [] for name, _ in fns}
        for _ in range(args.steps):
            for name, fn in fns:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                samples[name].append(e0.elapsed_time(e1))
        times = {name: float(np.median(v)) for name, v in samples.items()}
        same = bool(torch.equal(packed.view(torch.int16), serial.view(torch.int16)))
        results.append({"workload": w.name, "B": w.B, "H": w.H, "S": w.S, "P": w.P,
                        "plain_ms": round(times["plain"], 4), "packed_ms": round(times["packed"], 4),
                        "serial_ms": round(times["serial"], 4),
                        "packed_vs_plain_pct": round(100 * (times["packed"] / times["plain"] - 1), 2),
                        "serial_vs_plain_pct": round(100 * (times["serial"] / times["plain"] - 1), 2),
                        "packed_equals_serial_bitwise": same})
    print(json.dumps({"metric": "epilogue_overhead", "n_gpus": 1, "steps": args.steps,
                      "warmup": args.warmup, "results": results}), flush=True)


def torch_sdpa(args):
    """Context, not part of the path: torch's own fused attention kernel
    (scaled_dot_product_attention restricted to its flash backend, so it raises
    instead of falling back to the unfused math path) against this library's
    call, on the same resident bf16 inputs, interleaved per call (medians).
    Torch writes [B][S][H][D]; for B = 1 that is byte-identical to the P-way
    destination-ordered buffer, for B > 1 a separate relayout copy follows and
    is timed with it.  The two outputs are compared element by element."""
    import sequence_attention_amd as xs
    from torch.nn.attention import SDPBackend, sdpa_kernel

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sdpa = torch.nn.functional.scaled_dot_product_attention
    cases = [workloads.WORKLOADS[n] for n in ("image", "video", "long")]
    cases.append(workloads.custom(2, 32768, 4, 128, 8, index=4, name="video_b2"))
    results = []
    for w in cases:
        inp = workloads.make_inputs(w)
        q, k, v = (inp[n].to(dev) for n in "qkv")
        qt, kt, vt = (t.transpose(1, 2) for t in (q, k, v))  # [B][H][S][D] views, no copy
        ws_bytes = xs.workspace_size(w.B, w.S, w.H, w.D)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
        out = torch.empty((w.P, w.B, w.S // w.P, w.H, w.D), dtype=torch.bfloat16, device=dev)
        ref = torch.empty_like(out)
        T = w.S // w.P

        def run_xs():
            xs.fwd(q, k, v, w.P, inp["scale"], out=out, stream=stream, workspace=ws)

        def run_torch():
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                o = sdpa(qt, kt, vt, scale=inp["scale"])
            if w.B > 1:  # [B][S][H][D] -> [P][B][S/P][H][D]
                ref.copy_(o.transpose(1, 2).view(w.B, w.P, T, w.H, w.D).permute(1, 0, 2, 3, 4))
            return o

        fns = (("xs", run_xs), ("torch", run_torch))
        for _ in range(3):
            for _, fn in fns:
                fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _, fn in fns:
            fn()
        torch.cuda.synchronize()
        # about 3 s of timed calls per workload, at most --steps
        steps = int(min(args.steps, max(5, 3.0 / (time.perf_counter() - t0))))
        for _ in range(min(args.warmup, steps)):
            for _, fn in fns:
                fn()
        torch.cuda.synchronize()
        samples = {name: [] for name, _ in fns}
        for _ in range(steps):
            for name, fn in fns:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                samples[name].append(e0.elapsed_time(e1))
        o = run_torch()
        run_xs()
        torch.cuda.synchronize()
        if w.B == 1:
            assert o.transpose(1, 2).is_contiguous(), "torch output is not [B][S][H][D]"
            ref.view(-1).copy_(o.transpose(1, 2).reshape(-1))
        t = {name: float(np.median(s)) for name, s in samples.items()}
        results.append({"workload": w.name, "B": w.B, "H": w.H, "S": w.S, "D": w.D, "P": w.P,
                        "steps": steps, "xs_ms": round(t["xs"], 4), "torch_ms": round(t["torch"], 4),
                        "xs_tflops": round(w.flops / t["xs"] / 1e9, 1),
                        "torch_tflops": round(w.flops / t["torch"] / 1e9, 1),
                        "torch_includes_relayout": w.B > 1,
                        "speedup": round(t["torch"] / t["xs"], 3),
                        "max_abs_diff": float((out.float() - ref.float()).abs().max())})
    print(json.dumps({"metric": "torch_sdpa_comparison", "n_gpus": 1, "torch": torch.__version__,
                      "backend": "flash (scaled_dot_product_attention)", "results": results}),
          flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no cross-GPU step).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    if args.ceilings:
        if args.power:
            print(json.dumps({"metric": "mfma_ceilings_power", "n_gpus": 1, "iters": 2048,
                              "waves_per_simd": 2, "modes": ceiling_power(args.power)}), flush=True)
        else:
            print(json.dumps({"metric": "mfma_ceilings", "n_gpus": 1, "iters": 2048,
                              **ceilings(2048)}), flush=True)
        return
    if args.epilogue_overhead:
        epilogue_overhead(args)
        return
    if args.torch_sdpa:
        torch_sdpa(args)
        return
    if args.burst_gap:
        from sequence_attention_amd import burst_gap
        cases = [(workloads.WORKLOADS[n], workloads.make_inputs(workloads.WORKLOADS[n]))
                 for n in ("image", "video", "long")]
        res = burst_gap.characterise(torch.device("cuda:0"), cases,
                                     log=lambda m: print(m, file=sys.stderr, flush=True))
        print(json.dumps({"metric": "burst_gap_characterisation", "n_gpus": 1, **res}), flush=True)
        return
    import sequence_attention_amd as xs

    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    inp = workloads.make_inputs(w)
    q, k, v = (inp[n].to(dev) for n in "qkv")
    if args.in_layout == "chunked":
        q, k, v = (xs.chunk(t, w.P) for t in (q, k, v))
    out = torch.empty((w.P, w.B, w.S // w.P, w.H, w.D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    # split-key workspace (fp32 partials), allocated once outside the timed region
    nsplit = xs.split_count(w.B, w.S, w.H, w.D)
    ws_bytes = xs.workspace_size(w.B, w.S, w.H, w.D)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    def step():
        if w.dtype == "fp8":
            xs.fwd_fp8(q, k, v, inp["descales"], w.P, inp["scale"], out=out, stream=stream,
                       workspace=ws, in_layout=args.in_layout)
        else:
            xs.fwd(q, k, v, w.P, inp["scale"], out=out, stream=stream, workspace=ws,
                   in_layout=args.in_layout)

    # The plain signature itself (xs_attn_fwd / xs_attn_fwd_fp8 by name: no
    # workspace, so the schedule never cuts a tile), timed the same way on the same
    # inputs.  It runs before the product path's warm-up and timed steps, so those
    # start on a GPU whose clock has already settled (about 0.6 % on a run with 5
    # warm-up steps); its own result is compared with the product path's below.
    out_ns = torch.empty_like(out)
    sched_ns = xs.xs_attn_schedule(w.B, w.S, w.H, w.D, with_workspace=False, fp8=w.dtype == "fp8")

    def step_ns():
        if w.dtype == "fp8":
            dq, dk, dv = inp["descales"]
            rc = xs.xs_attn_fwd_fp8(q, k, v, dq, dk, dv, out_ns, w.B, w.S, w.H, w.D, w.P,
                                    inp["scale"], stream.cuda_stream)
        else:
            rc = xs.xs_attn_fwd(q, k, v, out_ns, w.B, w.S, w.H, w.D, w.P, inp["scale"],
                                stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(xs.xs_attn_strerror(rc))

    plain_entry = None
    if args.in_layout == "bshd" and not args.cold and not args.no_plain_entry and not args.power:
        for _ in range(min(args.warmup, 3)):
            step_ns()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            step_ns()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_ns = e0.elapsed_time(e1) / args.steps
        plain_entry = {"entry": "xs_attn_fwd_fp8" if w.dtype == "fp8" else "xs_attn_fwd",
                       "workspace_bytes": 0, "schedule": sched_ns, "steps": args.steps,
                       "ms_per_call": round(ms_ns, 4),
                       "value": round(w.flops / (ms_ns * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                       "measured": "before the product path's warm-up"}

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.power:
        print(json.dumps({"metric": "power", "n_gpus": 1, "workload": w.name,
                          "entry": "xs_attn_fwd_ex with a caller workspace",
                          **power_run(step, args.power, w.flops)}), flush=True)
        return
    if args.graph:
        # the library launches kernels only (no memset, no allocation), so one call
        # captures as is; every replay re-reads the current contents of q, k, v
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                if w.dtype == "fp8":
                    xs.fwd_fp8(q, k, v, inp["descales"], w.P, inp["scale"], out=out, workspace=ws,
                               in_layout=args.in_layout)
                else:
                    xs.fwd(q, k, v, w.P, inp["scale"], out=out, workspace=ws,
                           in_layout=args.in_layout)
        torch.cuda.synchronize()
        step = lambda: graph.replay()  # noqa: E731
        for _ in range(3):
            step()
        torch.cuda.synchronize()

    # Timed region: K back-to-back launches on the launch stream, bracketed by two
    # events.  A sample of the launches (every launch with --cold) is also
    # bracketed by its own pair of events, for the kernel's mean launch duration
    # in the roofline: each event between launches adds queue time of its own, so
    # instrumenting every launch would slow the back-to-back steps being timed.
    # at most every fourth call carries events (a short run still gets K/4 samples)
    every = 1 if args.cold else max(4, args.steps // args.samples)
    ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for i in range(0, args.steps, every)}
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    # the shader clock each XCC held over the timed launches: clock samples queued
    # right before and right after them on the same stream
    from sequence_attention_amd import _lib
    Lc = _lib.lib()
    clk_a = torch.zeros(1024 * 4, dtype=torch.int64, device=dev)
    clk_b = torch.zeros_like(clk_a)
    torch.cuda.synchronize()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.cold else None
    wall_khz = clock_sample(Lc, clk_a, stream)
    t_start.record(stream)
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        pair = ev.get(i)
        if pair is not None:
            pair[0].record(stream)
        step()
        if pair is not None:
            pair[1].record(stream)
    t_end.record(stream)
    clock_sample(Lc, clk_b, stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    xcc_ghz = live_clock(clk_a.cpu().numpy(), clk_b.cpu().numpy(), wall_khz)
    launch_ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev.values()])
    ms_per_step = total_ms / args.steps

    flops = w.flops
    kernel_tag = "attn_fwd_bf16" if w.dtype == "bf16" else "attn_fwd_fp8"
    if args.cold:  # the step time would include the flush: use the per-call events
        ms_per_step = float(np.median(launch_ms))
    value = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    achieved = flops / (float(launch_ms.mean()) * 1e-3) / 1e12

    if plain_entry is not None:
        plain_entry["equals_product_path_within"] = float((out_ns.float() - out.float()).abs().max())
    check = None
    if not args.no_check:
        from oracle import oracle
        rows = workloads.sample_rows(w, 32)
        ref = oracle.attention_rows(inp["q"], inp["k"], inp["v"], rows, inp["scale"], inp["descales"])
        idx = torch.as_tensor(rows, device=dev)
        got = xs.unpack(out, w.S)[idx[:, 0], idx[:, 1], idx[:, 2]].double().cpu().numpy()
        check = {"rows": len(rows), "max_abs": float(np.abs(got - ref).max()),
                 "rel_l2": float(np.linalg.norm(got - ref) / np.linalg.norm(ref))}

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0, sigma^2) inputs, shapes of the workload)",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "H_local": w.H, "D": w.D, "P": w.P,
                   "causal": False,
                   "entry": ("xs_attn_fwd_fp8_ex" if w.dtype == "fp8" else "xs_attn_fwd_ex")
                            + (" with a caller workspace" if ws_bytes else " (no workspace)"),
                   "schedule": xs.xs_attn_schedule(w.B, w.S, w.H, w.D, with_workspace=True,
                                                   fp8=w.dtype == "fp8"),
                   "key_splits": nsplit, "workspace_bytes": ws_bytes,
                   "caches": "evicted before every call (--cold)" if args.cold else "warm",
                   "launch": "hip graph replay" if args.graph else "direct",
                   "in_layout": args.in_layout},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "pct_of_bf16_peak": round(100.0 * value / PEAK_TFLOPS["bf16"], 2),
        "launch_ms": {"mean": round(float(launch_ms.mean()), 4), "min": round(float(launch_ms.min()), 4),
                      "median": round(float(np.median(launch_ms)), 4), "sampled_launches": len(launch_ms)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": recorded_traffic(kernel_tag, w.name),
                     "kernel": ("attn_fwd_bf16_kernel" if w.dtype == "bf16" else "attn_fwd_fp8_kernel")
                               + (" + attn_combine_kernel" if nsplit > 1 else ""),
                     "flops_per_launch": flops},
        "clock": run_clock(xcc_ghz, value, achieved, peak, profile_clock(kernel_tag, w.name, achieved, peak)),
        "plain_entry": plain_entry,
        "check": check,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
