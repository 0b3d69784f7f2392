"""The Burst-Gap microbenchmark on the GPU (through the C ABI): it writes
exactly what include/xs_burst_gap.h says into device memory and into
fine-grained host memory, and its timings behave as issue times should."""
import numpy as np
import pytest
import torch

import sequence_attention_amd as xs
from sequence_attention_amd import burst_gap as bg
from sequence_attention_amd._lib import lib

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _expected(producers, nbytes, nburst, ring=1):
    # region r of the ring holds the last burst b with b % ring == r; in it,
    # lane t of producer p wrote {p, t, b, 0x5eed} into every 16-byte slot
    # s*256 + t of the producer's part
    steps = nbytes // 4096
    t = np.arange(256, dtype=np.uint32)
    w = np.zeros((ring, producers, steps, 256, 4), dtype=np.uint32)
    w[..., 0] = np.arange(producers, dtype=np.uint32)[None, :, None, None]
    w[..., 1] = t[None, None, None, :]
    for r in range(ring):
        w[r, ..., 2] = r + ring * ((nburst - 1 - r) // ring)
    w[..., 3] = 0x5EED
    return w.reshape(-1)


def _run(dst_ptr, nbytes_total, producers, nbytes, nburst, gap, dev):
    times = torch.zeros(producers * 4 * (nburst + 3), dtype=torch.int64, device=dev)
    rc = lib().xs_burst_gap(dst_ptr, nbytes_total, producers, nbytes, nburst, gap, times.data_ptr(),
                            torch.cuda.current_stream(dev).cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    return times.cpu().numpy().reshape(producers, 4, nburst + 3)


@pytest.mark.parametrize("producers,nbytes,nburst,ring", [(3, 4096, 1, 1), (17, 12288, 3, 1),
                                                          (64, 65536, 4, 1), (5, 8192, 7, 3),
                                                          (9, 4096, 5, 5)])
def test_writes_the_documented_pattern_to_device_memory(gpu, producers, nbytes, nburst, ring):
    _say(f"burst-gap device P={producers} bytes={nbytes} bursts={nburst} ring={ring}")
    used = ring * producers * nbytes
    dst = torch.full((used + 4096,), 0xAB, dtype=torch.uint8, device=gpu)
    _run(dst.data_ptr(), used + 4095, producers, nbytes, nburst, 1000, gpu)  # +4095: no extra region
    got = dst[:used].cpu().numpy().view(np.uint32)
    assert np.array_equal(got, _expected(producers, nbytes, nburst, ring))
    assert (dst[used:].cpu().numpy() == 0xAB).all()   # nothing past the ring


def test_writes_the_documented_pattern_to_host_memory(gpu):
    producers, nbytes, nburst = 32, 65536, 3
    _say("burst-gap host memory")
    buf = bg.HostBuffer(producers * nbytes * nburst)
    try:
        buf.view()[:] = 0
        _run(buf.ptr, buf.nbytes, producers, nbytes, nburst, 0, gpu)
        assert np.array_equal(buf.view(np.uint32), _expected(producers, nbytes, nburst, nburst))
    finally:
        buf.free()


def test_timings_behave_like_issue_times(gpu):
    _say("burst-gap timings")
    buf = bg.HostBuffer(128 * 262144)
    try:
        busy = bg.measure(buf.ptr, buf.nbytes, 128, 262144, 5, 0, gpu)
        idle = bg.measure(buf.ptr, buf.nbytes, 128, 262144, 5, int(4e-3 * 2.1e9), gpu)
        small = bg.measure(buf.ptr, buf.nbytes, 128, 16384, 5, int(4e-3 * 2.1e9), gpu)
    finally:
        buf.free()
    for r in (busy, idle, small):
        print(f"  {r}", flush=True)
        assert 0.5e9 < r.clock_hz < 3.0e9
        assert r.t_first > 0 and r.t_steady > 0 and r.drain >= 0
    # a gap lets the drain catch up: steady bursts issue no slower than back-to-back ones
    assert idle.t_steady <= busy.t_steady * 1.05
    # a 16x smaller burst issues faster when nothing is outstanding
    assert small.t_steady < idle.t_steady
    # the recorded gap is what was asked for (to the clock-rate estimate)
    assert idle.G == pytest.approx(4e-3 * 2.1e9 / idle.clock_hz, rel=1e-9)


@pytest.mark.parametrize("producers,row_bytes,pitch,nburst,ring,coupled", [
    (3, 256, 1280, 2, 1, 0), (5, 128, 384, 5, 2, 1), (2, 256, 256, 3, 3, 0), (4, 256, 768, 3, 2, 1)])
def test_tile_pattern_writes_the_documented_rows(gpu, producers, row_bytes, pitch, nburst, ring,
                                                 coupled):
    # every row of every tile gets {producer, burst} in each 8-byte word of its
    # row_bytes; the bytes between rows keep their fill
    _say(f"burst-gap tiles P={producers} row={row_bytes} pitch={pitch} bursts={nburst} ring={ring}")
    region = 256 * pitch
    used = ring * producers * region
    dst = torch.full((used + 4096,), 0xAB, dtype=torch.uint8, device=gpu)
    times = torch.zeros(producers * 8 * (2 * nburst + 3), dtype=torch.int64, device=gpu)
    src = torch.ones(1 << 16, dtype=torch.int32, device=gpu) if coupled else None  # 256 KiB
    rc = lib().xs_burst_gap_tiles(dst.data_ptr(), used + region - 1, producers, row_bytes, pitch,
                                  nburst, 1000, coupled, src.data_ptr() if coupled else None,
                                  src.numel() * 4 if coupled else 0, 8, times.data_ptr(),
                                  torch.cuda.current_stream(gpu).cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    assert np.all(got[used:] == 0xAB)
    body = got[:used].reshape(ring, producers, 256, pitch)
    words = body[..., :row_bytes].copy().view(np.uint32).reshape(ring, producers, 256, row_bytes // 8, 2)
    for r in range(ring):
        last = r + ring * ((nburst - 1 - r) // ring)
        assert np.all(words[r, :, :, :, 0] == np.arange(producers, dtype=np.uint32)[:, None, None])
        assert np.all(words[r, :, :, :, 1] == last)
    assert np.all(body[..., row_bytes:] == 0xAB)
    t = times.cpu().numpy().reshape(producers, 8, 2 * nburst + 3)
    assert np.all(t[:, :, :2 * nburst] > 0) and np.all(t[:, :, 2 * nburst + 2] > 0)
