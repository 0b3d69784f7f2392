"""The C-ABI library without a GPU: it loads, exports every function the header
declares, and rejects bad arguments before any HIP call."""
import ctypes
import math
import subprocess

import numpy as np
import pytest

import sequence_attention_amd as xs
from sequence_attention_amd import _lib

XS_OK, XS_ERR_NULL, XS_ERR_SHAPE, XS_ERR_UNSUPPORTED, XS_ERR_ALIGN, XS_ERR_LAUNCH, XS_ERR_OVERLAP = (
    0, -1, -2, -3, -4, -5, -6)
XS_ERR_WORKSPACE = -7
XS_ERR_SCRATCH = -8

# distinct, 16-byte aligned, far-apart fake device addresses (never dereferenced)
Q, K, V, O = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def test_library_exports_every_declared_function():
    names = _lib.declared_functions()
    assert set(names) == {"xs_attn_fwd", "xs_attn_fwd_fp8", "xs_attn_fwd_ws", "xs_attn_fwd_fp8_ws",
                          "xs_attn_fwd_ex", "xs_attn_fwd_fp8_ex", "xs_attn_workspace_size",
                          "xs_attn_split_count", "xs_attn_strerror", "xs_attn_version",
                          "xs_attn_fwd_noalloc", "xs_attn_schedule", "xs_attn_schedule_ex", "xs_burst_gap",
                          "xs_burst_gap_tiles", "xs_mfma_ceiling", "xs_clock_sample"}
    L = _lib.lib()
    for n in names:
        assert getattr(L, n) is not None
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_version_and_strerror():
    assert xs.xs_attn_version() == 10500
    for code in (XS_OK, XS_ERR_NULL, XS_ERR_SHAPE, XS_ERR_UNSUPPORTED, XS_ERR_ALIGN, XS_ERR_LAUNCH,
                 XS_ERR_OVERLAP, XS_ERR_WORKSPACE, XS_ERR_SCRATCH, 12345):
        s = xs.xs_attn_strerror(code)
        assert isinstance(s, str) and s
    assert xs.xs_attn_strerror(12345) == "unknown status code"


def _fwd(**kw):
    a = dict(q=Q, k=K, v=V, out=O, B=1, S=256, H=2, D=64, P=2, scale=0.125)
    a.update(kw)
    return xs.xs_attn_fwd(a["q"], a["k"], a["v"], a["out"], a["B"], a["S"], a["H"], a["D"], a["P"],
                          a["scale"], None)


def _fwd8(**kw):
    a = dict(q=Q, k=K, v=V, out=O, B=1, S=256, H=2, D=64, P=2, scale=0.125, dq=0.01, dk=0.01,
             dv=0.01)
    a.update(kw)
    return xs.xs_attn_fwd_fp8(a["q"], a["k"], a["v"], a["dq"], a["dk"], a["dv"], a["out"], a["B"],
                              a["S"], a["H"], a["D"], a["P"], a["scale"], None)


@pytest.mark.parametrize("call", [_fwd, _fwd8])
def test_null_pointers(call):
    for name in ("q", "k", "v", "out"):
        assert call(**{name: 0}) == XS_ERR_NULL


@pytest.mark.parametrize("call", [_fwd, _fwd8])
def test_bad_shapes(call):
    for kw in (dict(B=0), dict(S=0), dict(H=0), dict(D=0), dict(P=0), dict(B=-1),
               dict(S=250, P=8), dict(S=7, P=2)):
        assert call(**kw) == XS_ERR_SHAPE, kw


@pytest.mark.parametrize("call", [_fwd, _fwd8])
def test_unsupported(call):
    for kw in (dict(D=32), dict(D=96), dict(D=256), dict(scale=math.inf), dict(scale=math.nan)):
        assert call(**kw) == XS_ERR_UNSUPPORTED, kw


def test_unsupported_fp8_descales():
    for kw in (dict(dq=math.inf), dict(dk=math.nan), dict(dv=-math.inf)):
        assert _fwd8(**kw) == XS_ERR_UNSUPPORTED, kw


@pytest.mark.parametrize("call", [_fwd, _fwd8])
def test_misaligned(call):
    for name, base in (("q", Q), ("k", K), ("v", V), ("out", O)):
        assert call(**{name: base + 8}) == XS_ERR_ALIGN, name


@pytest.mark.parametrize("call", [_fwd, _fwd8])
def test_output_overlapping_an_input(call):
    assert call(out=Q) == XS_ERR_OVERLAP
    assert call(out=K + 4096) == XS_ERR_OVERLAP
    assert call(v=O + 16) == XS_ERR_OVERLAP


def test_python_wrapper_rejects_cpu_tensors():
    import torch
    t = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        xs.fwd(t, t, t, 2)


def test_strerror_returns_static_c_strings():
    L = _lib.lib()
    a = L.xs_attn_strerror(XS_ERR_SHAPE)
    b = L.xs_attn_strerror(XS_ERR_SHAPE)
    assert a == b and isinstance(a, bytes)
    assert isinstance(ctypes.c_char_p(a).value, bytes)


def test_rows_of_one_batch_beyond_4gib_are_unsupported():
    # S * H * D * 2 bytes >= 4 GiB cannot be addressed with 32-bit buffer offsets
    assert _fwd(S=2 ** 24, H=1024, D=128, P=1) == XS_ERR_UNSUPPORTED


def _fwd_ws(ws, nbytes, **kw):
    a = dict(q=Q, k=K, v=V, out=O, B=1, S=4608, H=3, D=128, P=8, scale=0.088)
    a.update(kw)
    return xs.xs_attn_fwd_ws(a["q"], a["k"], a["v"], a["out"], a["B"], a["S"], a["H"], a["D"],
                             a["P"], a["scale"], ws, nbytes, None)


def _owner(u, units, groups):
    return ((u + 1) * groups - 1) // units


def test_schedule_plan_fills_the_grid():
    # 256 compute units (what the plan assumes when no GPU is visible), 256-row
    # tiles, units of two 64-key blocks.  Persistent shares cut a tile only where
    # a share ends inside it.
    assert xs.split_count(1, 32768, 5, 128) == 2    # 640 tiles on 256 shares: 2.5 tiles each
    assert xs.split_count(1, 131072, 3, 128) == 1   # 1536 tiles: 6 whole tiles per share
    assert xs.split_count(2, 32768, 4, 128) == 1    # 1024 tiles: 4 whole tiles per share
    assert xs.split_count(1, 256, 2, 64) == 1       # tiny: one workgroup per tile is cheaper
    assert xs.split_count(0, 4608, 3, 128) == 0
    # image: 54 tiles x 36 units; 216 shares of 9 units (every tile in 4 equal
    # pieces, one piece per share) beat 256 shares of 7-8 units that straddle
    # tiles; the pieces per tile follow from the schedule's own arithmetic
    units, groups, npair = 54 * 36, 216, 36
    most = max(_owner((t + 1) * npair - 1, units, groups) - _owner(t * npair, units, groups) + 1
               for t in range(54))
    assert xs.split_count(1, 4608, 3, 128) == most == 4
    assert xs.workspace_size(1, 4608, 3, 128) == 2 * 216 * 256 * (128 * 4 + 8)
    # workspace: two fp32 slots of 256 rows (O, m, l) per share, only when tiles are cut
    assert xs.workspace_size(1, 32768, 5, 128) == 2 * 256 * 256 * (128 * 4 + 8)
    assert xs.workspace_size(1, 131072, 3, 128) == 0
    assert xs.workspace_size(2, 32768, 4, 128) == 0
    assert xs.workspace_size(1, 4608, 3, 96) == 0


def test_schedule_owner_arithmetic():
    # owner(u) is the share whose range [floor(c U / G), floor((c+1) U / G)) holds u
    for units, groups in ((10, 4), (1944, 256), (163840, 256), (7, 7), (5, 3)):
        starts = [c * units // groups for c in range(groups + 1)]
        for u in range(units):
            c = _owner(u, units, groups)
            assert starts[c] <= u < starts[c + 1]


def test_workspace_errors_before_any_launch():
    need = xs.workspace_size(1, 4608, 3, 128)
    assert need > 0
    W = 0x50000000
    assert _fwd_ws(W + 8, need) == XS_ERR_ALIGN
    assert _fwd_ws(W, need - 16) == XS_ERR_WORKSPACE
    assert _fwd_ws(W, need, D=96) == XS_ERR_UNSUPPORTED
    # the partials may not land in an input or the output
    nbytes = 1 * 4608 * 3 * 128 * 2
    assert _fwd_ws(O + 16, need) == XS_ERR_OVERLAP
    assert _fwd_ws(Q - need + 16, need) == XS_ERR_OVERLAP      # runs into q
    assert _fwd_ws(V + nbytes - 16, need) == XS_ERR_OVERLAP    # starts inside v


def _fwd_ex(**kw):
    a = dict(q=Q, k=K, v=V, layout=0, out=O, lse=None, B=2, S=256, H=2, D=64, P=2, scale=0.125)
    a.update(kw)
    return xs.xs_attn_fwd_ex(a["q"], a["k"], a["v"], a["layout"], a["out"], a["lse"], a["B"],
                             a["S"], a["H"], a["D"], a["P"], a["scale"], None, 0, None)


def _fwd8_ex(**kw):
    a = dict(q=Q, k=K, v=V, layout=0, out=O, lse=None, B=2, S=256, H=2, D=64, P=2, scale=0.125)
    a.update(kw)
    return xs.xs_attn_fwd_fp8_ex(a["q"], a["k"], a["v"], a["layout"], 0.01, 0.01, 0.01, a["out"],
                                 a["lse"], a["B"], a["S"], a["H"], a["D"], a["P"], a["scale"], None,
                                 0, None)


@pytest.mark.parametrize("call", [_fwd_ex, _fwd8_ex])
def test_ex_rejects_unknown_layouts(call):
    for layout in (-1, 2, 7, 0x102, 0x200, 0x300):
        assert call(layout=layout) == XS_ERR_UNSUPPORTED


def test_one_launch_flag_is_accepted_with_either_layout():
    # the flag is stripped before the layout is checked: a call that then fails on
    # its misaligned workspace (checked after the layout) reports XS_ERR_ALIGN
    need = xs.workspace_size(1, 4608, 3, 128)
    W = 0x50000000 + 8
    for layout in (0, 1, xs.ONE_LAUNCH, xs.ONE_LAUNCH | xs.LAYOUT_CHUNKED):
        assert xs.xs_attn_fwd_ex(Q, K, V, layout, O, None, 1, 4608, 3, 128, 8, 0.125, W, need,
                                 None) == XS_ERR_ALIGN, layout
        assert xs.xs_attn_fwd_fp8_ex(Q, K, V, layout, 0.01, 0.01, 0.01, O, None, 1, 4608, 3, 128,
                                     8, 0.125, W, need, None) == XS_ERR_ALIGN, layout
    assert xs.xs_attn_fwd_ex(Q, K, V, 0x200, O, None, 1, 4608, 3, 128, 8, 0.125, W, need,
                             None) == XS_ERR_UNSUPPORTED


@pytest.mark.parametrize("call", [_fwd_ex, _fwd8_ex])
def test_ex_chunked_inputs_need_whole_key_blocks_per_chunk(call):
    # B > 1 and P > 1: S/P must be a multiple of 64
    W = 0x50000000
    assert call(layout=1, S=192, P=2) == XS_ERR_UNSUPPORTED          # T = 96
    # T = 576 = 9 * 64 is allowed (a misaligned lse shows the layout check passed)
    assert call(layout=1, S=4608, P=8, B=3, lse=W + 2) == XS_ERR_ALIGN
    # with B = 1 or P = 1 the chunk layout is the plain layout: no restriction
    assert call(layout=1, S=192, P=2, B=1, lse=W + 2) == XS_ERR_ALIGN    # got past the layout check
    assert call(layout=1, S=192, P=1, B=2, lse=W + 2) == XS_ERR_ALIGN


@pytest.mark.parametrize("call", [_fwd_ex, _fwd8_ex])
def test_ex_lse_alignment_and_overlap(call):
    W = 0x50000000
    assert call(lse=W + 2) == XS_ERR_ALIGN
    assert call(lse=Q) == XS_ERR_OVERLAP
    assert call(lse=O + 64) == XS_ERR_OVERLAP
    assert call(lse=V - 4) == XS_ERR_OVERLAP        # the lse range runs into v


def test_ex_validates_the_base_arguments_first():
    assert _fwd_ex(q=0) == XS_ERR_NULL
    assert _fwd_ex(D=96) == XS_ERR_UNSUPPORTED
    assert _fwd_ex(out=Q) == XS_ERR_OVERLAP


def test_burst_gap_validates_before_any_launch():
    L = _lib.lib()
    D, T = 0x60000000, 0x70000000
    assert L.xs_burst_gap(0, 1 << 20, 4, 4096, 2, 0, T, None) == -1
    assert L.xs_burst_gap(D, 1 << 20, 4, 4096, 2, 0, 0, None) == -1
    for producers, nbytes, nburst, gap in ((0, 4096, 2, 0), (4097, 4096, 2, 0), (4, 4000, 2, 0),
                                           (4, 0, 2, 0), (4, 4096, 0, 0), (4, 4096, 2, -1),
                                           (4, 4096, 2, 1 << 33), (4, 4096, 4096, 1 << 32),
                                           (1024, 4096, 2, 0)):           # last: dst too small
        assert L.xs_burst_gap(D, 1 << 20, producers, nbytes, nburst, gap, T, None) == -2
    assert L.xs_burst_gap(D + 8, 1 << 20, 4, 4096, 2, 0, T, None) == -4
    assert L.xs_burst_gap(D, 1 << 20, 4, 4096, 2, 0, T + 4, None) == -4


def test_burst_gap_tiles_validates_before_any_launch():
    L = _lib.lib()
    D, T = 0x60000000, 0x70000000
    f = L.xs_burst_gap_tiles
    assert f(0, 1 << 24, 4, 256, 1280, 2, 0, 0, None, 0, 0, T, None) == -1
    assert f(D, 1 << 24, 4, 256, 1280, 2, 0, 0, None, 0, 0, 0, None) == -1
    for producers, row_bytes, pitch, nburst, gap in (
            (0, 256, 1280, 2, 0), (4097, 256, 1280, 2, 0), (4, 8, 1280, 2, 0),
            (4, 250, 1280, 2, 0), (4, 8192, 8192, 2, 0), (4, 256, 128, 2, 0),
            (4, 256, 1288, 2, 0), (4, 256, 1280, 0, 0), (4, 256, 1280, 2, -1),
            (4, 256, 1280, 4096, 1 << 32), (64, 256, 1280, 2, 0)):   # last: dst too small
        assert f(D, 1 << 24, producers, row_bytes, pitch, nburst, gap, 0, None, 0, 0, T, None) == -2
    assert f(D + 8, 1 << 24, 4, 256, 1280, 2, 0, 0, None, 0, 0, T, None) == -4
    assert f(D, 1 << 24, 4, 256, 1280, 2, 0, 0, None, 0, 0, T + 4, None) == -4
    S = 0x50000000
    for src_bytes, loads in ((1 << 20, 0), (1 << 20, 65537), (3000, 4), ((1 << 20) + 16, 4)):
        assert f(D, 1 << 24, 4, 256, 1280, 2, 0, 0, S, src_bytes, loads, T, None) == -2
    assert f(D, 1 << 24, 4, 256, 1280, 2, 0, 0, S + 8, 1 << 20, 4, T, None) == -4


def test_mfma_ceiling_validates_before_any_launch():
    L = _lib.lib()
    S, n = 0x60000000, 1024 * 512 * 4
    assert L.xs_mfma_ceiling(0, 2, 16, None, n, None) == -1
    for mode, waves, iters in ((-1, 2, 16), (13, 2, 16), (0, 0, 16), (0, 3, 16), (0, 2, 0),
                               (0, 2, (1 << 20) + 1)):
        assert L.xs_mfma_ceiling(mode, waves, iters, S, n, None) == -2
    assert L.xs_mfma_ceiling(0, 2, 16, S, n - 4, None) == -3
    assert L.xs_mfma_ceiling(0, 2, 16, S + 2, n, None) == -4


def test_clock_sample_validates_before_any_launch():
    L = _lib.lib()
    S, n = 0x60000000, 1024 * 4 * 8
    khz = ctypes.c_int(0)
    assert L.xs_clock_sample(None, n, ctypes.byref(khz), None) == -1
    assert L.xs_clock_sample(S, n, None, None) == -1
    assert L.xs_clock_sample(S, n - 8, ctypes.byref(khz), None) == -3
    assert L.xs_clock_sample(S + 4, n, ctypes.byref(khz), None) == -4


def test_noalloc_entry_validates_before_any_hip_call():
    L = _lib.lib()
    f = L.xs_attn_fwd_noalloc
    assert f(None, K, V, O, 1, 64, 1, 64, 1, 0.125, None) == XS_ERR_NULL
    assert f(Q, K, V, O, 1, 64, 1, 64, 3, 0.125, None) == XS_ERR_SHAPE
    assert f(Q, K, V, O, 1, 64, 1, 96, 1, 0.125, None) == XS_ERR_UNSUPPORTED
    assert f(Q, K, V, O, 1, 64, 1, 64, 1, math.inf, None) == XS_ERR_UNSUPPORTED
    assert f(Q + 8, K, V, O, 1, 64, 1, 64, 1, 0.125, None) == XS_ERR_ALIGN
    assert f(Q, K, V, Q, 1, 64, 1, 64, 1, 0.125, None) == XS_ERR_OVERLAP
    assert "static scratch" in xs.xs_attn_strerror(XS_ERR_SCRATCH)


def test_noalloc_scratch_covers_every_schedule_of_a_256_cu_device():
    # the largest cut schedule: one workgroup per compute unit, two 256-row
    # slots of fp32 O (D = 128) plus max and sum per row
    text = open(_lib.HEADER_PATH).read()
    size = int(text.split("#define XS_NOALLOC_SCRATCH_BYTES")[1].split()[0])
    assert size == 2 * 256 * 256 * (4 * 128 + 8) == 65 * 2 ** 20


def test_schedule_query_is_consistent_with_split_count():
    for shape in [(1, 4608, 3, 128), (1, 32768, 5, 128), (2, 1000, 3, 64), (1, 131072, 3, 128)]:
        s = xs.xs_attn_schedule(*shape)
        assert s["pieces"] == xs.split_count(*shape)
        assert xs.xs_attn_schedule(*shape, with_workspace=False)["pieces"] == 1
        assert s["groups"] >= 1 or s["half_tiles"] >= 1
        assert s["whole_rounds"] >= 0
    with pytest.raises(xs.XsAttnError):
        xs.xs_attn_schedule(1, 64, 1, 96)


def test_half_tiles_fill_the_last_round():
    # without a device the plan assumes 256 compute units
    tiles = lambda B, S, H: B * H * -(-S // 256)
    # video share without a workspace: 640 tiles = 2 whole rounds + 128 tiles,
    # which run as 256 half tiles; with a workspace they are cut by keys instead
    s = xs.xs_attn_schedule(1, 32768, 5, 128, with_workspace=False)
    assert (s["groups"], s["whole_rounds"], s["pieces"], s["half_tiles"]) == (256, 2, 1, 256)
    s = xs.xs_attn_schedule(1, 32768, 5, 128, with_workspace=True)
    assert (s["groups"], s["whole_rounds"], s["pieces"], s["half_tiles"]) == (256, 2, 2, 0)
    # fp8 calls are scheduled alike
    s8 = xs.xs_attn_schedule(1, 32768, 5, 128, with_workspace=False, fp8=True)
    assert s8 == xs.xs_attn_schedule(1, 32768, 5, 128, with_workspace=False)
    assert tiles(1, 32768, 5) == 640
    # image share without a workspace: 54 tiles, no whole round, 108 half tiles
    s = xs.xs_attn_schedule(1, 4608, 3, 128, with_workspace=False)
    assert (s["groups"], s["whole_rounds"], s["half_tiles"]) == (0, 0, 108)
    # a head whose last tile holds at most 128 rows has one half tile fewer:
    # S = 7000 -> 28 tiles, 55 half tiles per head; 280 tiles = 1 round + 24
    # tiles, the first of them tile 4 of head 9 (of 10)
    s = xs.xs_attn_schedule(2, 7000, 5, 128, with_workspace=False)
    assert (s["groups"], s["whole_rounds"], s["half_tiles"]) == (256, 1, 55 - 8)
    # long share: 6 exact rounds, nothing left over
    s = xs.xs_attn_schedule(1, 131072, 3, 128, with_workspace=False)
    assert (s["groups"], s["whole_rounds"], s["half_tiles"]) == (256, 6, 0)
    # more than half a round left over: twice as many half tiles would not fit
    # one round, so the plan keeps full tiles (200 tiles, one round)
    s = xs.xs_attn_schedule(1, 200 * 256, 1, 128, with_workspace=False)
    assert s["half_tiles"] == 0 and s["groups"] == 200


def test_half_tiles_cover_exactly_the_tiles_after_the_whole_rounds():
    # without a device the plan assumes 256 compute units; rows of the tiles
    # [whole_rounds * 256, tiles) must be exactly the rows of the half tiles, a
    # tile of more than 128 rows giving two and one of at most 128 rows one
    rng = np.random.default_rng(7)
    seen = 0
    for _ in range(400):
        B, H = int(rng.integers(1, 5)), int(rng.integers(1, 41))
        S = int(rng.integers(1, 20000))
        D = int(rng.choice([64, 128]))
        s = xs.xs_attn_schedule(B, S, H, D, with_workspace=False)
        mt = -(-S // 256)
        tiles = B * H * mt
        if s["half_tiles"] == 0:
            continue
        seen += 1
        t0 = s["whole_rounds"] * 256
        assert s["groups"] == (256 if s["whole_rounds"] else 0)
        assert 0 < tiles - t0 <= 128 and t0 <= tiles
        rows = lambda m: min(256, S - 256 * m)  # noqa: E731
        expect = sum(2 if rows(t % mt) > 128 else 1 for t in range(t0, tiles))
        assert s["half_tiles"] == expect <= 256, (B, S, H, D, s)
    assert seen > 50
