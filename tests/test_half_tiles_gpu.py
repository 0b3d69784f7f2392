"""GPU parity of the half-height tiles: a call whose schedule cuts no tile runs
the tiles left after its whole rounds (at most half a round of them) as 128-row
tiles of the same kernel with 4 wavefronts instead of 8, in a second launch,
one workgroup each (bf16 and fp8).

* shapes whose last round runs as half tiles, on every element of out_packed
  against the fp64 oracle (NaN-prefilled, through xs_attn_fwd by name): a
  ragged sequence whose last tile per head holds fewer than 128 rows (so one
  half tile is missing there and the other is partly masked), the first
  remaining tile in the middle of a head, B = 2 for the relayout; and D = 64;
* the log-sum-exp output and chunk-layout inputs on a half-tile schedule;
* the 4-wave and the 8-wave kernel give bit-identical rows: each row's
  arithmetic (its key order, its fast pass and lazy rescale) does not depend on
  how many waves share the tile, so the same heads computed in whole tiles
  (a shape of exactly one round) and in half tiles must agree bit for bit;
* out_packed in host memory (behind a link) keeps the single-launch schedule of
  full tiles and gives the same bytes, as does that schedule asked for with
  XS_ONE_LAUNCH.

Bar: max-abs 1e-2 / 5e-2 and relative L2 1e-2 / 8e-2 (bf16 / fp8) on every
element; the LSE within the 5e-3 bar derived for the log-sum-exp output.
"""
import numpy as np
import pytest
import torch

import sequence_attention_amd as xs
import workloads
from oracle import oracle

pytestmark = pytest.mark.gpu

TOL = {"bf16": (1e-2, 1e-2), "fp8": (5e-2, 8e-2)}  # max-abs, rel-L2
LSE_BAR = 5e-3


def _say(*a):
    print("[case]", *a, flush=True)


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _gate(got, ref, what, tol=TOL["bf16"]):
    err = np.abs(got - ref)
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"  {what}: max_abs={err.max():.3e} rel_l2={rel:.3e} ({got.size} elements)", flush=True)
    assert np.isfinite(got).all(), f"{what}: non-finite output (unwritten?)"
    assert err.max() <= tol[0] and rel <= tol[1], f"{what}: max_abs={err.max():.3e} rel={rel:.3e}"


def _cus(dev):
    return torch.cuda.get_device_properties(dev).multi_processor_count


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("B,S,H,D,P", [(2, 7000, 5, 128, 8), (1, 4000, 20, 64, 4)])
def test_half_tile_round_every_element(gpu, dtype, B, S, H, D, P):
    w = workloads.custom(B, S, H, D, P, dtype=dtype, index=8300 + D + (dtype == "fp8"))
    s = xs.xs_attn_schedule(B, S, H, D, with_workspace=False, fp8=dtype == "fp8")
    tiles = B * H * -(-S // 256)
    cus = _cus(gpu)
    _say(f"half tiles {dtype} B={B} S={S} H={H} D={D} P={P}: {tiles} tiles on {cus} CUs, "
         f"schedule {s}")
    assert s["half_tiles"] > 0 and s["whole_rounds"] >= 1, "the shape must end in half tiles"
    inp = workloads.make_inputs(w)
    q, k, v = (inp[n].to(gpu) for n in "qkv")
    out = torch.full((P, B, S // P, H, D), float("nan"), dtype=torch.bfloat16, device=gpu)
    stream = torch.cuda.current_stream(gpu).cuda_stream
    if dtype == "fp8":
        dq, dk, dv = inp["descales"]
        rc = xs.xs_attn_fwd_fp8(q, k, v, dq, dk, dv, out, B, S, H, D, P, inp["scale"], stream)
    else:
        rc = xs.xs_attn_fwd(q, k, v, out, B, S, H, D, P, inp["scale"], stream)
    assert rc == 0, xs.xs_attn_strerror(rc)
    torch.cuda.synchronize()
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], P, inp["scale"], inp["descales"])
    _gate(_f64(out), ref, f"{dtype} B={B} S={S} H={H} D={D}", TOL[dtype])


def test_half_tiles_with_lse_and_chunked_inputs(gpu):
    # 2 x 3 heads x 10 tiles = 60 tiles: no whole round, 120 half tiles (the
    # last tile of a head holds 2560 - 2304 = 256 rows: both halves present)
    B, S, H, D, P = 2, 2560, 3, 128, 4
    w = workloads.custom(B, S, H, D, P, index=8350)
    s = xs.xs_attn_schedule(B, S, H, D, with_workspace=False)
    _say(f"half tiles with lse and chunked inputs B={B} S={S} H={H} D={D} P={P}, schedule {s}")
    assert s["half_tiles"] == 2 * B * H * (S // 256) and s["groups"] == 0
    inp = workloads.make_inputs(w)
    q, k, v = (inp[n].to(gpu) for n in "qkv")
    out, lse = xs.fwd(q, k, v, P, inp["scale"], workspace=None, lse=True)
    qc, kc, vc = (xs.chunk(t, P) for t in (q, k, v))
    out_c, lse_c = xs.fwd(qc, kc, vc, P, inp["scale"], workspace=None, lse=True,
                          in_layout="chunked")
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention_packed(inp["q"], inp["k"], inp["v"], P, inp["scale"],
                                           with_lse=True)
    _gate(_f64(out), ref_o, "O (lse requested)")
    d = np.abs(_f64(lse) - ref_l)
    print(f"  lse max_abs={d.max():.3e}", flush=True)
    assert np.isfinite(_f64(lse)).all() and d.max() <= LSE_BAR
    assert torch.equal(out.view(torch.int16), out_c.view(torch.int16)), "chunked inputs differ"
    assert torch.equal(lse, lse_c), "chunked inputs: lse differs"


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("S,D", [(1000, 64), (1000, 128), (4096, 128)])
def test_half_and_whole_tiles_bit_identical(gpu, S, D, dtype):
    # H_full heads make exactly one round of whole tiles on this device (no
    # half tiles); the first few of the same heads alone leave the chip mostly
    # idle and run as half tiles.  Heads are independent, so the rows of those
    # heads must agree bit for bit between the two calls.
    cus = _cus(gpu)
    mt = -(-S // 256)
    if cus % mt:
        pytest.skip(f"{cus} CUs is not a multiple of {mt} tiles per head")
    H_full, P, B = cus // mt, 8, 1
    H_few = max(1, H_full // 8)
    w = workloads.custom(B, S, H_full, D, P, dtype=dtype, index=8400 + D + S + (dtype == "fp8"))
    sf = xs.xs_attn_schedule(B, S, H_full, D, with_workspace=False)
    sh = xs.xs_attn_schedule(B, S, H_few, D, with_workspace=False)
    _say(f"bit identity {dtype} S={S} D={D}: {H_full} heads {sf} against {H_few} heads {sh}")
    assert sf["half_tiles"] == 0 and sf["whole_rounds"] == 1 and sf["groups"] == cus
    assert sh["half_tiles"] > 0 and sh["groups"] == 0
    inp = workloads.make_inputs(w)
    q, k, v = (inp[n].to(gpu) for n in "qkv")
    few_in = [t[:, :, :H_few].contiguous() for t in (q, k, v)]
    if dtype == "fp8":
        # the call without the log-sum-exp (the fp8 share's) and the one with it
        # run different kernel instantiations; check both
        full = xs.fwd_fp8(q, k, v, inp["descales"], P, inp["scale"], workspace=None)
        few = xs.fwd_fp8(*few_in, inp["descales"], P, inp["scale"], workspace=None)
        torch.cuda.synchronize()
        assert torch.equal(xs.unpack(full, S)[:, :, :H_few].contiguous().view(torch.int16),
                           xs.unpack(few, S).contiguous().view(torch.int16))
        full, lse_full = xs.fwd_fp8(q, k, v, inp["descales"], P, inp["scale"], workspace=None,
                                    lse=True)
        few, lse_few = xs.fwd_fp8(*few_in, inp["descales"], P, inp["scale"], workspace=None,
                                  lse=True)
    else:
        full, lse_full = xs.fwd(q, k, v, P, inp["scale"], workspace=None, lse=True)
        few, lse_few = xs.fwd(*few_in, P, inp["scale"], workspace=None, lse=True)
    torch.cuda.synchronize()
    a = xs.unpack(full, S)[:, :, :H_few]
    b = xs.unpack(few, S)
    assert torch.isfinite(b.float()).all()
    assert torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))
    assert torch.equal(lse_full[:, :H_few], lse_few)


def test_output_behind_a_link_keeps_full_tiles(gpu):
    # out_packed in fine-grained host memory (the stand-in for a remote
    # destination): the call keeps the single-launch schedule of full tiles,
    # whose rows are bit-identical to the half-tile schedule's in device memory
    from sequence_attention_amd.burst_gap import HostBuffer

    w = workloads.WORKLOADS["image"].with_(index=8500)
    s = xs.xs_attn_schedule(w.B, w.S, w.H, w.D, with_workspace=False)
    _say(f"host-memory output, image share, device-output schedule {s}")
    assert s["half_tiles"] > 0
    inp = workloads.make_inputs(w)
    q, k, v = (inp[n].to(gpu) for n in "qkv")
    out = torch.full((w.P, w.B, w.S // w.P, w.H, w.D), float("nan"), dtype=torch.bfloat16,
                     device=gpu)
    stream = torch.cuda.current_stream(gpu).cuda_stream
    host = HostBuffer(out.numel() * 2)
    try:
        host.view(np.uint8)[:] = 0xFF  # NaN in bf16: an unwritten row cannot pass
        for ptr in (out.data_ptr(), host.ptr):
            rc = xs.xs_attn_fwd(q, k, v, ptr, w.B, w.S, w.H, w.D, w.P, inp["scale"], stream)
            assert rc == 0, xs.xs_attn_strerror(rc)
        torch.cuda.synchronize()
        got = host.view(np.uint16).copy()
    finally:
        host.free()
    assert np.array_equal(got, out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1))
    # the same one-launch schedule asked for explicitly, output in device memory
    one = torch.full_like(out, float("nan"))
    rc = xs.xs_attn_fwd_ex(q, k, v, xs.LAYOUT_BSHD | xs.ONE_LAUNCH, one, None, w.B, w.S, w.H, w.D,
                           w.P, inp["scale"], None, 0, stream)
    assert rc == 0, xs.xs_attn_strerror(rc)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), out.view(torch.int16))
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], w.P, inp["scale"])
    _gate(_f64(out), ref, "device-memory output (half tiles)")
