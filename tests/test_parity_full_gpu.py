"""GPU parity at the full sizes of the workloads, and of the two plain entry points
(no workspace argument) called by name, against the fp64 CPU oracle.

* video and fp8 shares: every element of out_packed, both through the product
  path (the split schedule with a caller workspace, what the benchmark times)
  and through xs_attn_fwd / xs_attn_fwd_fp8 themselves (no workspace: the uncut
  schedule; for bf16 video two rounds of whole tiles, then the remaining 128
  tiles as 256 half-height tiles), each output prefilled with NaN so an
  unwritten element cannot pass;
* long share: NaN prefill, every element finite, and three rows of every
  256-row query tile (its first, its last and one drawn at random) against the
  oracle -- every tile of the schedule is checked, not only a sample of rows;
* a share whose plan runs a round of whole tiles on every compute unit and then
  cuts the remainder tiles between workgroups (the path of the three large
  shares), on every element;
* xs_attn_fwd and xs_attn_fwd_fp8 called by name through ctypes on the image
  share, where the default plan would cut tiles, on every element (bf16: all
  of it in half-height tiles).

Bar: max-abs 1e-2 (bf16 inputs) / 5e-2 (fp8) and relative L2 1e-2 / 8e-2 on every
compared element, the stated tolerance on the workloads' own inputs.
"""
import numpy as np
import pytest
import torch

import sequence_attention_amd as xs
import workloads
from oracle import oracle

pytestmark = pytest.mark.gpu

TOL = {"bf16": (1e-2, 1e-2), "fp8": (5e-2, 8e-2)}  # (max-abs, rel-L2)
TILE = 256  # query rows per tile of the schedule


def _say(*a):
    print("[case]", *a, flush=True)


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _gate(got, ref, dtype, what):
    err = np.abs(got - ref)
    max_abs = float(err.max())
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} ({got.size} elements)", flush=True)
    ta, tr = TOL[dtype]
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert max_abs <= ta and rel <= tr, f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}"


def _nan_out(w, dev):
    return torch.full((w.P, w.B, w.S // w.P, w.H, w.D), float("nan"), dtype=torch.bfloat16,
                      device=dev)


def _product_path(w, inp, q, k, v, dev):
    """The call the benchmark times: fwd / fwd_fp8 with a caller-owned workspace."""
    out = _nan_out(w, dev)
    nbytes = xs.workspace_size(w.B, w.S, w.H, w.D)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
    if w.dtype == "fp8":
        xs.fwd_fp8(q, k, v, inp["descales"], w.P, inp["scale"], out=out, workspace=ws)
    else:
        xs.fwd(q, k, v, w.P, inp["scale"], out=out, workspace=ws)
    return out


def _by_name(w, inp, q, k, v, dev):
    """xs_attn_fwd / xs_attn_fwd_fp8 through ctypes, on the current stream."""
    out = _nan_out(w, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    if w.dtype == "fp8":
        dq, dk, dv = inp["descales"]
        rc = xs.xs_attn_fwd_fp8(q, k, v, dq, dk, dv, out, w.B, w.S, w.H, w.D, w.P, inp["scale"],
                                stream)
    else:
        rc = xs.xs_attn_fwd(q, k, v, out, w.B, w.S, w.H, w.D, w.P, inp["scale"], stream)
    assert rc == 0, xs.xs_attn_strerror(rc)
    return out


@pytest.mark.parametrize("name", ["video", "fp8"])
def test_full_size_every_element(gpu, name):
    w = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(w)
    q, k, v = (inp[n].to(gpu) for n in "qkv")
    _say(f"{name} full size, B={w.B} S={w.S} H={w.H} D={w.D} P={w.P}, "
         f"pieces per tile <= {xs.split_count(w.B, w.S, w.H, w.D)}")
    outs = {"product path (workspace)": _product_path(w, inp, q, k, v, gpu),
            "by name, no workspace": _by_name(w, inp, q, k, v, gpu)}
    torch.cuda.synchronize()
    outs = {key: _f64(o) for key, o in outs.items()}
    _say(f"{name}: oracle on all {w.B * w.S * w.H} rows")
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], w.P, inp["scale"], inp["descales"])
    for key, got in outs.items():
        _gate(got, ref, w.dtype, f"{name} {key}")


def test_long_every_tile(gpu):
    w = workloads.WORKLOADS["long"]
    inp = workloads.make_inputs(w)
    q, k, v = (inp[n].to(gpu) for n in "qkv")
    _say(f"long full size, B={w.B} S={w.S} H={w.H} D={w.D} P={w.P}")
    outs = {"product path (workspace)": _product_path(w, inp, q, k, v, gpu),
            "by name, no workspace": _by_name(w, inp, q, k, v, gpu)}
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    rows = []
    for b in range(w.B):
        for h in range(w.H):
            for m0 in range(0, w.S, TILE):
                last = min(m0 + TILE, w.S) - 1
                for s in (m0, last, int(rng.integers(m0, last + 1))):
                    rows.append((b, s, h))
    rows = np.asarray(rows, dtype=np.int64)
    _say(f"long: oracle on {len(rows)} rows (3 per 256-row tile)")
    ref = oracle.attention_rows(inp["q"], inp["k"], inp["v"], rows, inp["scale"])
    idx = torch.as_tensor(rows, device=gpu)
    for key, out in outs.items():
        assert torch.isfinite(out.float()).all(), f"{key}: an element is not finite (unwritten?)"
        got = _f64(xs.unpack(out, w.S)[idx[:, 0], idx[:, 1], idx[:, 2]])
        _gate(got, ref, "bf16", f"long {key}, 3 rows of every tile")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_whole_tile_round_then_cut_remainder_every_element(gpu, dtype):
    # 1 x 10 heads x 32 tiles = 320 tiles on a 256-CU GPU: one round of whole
    # tiles on every compute unit, then the 64 remaining tiles' key ranges shared
    # by all workgroups (cut tiles, merged), as on the video share.
    B, S, H, D, P = 1, 8192, 10, 128, 8
    w = workloads.custom(B, S, H, D, P, dtype=dtype, index=8100 + (dtype == "fp8"))
    tiles = B * H * ((S + TILE - 1) // TILE)
    cus = torch.cuda.get_device_properties(gpu).multi_processor_count
    assert tiles > cus, "the shape must give every compute unit at least one whole tile"
    assert xs.split_count(B, S, H, D) > 1, "the remainder tiles must be cut"
    inp = workloads.make_inputs(w)
    q, k, v = (inp[n].to(gpu) for n in "qkv")
    _say(f"whole-tile round + cut remainder {dtype} B={B} S={S} H={H} D={D} P={P}")
    outs = {"product path (workspace)": _product_path(w, inp, q, k, v, gpu),
            "by name, no workspace": _by_name(w, inp, q, k, v, gpu)}
    torch.cuda.synchronize()
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], P, inp["scale"], inp["descales"])
    for key, out in outs.items():
        _gate(_f64(out), ref, dtype, f"{dtype} {key}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_plain_entry_points_by_name(gpu, dtype):
    # The image share: 54 tiles on 256 CUs, where the default (workspace) plan
    # cuts every tile; the plain signatures take no workspace and run the
    # uncut schedule.
    w = workloads.WORKLOADS["image"].with_(dtype=dtype, index=8200 + (dtype == "fp8"))
    assert xs.split_count(w.B, w.S, w.H, w.D) > 1
    inp = workloads.make_inputs(w)
    q, k, v = (inp[n].to(gpu) for n in "qkv")
    _say(f"by name {dtype} B={w.B} S={w.S} H={w.H} D={w.D} P={w.P}")
    out = _by_name(w, inp, q, k, v, gpu)
    torch.cuda.synchronize()
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], w.P, inp["scale"], inp["descales"])
    _gate(_f64(out), ref, dtype, f"xs_attn_fwd{'_fp8' if dtype == 'fp8' else ''}")
