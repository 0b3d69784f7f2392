"""GPU parity of the two optional parts of the extended entry points
(xs_attn_fwd_ex / xs_attn_fwd_fp8_ex, through the C ABI):

* the row log-sum-exp output lse[B][H][S] against the oracle's fp64 value, and
* inputs in the pre-attention All-to-All chunk layout [P][B][S/P][H][D], which
  must give bit for bit the output of the same inputs in [B][S][H][D] (only the
  load addresses differ; tile shapes and reduction order do not), and match the
  oracle run on the chunk layout directly.

Bar for lse, derived from the arithmetic: the kernel's lse is m + log2(l) with l
the fp32 sum of the probabilities before their rounding to bf16 / e4m3.  The
fp32 scores carry at most D * 2^-24 * scale * sum_d |q_d k_d| (<= 1e-4 for these
inputs); the fp32 sums add at most n * 2^-24 relative for n <= 16384 terms per
lane (1e-3); exp2/log2 approximations add < 1e-6.  fp8's matrix core sums the
e4m3 products less precisely than fp32 (up to about 2^-12.8 of
scale * sum_d |q_d k_d|, pinned by test_score_accumulation_precision): for these
N(0, 1) inputs that sum is about 7, adding at most 1e-3.  Total < 2.2e-3; the
bar is 5e-3 (it also covers the bf16 rounding of every probability, 2^-8, which
an implementation summing the rounded values would add).
"""
import numpy as np
import pytest
import torch

import sequence_attention_amd as xs
import workloads
from oracle import oracle

pytestmark = pytest.mark.gpu

LSE_BAR = 5e-3
TOL = {"bf16": (1e-2, 1e-2), "fp8": (5e-2, 8e-2)}


def _say(*a):
    print("[case]", *a, flush=True)


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _call(inp, dev, P, *, lse=True, layout="bshd", workspace="auto", tensors=None):
    w = inp["workload"]
    q, k, v = tensors if tensors is not None else [inp[n].to(dev) for n in "qkv"]
    if w.dtype == "fp8":
        r = xs.fwd_fp8(q, k, v, inp["descales"], P, inp["scale"], workspace=workspace, lse=lse,
                       in_layout=layout)
    else:
        r = xs.fwd(q, k, v, P, inp["scale"], workspace=workspace, lse=lse, in_layout=layout)
    torch.cuda.synchronize()
    return r


def _gate(got, ref, dtype, what):
    err = np.abs(got - ref)
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"  {what} max_abs={err.max():.3e} rel_l2={rel:.3e}", flush=True)
    ta, tr = TOL[dtype]
    assert err.max() <= ta and rel <= tr and np.isfinite(got).all(), what


# ------------------------------------------------------------------ log-sum-exp
LSE_SHAPES = [
    # (B, S, H, D, P)
    (1, 16, 1, 64, 2), (2, 192, 3, 128, 4), (1, 200, 2, 128, 8), (3, 130, 2, 64, 2),
    (1, 1, 2, 128, 1), (2, 576, 1, 64, 3), (1, 4608, 3, 128, 8),
]


@pytest.mark.parametrize("split", ["auto", None])
@pytest.mark.parametrize("B,S,H,D,P", LSE_SHAPES)
def test_lse_every_row(gpu, B, S, H, D, P, split):
    w = workloads.custom(B, S, H, D, P, index=3000 + S + D + B)
    inp = workloads.make_inputs(w)
    _say(f"lse B={B} S={S} H={H} D={D} P={P} split={split} nsplit={xs.split_count(B, S, H, D)}")
    ref_o, ref_l = oracle.attention_packed(inp["q"], inp["k"], inp["v"], P, inp["scale"],
                                           with_lse=True)
    out, lse = _call(inp, gpu, P, workspace=split)
    assert tuple(lse.shape) == (B, H, S)
    d = np.abs(_f64(lse) - ref_l)
    print(f"  lse max_abs={d.max():.3e}", flush=True)
    assert d.max() <= LSE_BAR
    _gate(_f64(out), ref_o, "bf16", "O with lse requested")


@pytest.mark.parametrize("split", ["auto", None])
def test_lse_fp8(gpu, split):
    w = workloads.custom(2, 640, 3, 128, 8, dtype="fp8", index=3100)
    inp = workloads.make_inputs(w)
    _say(f"lse fp8 B=2 S=640 H=3 split={split}")
    ref_o, ref_l = oracle.attention_packed(inp["q"], inp["k"], inp["v"], w.P, inp["scale"],
                                           inp["descales"], with_lse=True)
    out, lse = _call(inp, gpu, w.P, workspace=split)
    d = np.abs(_f64(lse) - ref_l)
    print(f"  lse max_abs={d.max():.3e}", flush=True)
    assert d.max() <= LSE_BAR
    _gate(_f64(out), ref_o, "fp8", "fp8 O with lse requested")


@pytest.mark.parametrize("name,nrows", [("video", 64), ("fp8", 64)])
def test_lse_full_size_sampled_rows(gpu, name, nrows):
    w = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(w)
    _say(f"lse {name} sampled {nrows} rows")
    out, lse = _call(inp, gpu, w.P)
    rows = workloads.sample_rows(w, nrows)
    ref_o, ref_l = oracle.attention_rows(inp["q"], inp["k"], inp["v"], rows, inp["scale"],
                                         inp["descales"], with_lse=True)
    idx = torch.as_tensor(rows, device=gpu)
    got_l = _f64(lse[idx[:, 0], idx[:, 2], idx[:, 1]])
    d = np.abs(got_l - ref_l)
    print(f"  lse max_abs={d.max():.3e}", flush=True)
    assert d.max() <= LSE_BAR
    o = xs.unpack(out, w.S)
    _gate(_f64(o[idx[:, 0], idx[:, 1], idx[:, 2]]), ref_o, w.dtype, f"{name} O")


def test_lse_does_not_change_the_output(gpu):
    w = workloads.custom(2, 256, 2, 128, 4, index=3200)
    inp = workloads.make_inputs(w)
    _say("lse on/off bit-exact")
    a = _call(inp, gpu, w.P, lse=None)
    b, _ = _call(inp, gpu, w.P, lse=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_lse_closed_forms(gpu):
    # K = 0: every score is 0, lse = ln S; S = 1: lse = the single score
    w = workloads.custom(1, 256, 2, 64, 2, index=3300)
    inp = workloads.make_inputs(w)
    q, v = inp["q"].to(gpu), inp["v"].to(gpu)
    k = torch.zeros_like(q)
    _say("lse K=0")
    _, lse = xs.fwd(q, k, v, 2, inp["scale"], lse=True)
    torch.cuda.synchronize()
    np.testing.assert_allclose(_f64(lse), np.log(256.0), rtol=0, atol=1e-5)
    w1 = workloads.custom(2, 1, 3, 128, 1, index=3301)
    inp1 = workloads.make_inputs(w1)
    _say("lse S=1")
    _, lse1 = xs.fwd(*[inp1[n].to(gpu) for n in "qkv"], 1, 0.7, lse=True)
    torch.cuda.synchronize()
    s = 0.7 * (inp1["q"].double() * inp1["k"].double()).sum(-1)      # [B][1][H]
    np.testing.assert_allclose(_f64(lse1), s.permute(0, 2, 1).numpy(), rtol=0, atol=2e-5)


def test_score_accumulation_precision(gpu):
    # With one key the row log-sum-exp is the score itself, so lse - scale * q.k
    # (exact, fp64) is the error of the score MFMAs' dot product.  Pinned here
    # because the log-sum-exp bars rest on it: the bf16 matrix core sums the
    # exact products as fp32 does (D * 2^-24 of scale * sum_d |q_d k_d| is the
    # fp32 bound; 2^-20 is checked), the e4m3 one much more coarsely (measured up
    # to 2^-12.8; 2^-11 is checked).  One dominant product per dot (|q_0 k_0|
    # about 999 times the rest) is the hard case for the e4m3 sum.
    g = torch.Generator().manual_seed(3)
    for dtype, eps in (("bf16", 2.0 ** -20), ("fp8", 2.0 ** -11)):
        for mag in (1.0, 30.0):
            B, H, D = 64, 8, 128
            qf = torch.randn(B, 1, H, D, generator=g) * mag
            kf = torch.randn(B, 1, H, D, generator=g) * mag
            qf[..., 0] = mag
            kf[..., 0] = 999.0
            _say(f"score accumulation {dtype} magnitude {mag}")
            if dtype == "fp8":
                dq, dk = float(qf.abs().max()) / 448.0, float(kf.abs().max()) / 448.0
                q8, k8 = (qf / dq).to(torch.float8_e4m3fn), (kf / dk).to(torch.float8_e4m3fn)
                qe, ke = q8.to(torch.float64) * dq, k8.to(torch.float64) * dk
                _, lse = xs.fwd_fp8(q8.to(gpu), k8.to(gpu), torch.ones_like(q8).to(gpu),
                                    (dq, dk, 1.0), 1, 0.0883883476, lse=True)
            else:
                q, k = qf.to(torch.bfloat16), kf.to(torch.bfloat16)
                qe, ke = q.to(torch.float64), k.to(torch.float64)
                _, lse = xs.fwd(q.to(gpu), k.to(gpu), torch.ones_like(q).to(gpu), 1, 0.0883883476,
                                lse=True)
            torch.cuda.synchronize()
            exact = ((qe * ke).sum(-1) * 0.0883883476).permute(0, 2, 1).numpy()  # [B][H][1]
            absdot = ((qe * ke).abs().sum(-1) * 0.0883883476).permute(0, 2, 1).numpy()
            rel = float((np.abs(_f64(lse) - exact) / absdot).max())
            print(f"  max error / (scale sum|q k|) = 2^{np.log2(max(rel, 1e-30)):.1f}", flush=True)
            assert rel <= eps


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_lse_and_workspace_stay_in_bounds(gpu, dtype):
    # lse is written on every row and nowhere else; the kernels touch only the
    # workspace_size bytes of a larger workspace
    B, S, H, D, P = 1, 4608, 3, 128, 8          # the image share: a cut schedule
    w = workloads.custom(B, S, H, D, P, dtype=dtype, index=3700)
    inp = workloads.make_inputs(w)
    q, k, v = [inp[n].to(gpu) for n in "qkv"]
    nl, pad = B * H * S, 1024
    lbig = torch.full((nl + 2 * pad,), float("nan"), dtype=torch.float32, device=gpu)
    lbig[:pad] = 5.0
    lbig[pad + nl:] = -9.0
    lse = lbig[pad:pad + nl].view(B, H, S)
    need = xs.workspace_size(B, S, H, D)
    assert need > 0
    wbig = torch.full((need + 2 * 4096,), 0xA5, dtype=torch.uint8, device=gpu)
    ws = wbig[4096:4096 + need]
    _say(f"bounds {dtype}: lse {nl} floats, workspace {need} bytes")
    if dtype == "fp8":
        xs.fwd_fp8(q, k, v, inp["descales"], P, inp["scale"], workspace=ws, lse=lse)
    else:
        xs.fwd(q, k, v, P, inp["scale"], workspace=ws, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(lse).any()
    assert torch.all(lbig[:pad] == 5.0) and torch.all(lbig[pad + nl:] == -9.0)
    assert torch.all(wbig[:4096] == 0xA5) and torch.all(wbig[4096 + need:] == 0xA5)


# ------------------------------------------------------------------ chunk-layout inputs
CHUNKED = [
    # (B, S, H, D, P, dtype): T = S/P a multiple of 64 whenever B > 1 and P > 1
    (2, 256, 2, 128, 2, "bf16"), (3, 512, 1, 64, 4, "bf16"), (2, 4608, 3, 128, 8, "bf16"),
    (2, 1024, 2, 128, 8, "fp8"), (1, 200, 2, 128, 8, "bf16"), (2, 130, 2, 64, 1, "bf16"),
]


@pytest.mark.parametrize("B,S,H,D,P,dtype", CHUNKED)
def test_chunked_inputs_equal_bshd_bit_for_bit(gpu, B, S, H, D, P, dtype):
    w = workloads.custom(B, S, H, D, P, dtype=dtype, index=3400 + S + B + P)
    inp = workloads.make_inputs(w)
    q, k, v = [inp[n].to(gpu) for n in "qkv"]
    for split in ("auto", None):
        _say(f"chunked B={B} S={S} H={H} D={D} P={P} {dtype} split={split}")
        want, want_l = _call(inp, gpu, P, workspace=split, tensors=(q, k, v))
        got, got_l = _call(inp, gpu, P, workspace=split, layout="chunked",
                           tensors=tuple(xs.chunk(t, P) for t in (q, k, v)))
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
        assert torch.equal(got_l, want_l)


@pytest.mark.parametrize("B,S,H,D,P,dtype", [(3, 384, 2, 128, 3, "bf16"), (2, 512, 2, 64, 4, "fp8")])
def test_chunked_inputs_against_the_oracle(gpu, B, S, H, D, P, dtype):
    w = workloads.custom(B, S, H, D, P, dtype=dtype, index=3500 + S)
    inp = workloads.make_inputs(w)
    qc, kc, vc = (xs.chunk(inp[n], P) for n in "qkv")       # CPU copies in the chunk layout
    _say(f"chunked vs oracle B={B} S={S} P={P} {dtype}")
    ref_o, ref_l = oracle.attention_packed(qc, kc, vc, P, inp["scale"], inp["descales"], in_P=P,
                                           with_lse=True)
    out, lse = _call(inp, gpu, P, layout="chunked", tensors=(qc.to(gpu), kc.to(gpu), vc.to(gpu)))
    _gate(_f64(out), ref_o, dtype, "chunked O")
    assert np.abs(_f64(lse) - ref_l).max() <= LSE_BAR


def test_chunked_wrapper_checks_shapes(gpu):
    w = workloads.custom(2, 256, 2, 64, 2, index=3600)
    inp = workloads.make_inputs(w)
    q, k, v = [inp[n].to(gpu) for n in "qkv"]
    with pytest.raises(ValueError):
        xs.fwd(q, k, v, 2, in_layout="chunked")                   # 4-D given
    qc, kc, vc = (xs.chunk(t, 2) for t in (q, k, v))
    with pytest.raises(ValueError):
        xs.fwd(qc, kc, vc, 4, in_layout="chunked")                # leading dim is not P
    with pytest.raises(ValueError):
        xs.fwd(q, k, v, 2, lse=torch.empty(3, device=gpu))        # wrong lse shape
    bad = workloads.custom(2, 192, 1, 64, 2, index=3601)          # T = 96: not whole blocks
    bi = workloads.make_inputs(bad)
    with pytest.raises(xs.XsAttnError):
        xs.fwd(*(xs.chunk(bi[n].to(gpu), 2) for n in "qkv"), 2, in_layout="chunked")
