"""GPU parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Bar: every element of out_packed within max-abs 1e-2 (bf16 inputs) or 5e-2
(fp8 inputs) of the oracle on the same seeded bytes, plus a relative-L2 gate
(1e-2 bf16, 8e-2 fp8) that a zero or badly scaled output cannot pass; the
relayout is bit-exact (P = k equals the pack of P = 1 bit for bit).  Small
shapes and the image share are checked on every element here, the full-size
workloads additionally on sampled rows (which touch every destination slice)
and by properties that hold at any size; tests/test_parity_full_gpu.py checks
the video and fp8 shares on every element and the long share on three rows of
every query tile.
"""
import math

import numpy as np
import pytest
import torch

import sequence_attention_amd as xs
import workloads
from oracle import oracle

pytestmark = pytest.mark.gpu

TOL = {"bf16": (1e-2, 1e-2), "fp8": (5e-2, 8e-2)}  # (max-abs, rel-L2)


def _say(*a):
    print("[case]", *a, flush=True)


def to_gpu(inp, dev):
    return [inp[n].to(dev) for n in "qkv"]


def run(inp, P, dev, scale=None, tensors=None):
    w = inp["workload"]
    q, k, v = tensors if tensors is not None else to_gpu(inp, dev)
    scale = inp["scale"] if scale is None else scale
    _say(w.name, f"B={q.shape[0]} S={q.shape[1]} H={q.shape[2]} D={q.shape[3]} P={P}",
         w.dtype, f"scale={scale}")
    if w.dtype == "fp8":
        out = xs.fwd_fp8(q, k, v, inp["descales"], P, scale)
    else:
        out = xs.fwd(q, k, v, P, scale)
    torch.cuda.synchronize()
    return out


def gate(got, ref, dtype):
    """(max-abs, rel-L2) of got vs ref, and whether both are within the bar."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    ta, tr = TOL[dtype]
    return max_abs, rel, (max_abs <= ta and rel <= tr and np.isfinite(got).all())


def assert_gate(got, ref, dtype, what=""):
    max_abs, rel, ok = gate(got, ref, dtype)
    print(f"  {what} max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    assert ok, f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} exceed {TOL[dtype]}"


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


from fp8_bounds import CODE_SPREAD, fp8_bounds  # noqa: E402,F401


# ------------------------------------------------------------------ small shapes, every element
SMALL = [
    # (B, S, H, D, P)
    (1, 16, 1, 64, 2), (2, 16, 3, 128, 1), (1, 64, 3, 64, 4), (2, 64, 1, 128, 8),
    (1, 192, 1, 128, 8), (2, 192, 3, 64, 4), (1, 200, 3, 128, 8), (2, 200, 1, 64, 5),
    (1, 576, 3, 128, 8), (2, 576, 1, 64, 3), (1, 257, 2, 128, 1), (3, 130, 2, 64, 2),
    (1, 1, 1, 128, 1), (2, 1, 2, 64, 1), (1, 320, 1, 128, 320), (1, 600, 2, 128, 6),
]


@pytest.mark.parametrize("B,S,H,D,P", SMALL)
def test_small_shapes_every_element(gpu, B, S, H, D, P):
    w = workloads.custom(B, S, H, D, P, index=1000 + S + 7 * D + B + H)
    inp = workloads.make_inputs(w)
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], P, inp["scale"])
    out = run(inp, P, gpu)
    assert tuple(out.shape) == (P, B, S // P, H, D)
    assert_gate(f64(out), ref, "bf16", f"B={B} S={S} H={H} D={D} P={P}")


@pytest.mark.parametrize("B,S,H,D,P", [(1, 64, 2, 64, 4), (2, 200, 3, 128, 8), (1, 576, 1, 128, 8)])
def test_small_shapes_fp8_every_element(gpu, B, S, H, D, P):
    w = workloads.custom(B, S, H, D, P, dtype="fp8", index=2000 + S + D)
    inp = workloads.make_inputs(w)
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], P, inp["scale"], inp["descales"])
    out = run(inp, P, gpu)
    assert_gate(f64(out), ref, "fp8", f"fp8 B={B} S={S} H={H} D={D} P={P}")


def test_tiny_workload_every_element(gpu):
    w = workloads.WORKLOADS["tiny"]
    inp = workloads.make_inputs(w)
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], w.P, inp["scale"])
    out = run(inp, w.P, gpu)
    assert_gate(f64(out), ref, "bf16", "tiny")


# ------------------------------------------------------------------ full-size workloads, sampled rows
def _sampled_parity(gpu, name, nrows):
    w = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(w)
    out = run(inp, w.P, gpu)
    rows = workloads.sample_rows(w, nrows)
    ref = oracle.attention_rows(inp["q"], inp["k"], inp["v"], rows, inp["scale"], inp["descales"])
    o = xs.unpack(out, w.S)
    idx = torch.as_tensor(rows, device=out.device)
    got = f64(o[idx[:, 0], idx[:, 1], idx[:, 2]])
    assert_gate(got, ref, w.dtype, f"{name} sampled {len(rows)} rows")
    # whole-buffer properties: finite, and every row a convex combination of V rows
    assert torch.isfinite(out.float()).all()
    return w, inp, out


@pytest.mark.parametrize("name,nrows", [("image", 256), ("video", 96), ("long", 48), ("fp8", 96)])
def test_full_size_workload_sampled_rows(gpu, name, nrows):
    _sampled_parity(gpu, name, nrows)


@pytest.mark.parametrize("B,S,H,D,P,dtype,nrows", [
    (1, 262144, 1, 128, 8, "bf16", 32),   # twice the long share's sequence, one head
    (8, 2048, 2, 64, 8, "bf16", 64),      # many batches: the relayout interleaves 8 of them
    (4, 65536, 1, 128, 16, "fp8", 32),
])
def test_large_shapes_sampled_rows(gpu, B, S, H, D, P, dtype, nrows):
    w = workloads.custom(B, S, H, D, P, dtype=dtype, index=7000 + B + H)
    inp = workloads.make_inputs(w)
    for split in ("auto", None):
        _say(f"large B={B} S={S} H={H} D={D} P={P} {dtype} split={split}")
        q, k, v = to_gpu(inp, gpu)
        if dtype == "fp8":
            out = xs.fwd_fp8(q, k, v, inp["descales"], P, inp["scale"], workspace=split)
        else:
            out = xs.fwd(q, k, v, P, inp["scale"], workspace=split)
        torch.cuda.synchronize()
        rows = workloads.sample_rows(w, nrows)
        ref = oracle.attention_rows(inp["q"], inp["k"], inp["v"], rows, inp["scale"],
                                    inp["descales"])
        o = xs.unpack(out, S)
        idx = torch.as_tensor(rows, device=out.device)
        assert_gate(f64(o[idx[:, 0], idx[:, 1], idx[:, 2]]), ref, dtype, f"split={split}")
        assert torch.isfinite(out.float()).all()


def test_image_workload_every_element(gpu):
    # 4608 x 3 rows of 4608 keys: affordable for the oracle on the host
    w = workloads.WORKLOADS["image"]
    inp = workloads.make_inputs(w)
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], w.P, inp["scale"])
    out = run(inp, w.P, gpu)
    assert_gate(f64(out), ref, "bf16", "image (all rows)")


# ------------------------------------------------------------------ bit-exact relayout and determinism
@pytest.mark.parametrize("B,S,H,D", [(2, 576, 3, 128), (3, 200, 2, 64), (2, 4096, 2, 128)])
def test_relayout_is_bit_exact(gpu, B, S, H, D):
    w = workloads.custom(B, S, H, D, 1, index=3000 + S)
    inp = workloads.make_inputs(w)
    tens = to_gpu(inp, gpu)
    base = xs.unpack(run(inp, 1, gpu, tensors=tens), S)
    for P in [p for p in (2, 4, 8, S) if S % p == 0]:
        out = run(inp, P, gpu, tensors=tens)
        want = torch.stack(torch.split(base, S // P, dim=1))  # [P][B][T][H][D]
        assert torch.equal(out.view(torch.int16), want.contiguous().view(torch.int16)), f"P={P}"


def test_deterministic_across_runs(gpu):
    w = workloads.custom(2, 1000, 3, 128, 8, index=3100)
    inp = workloads.make_inputs(w)
    tens = to_gpu(inp, gpu)
    a = run(inp, 8, gpu, tensors=tens)
    b = run(inp, 8, gpu, tensors=tens)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_output_fully_written_and_canaries_untouched(gpu):
    B, S, H, D, P = 2, 200, 3, 128, 8
    w = workloads.custom(B, S, H, D, P, index=3200)
    inp = workloads.make_inputs(w)
    q, k, v = to_gpu(inp, gpu)
    n = P * B * (S // P) * H * D
    pad = 4096
    big = torch.full((n + 2 * pad,), float("nan"), dtype=torch.bfloat16, device=gpu)
    big[:pad] = 7.0
    big[pad + n:] = -3.0
    out = big[pad:pad + n].view(P, B, S // P, H, D)
    _say("canary", B, S, H, D, P)
    xs.fwd(q, k, v, P, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any()
    assert torch.all(big[:pad] == 7.0) and torch.all(big[pad + n:] == -3.0)


# ------------------------------------------------------------------ metamorphic (bit-exact)
def test_scale_metamorphic_half_q_double_scale(gpu):
    w = workloads.custom(2, 300, 2, 128, 4, index=3300)
    inp = workloads.make_inputs(w)
    q, k, v = to_gpu(inp, gpu)
    a = run(inp, 4, gpu, tensors=(q, k, v))
    b = run(inp, 4, gpu, scale=2 * inp["scale"], tensors=(q * 0.5, k, v))  # halving bf16 is exact
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_value_linearity_double_v(gpu):
    w = workloads.custom(1, 300, 3, 64, 4, index=3400)
    inp = workloads.make_inputs(w)
    q, k, v = to_gpu(inp, gpu)
    a = run(inp, 4, gpu, tensors=(q, k, v))
    b = run(inp, 4, gpu, tensors=(q, k, v * 2))
    assert torch.equal((a * 2).view(torch.int16), b.view(torch.int16))


# ------------------------------------------------------------------ special cases
def test_constant_v_gives_constant_output(gpu):
    w = workloads.custom(1, 1000, 2, 128, 8, index=3500)
    inp = workloads.make_inputs(w)
    inp["v"] = torch.full_like(inp["v"], -1.25)
    out = run(inp, 8, gpu)
    # sum_j bf16(p_j) / sum_j p_j = 1 within the bf16 rounding averaged over the row
    # (about 1e-4), far below half an ulp of 1.25 (2^-8); -1.25 is exact in bf16
    assert torch.all(out.float() == -1.25)


def test_zero_keys_give_mean_of_values(gpu):
    w = workloads.custom(2, 512, 2, 64, 4, index=3600)
    inp = workloads.make_inputs(w)
    inp["k"] = torch.zeros_like(inp["k"])
    ref = inp["v"].double().mean(dim=1, keepdim=True).expand(2, 512, 2, 64).numpy()
    out = run(inp, 4, gpu)
    assert_gate(f64(xs.unpack(out, 512)), ref, "bf16", "K=0")


def test_one_hot_selection_is_exact(gpu):
    S = D = 64
    pi = np.array([(3 * i + 5) % S for i in range(S)])
    k = torch.zeros((1, S, 1, D), dtype=torch.bfloat16)
    q = torch.zeros((1, S, 1, D), dtype=torch.bfloat16)
    for j in range(S):
        k[0, j, 0, j] = 16.0
    for i in range(S):
        q[0, i, 0, pi[i]] = 16.0
    v = torch.randn((1, S, 1, D), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    _say("one-hot", S, D)
    out = xs.fwd(q.to(gpu), k.to(gpu), v.to(gpu), 1, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(out[0, 0, :, 0].cpu().view(torch.int16), v[0, pi, 0].view(torch.int16))


def test_single_key_returns_values(gpu):
    w = workloads.custom(2, 1, 3, 128, 1, index=3700)
    inp = workloads.make_inputs(w)
    out = run(inp, 1, gpu)
    assert torch.equal(out[0].cpu().view(torch.int16), inp["v"].view(torch.int16))


@pytest.mark.parametrize("scale", [-0.0883883461356163, 0.0])
def test_other_scales(gpu, scale):
    w = workloads.custom(1, 333, 2, 128, 9, index=3800)
    inp = workloads.make_inputs(w)
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], 9, scale)
    out = run(inp, 9, gpu, scale=scale)
    assert_gate(f64(out), ref, "bf16", f"scale={scale}")


def test_peaked_softmax_within_rounding_bound(gpu):
    # scale 0.7 at D=128 makes a few keys dominate each row, so the bf16 rounding
    # errors no longer average out.  With u = 2^-8 the unit roundoff of bf16
    # (7 stored mantissa bits), rounding each weight p_j to bf16 moves O_i by at
    # most u * sum_j w_ij |v_j|, and rounding O_i itself adds u * |O_i|; the
    # fp32 terms are far smaller.  sum_j w_ij |v_j| is the oracle run on |V|.
    w = workloads.custom(1, 333, 2, 128, 9, index=3800)
    inp = workloads.make_inputs(w)
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], 9, 0.7)
    ref_abs = oracle.attention_packed(inp["q"], inp["k"], inp["v"].abs(), 9, 0.7)
    got = f64(run(inp, 9, gpu, scale=0.7))
    u = 2.0 ** -8
    bound = u * np.abs(ref) + u * (1 + u) * ref_abs + 1e-5
    worst = float((np.abs(got - ref) / bound).max())
    print(f"  scale=0.7 worst error / bound = {worst:.3f}", flush=True)
    assert worst <= 1.0
    assert gate(got, ref, "bf16")[1] <= 1e-2


def _rising_scores(B, S, H, D, dtype, index):
    """Inputs whose scores rise along the keys: q[..., 0] = 1 and k[:, j, :, 0] = j, so
    with scale 1/sqrt(D) every 64-key block's max exceeds the previous one by about
    64 * scale * log2(e) > 8 (log2 units) and the running max moves (and O, l are
    rescaled) in nearly every block, including the ragged last one."""
    w = workloads.custom(B, S, H, D, 1, dtype=dtype, index=index)
    inp = workloads.make_inputs(w)
    if dtype == "fp8":
        dq, dk, dv = inp["descales"]
        q = inp["q"].to(torch.float32) * dq
        k = inp["k"].to(torch.float32) * dk
        q[..., 0] = 1.0
        k[..., 0] = torch.arange(S, dtype=torch.float32).view(1, S, 1)
        dq, dk = float(q.abs().max()) / 448.0, float(k.abs().max()) / 448.0
        inp["q"] = (q / dq).to(torch.float8_e4m3fn)
        inp["k"] = (k / dk).to(torch.float8_e4m3fn)
        inp["descales"] = (dq, dk, dv)
    else:
        inp["q"][..., 0] = 1.0
        inp["k"][..., 0] = torch.arange(S, dtype=torch.float32).view(1, S, 1).to(torch.bfloat16)
    return w, inp


def _sloped_scores(B, S, H, D, rise, index):
    """bf16 inputs whose scores rise linearly along the keys by `rise` log2 units
    over the whole sequence (q[..., 0] = 1, k[:, j, :, 0] = j * slope): the kernel's
    first pass keeps the first block's max, so its probabilities grow to about
    2^rise; below 2^40 that pass's result stands, above it the piece is computed
    again with the lazy rescale."""
    w = workloads.custom(B, S, H, D, 1, index=index)
    inp = workloads.make_inputs(w)
    slope = rise / ((S - 1) * inp["scale"] * math.log2(math.e))
    inp["q"][..., 0] = 1.0
    inp["k"][..., 0] = (torch.arange(S, dtype=torch.float32) * slope).view(1, S, 1).to(torch.bfloat16)
    return w, inp


@pytest.mark.parametrize("rise", [12.0, 30.0, 38.0, 44.0, 90.0, 200.0])
@pytest.mark.parametrize("B,S,H,D,P", [(2, 1024, 2, 64, 4), (2, 2048, 2, 128, 8)])
def test_scores_rising_across_the_fast_pass_limit(gpu, rise, B, S, H, D, P):
    # Rows whose running max rises by `rise` log2 units: below 2^40 the first
    # pass's probabilities (up to 2^rise) are used as they are, above it the
    # piece is redone with the lazy rescale; both must match the oracle, with and
    # without the split-key workspace (cut pieces see a smaller rise each).
    w, inp = _sloped_scores(B, S, H, D, rise, 4700 + S + D + int(rise))
    scale = inp["scale"]
    _say(f"sloped scores rise={rise} B={B} S={S} H={H} D={D} P={P}")
    ref, ref_l = oracle.attention_packed(inp["q"], inp["k"], inp["v"], P, scale, with_lse=True)
    ref_abs = oracle.attention_packed(inp["q"], inp["k"], inp["v"].abs(), P, scale)
    u = 2.0 ** -8
    bound = u * np.abs(ref) + u * (1 + u) * ref_abs + 1e-5
    q, k, v = to_gpu(inp, gpu)
    # the chunk layout too: a piece run a second time restarts the chunk cursors
    # of its K/V addresses from the piece's first block
    qc, kc, vc = (xs.chunk(t, P) for t in (q, k, v))
    for layout, args in (("bshd", (q, k, v)), ("chunked", (qc, kc, vc))):
        for ws in (None, "auto"):
            out_l, lse = xs.fwd(*args, P, scale, lse=True, workspace=ws, in_layout=layout)
            torch.cuda.synchronize()
            got = f64(out_l)
            worst = float((np.abs(got - ref) / bound).max())
            d = np.abs(f64(lse) - ref_l)
            print(f"  {layout} workspace={ws}: worst error / bound = {worst:.3f}, "
                  f"lse max_abs={d.max():.3e}", flush=True)
            assert worst <= 1.0 and np.isfinite(got).all()
            assert d.max() <= 5e-3


def _mid_block_spikes(B, S, H, D, index):
    """bf16 inputs whose large scores sit only in the last 16 keys of every 64-key
    block: q[..., 0] = 1 and k[:, j, :, 0] = (j // 64) * 16 sqrt(D) for j % 64 >= 48,
    else 0.  Each block's spike exceeds the previous block's max by 16 * 1.44 = 23
    (log2 units) while its first 48 keys score far below it, so the kernel's
    probabilities of those 48 keys pass and the overflow is found among the last
    keys, computed under the first half of P V: the running max moves after half
    the block is already weighted into O."""
    w = workloads.custom(B, S, H, D, 1, index=index)
    inp = workloads.make_inputs(w)
    j = torch.arange(S)
    spike = torch.where(j % 64 >= 48, (j // 64).to(torch.float32) * 16.0 * D ** 0.5, 0.0)
    inp["q"][..., 0] = 1.0
    inp["k"][..., 0] = spike.view(1, S, 1).to(torch.bfloat16)
    return w, inp


@pytest.mark.parametrize("B,S,H,D,P", [(2, 1000, 2, 64, 4), (1, 777, 3, 128, 7), (1, 4608, 2, 128, 8)])
def test_running_max_moves_mid_block(gpu, B, S, H, D, P):
    w, inp = _mid_block_spikes(B, S, H, D, 4600 + S + D)
    scale = inp["scale"]
    _say(f"mid-block spikes B={B} S={S} H={H} D={D} P={P}")
    ref, ref_l = oracle.attention_packed(inp["q"], inp["k"], inp["v"], P, scale, with_lse=True)
    ref_abs = oracle.attention_packed(inp["q"], inp["k"], inp["v"].abs(), P, scale)
    u = 2.0 ** -8
    bound = u * np.abs(ref) + u * (1 + u) * ref_abs + 1e-5
    q, k, v = to_gpu(inp, gpu)
    for ws in (None, "auto"):
        out = xs.fwd(q, k, v, P, scale, workspace=ws)
        out_l, lse = xs.fwd(q, k, v, P, scale, lse=True, workspace=ws)
        torch.cuda.synchronize()
        for name, o in (("O", out), ("O with lse", out_l)):
            got = f64(o)
            worst = float((np.abs(got - ref) / bound).max())
            print(f"  workspace={ws} {name}: worst error / bound = {worst:.3f}", flush=True)
            assert worst <= 1.0 and np.isfinite(got).all(), name
        d = np.abs(f64(lse) - ref_l)
        print(f"  workspace={ws} lse max_abs={d.max():.3e}", flush=True)
        assert d.max() <= 5e-3


@pytest.mark.parametrize("dtype,B,S,H,D,P", [("bf16", 2, 1000, 2, 64, 4), ("bf16", 1, 777, 3, 128, 7),
                                             ("fp8", 2, 1000, 2, 128, 8)])
def test_running_max_moves_every_block(gpu, dtype, B, S, H, D, P):
    # Rounding bound as in the peaked-softmax tests (a few keys dominate each
    # row); with the log-sum-exp checked against the oracle's at the usual bar.
    w, inp = _rising_scores(B, S, H, D, dtype, 4400 + S + D)
    scale = inp["scale"]
    _say(f"rising scores {dtype} B={B} S={S} H={H} D={D} P={P}")
    ref, ref_l = oracle.attention_packed(inp["q"], inp["k"], inp["v"], P, scale, inp["descales"],
                                         with_lse=True)
    if dtype == "fp8":
        bound_l, bound = fp8_bounds(inp, P, scale)
        q, k, v = to_gpu(inp, gpu)
        out = xs.fwd_fp8(q, k, v, inp["descales"], P, scale)
        out_l, lse = xs.fwd_fp8(q, k, v, inp["descales"], P, scale, lse=True)
    else:
        ref_abs = oracle.attention_packed(inp["q"], inp["k"], inp["v"].abs(), P, scale)
        u = 2.0 ** -8
        bound = u * np.abs(ref) + u * (1 + u) * ref_abs + 1e-5
        bound_l = bound
        q, k, v = to_gpu(inp, gpu)
        out = xs.fwd(q, k, v, P, scale)
        out_l, lse = xs.fwd(q, k, v, P, scale, lse=True)
    torch.cuda.synchronize()
    for name, o, bd in (("O", out, bound), ("O with lse", out_l, bound_l)):
        got = f64(o)
        worst = float((np.abs(got - ref) / bd).max())
        print(f"  {name}: worst error / bound = {worst:.3f}", flush=True)
        assert worst <= 1.0 and np.isfinite(got).all(), name
    d = np.abs(f64(lse) - ref_l)
    print(f"  lse max_abs={d.max():.3e}", flush=True)
    # bf16: the 5e-3 bar of the log-sum-exp tests.  fp8: the e4m3 matrix core sums
    # its products less precisely than fp32 (measured: up to 2^-12.8 of
    # scale * sum_d |q_d k_d|, test_score_accumulation_precision), and the scores
    # here reach 90: the bar adds 2^-11 scale * max_j sum_d |q_d k_jd| per row.
    bar = 5e-3
    if dtype == "fp8":
        dq, dk, _ = inp["descales"]
        qa = inp["q"].to(torch.float64).abs() * dq
        ka = inp["k"].to(torch.float64).abs() * dk
        sabs = torch.einsum("bqhd,bkhd->bhqk", qa, ka).amax(-1).numpy() * scale  # [B][H][S]
        bar = 5e-3 + 2.0 ** -11 * sabs
    assert (d <= bar).all()


# ------------------------------------------------------------------ the gate rejects wrong answers
def test_negative_controls_fail_the_gate(gpu):
    w = workloads.WORKLOADS["video"].with_(S=8192)  # same statistics, cheaper oracle
    inp = workloads.make_inputs(w)
    rows = workloads.sample_rows(w, 48)
    ref = oracle.attention_rows(inp["q"], inp["k"], inp["v"], rows, inp["scale"])
    q, k, v = to_gpu(inp, gpu)
    idx = torch.as_tensor(rows, device=gpu)

    def pick(out):
        return f64(xs.unpack(out, w.S)[idx[:, 0], idx[:, 1], idx[:, 2]])

    good = run(inp, w.P, gpu, tensors=(q, k, v))
    assert gate(pick(good), ref, "bf16")[2]
    assert not gate(np.zeros_like(ref), ref, "bf16")[2], "zeros"
    assert not gate(pick(run(inp, w.P, gpu, scale=1.0, tensors=(q, k, v))), ref, "bf16")[2], "scale"
    swapped = torch.roll(good, 1, dims=0)  # destination slices exchanged
    assert not gate(pick(swapped), ref, "bf16")[2], "slices"
    wrong_head = (q, torch.roll(k, 1, dims=2).contiguous(), torch.roll(v, 1, dims=2).contiguous())
    assert not gate(pick(run(inp, w.P, gpu, tensors=wrong_head)), ref, "bf16")[2], "head"


# ------------------------------------------------------------------ fp8 path: exactness properties
def test_fp8_relayout_is_bit_exact_and_deterministic(gpu):
    w = workloads.custom(2, 1000, 3, 128, 8, dtype="fp8", index=4000)
    inp = workloads.make_inputs(w)
    q, k, v = to_gpu(inp, gpu)
    base = xs.unpack(run(inp, 1, gpu, tensors=(q, k, v)), w.S)
    for P in (2, 8, 1000):
        out = run(inp, P, gpu, tensors=(q, k, v))
        want = torch.stack(torch.split(base, w.S // P, dim=1)).contiguous()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"P={P}"
    again = xs.unpack(run(inp, 1, gpu, tensors=(q, k, v)), w.S)
    assert torch.equal(again.view(torch.int16), base.view(torch.int16))


def test_fp8_descale_metamorphic(gpu):
    # (2 dq) * (scale / 2) = dq * scale exactly in fp32, so the exponent factor is
    # unchanged; doubling dv doubles every output exactly.
    w = workloads.custom(1, 700, 2, 128, 7, dtype="fp8", index=4100)
    inp = workloads.make_inputs(w)
    q, k, v = to_gpu(inp, gpu)
    dq, dk, dv = inp["descales"]
    _say("fp8 descale metamorphic")
    a = xs.fwd_fp8(q, k, v, (dq, dk, dv), 7, inp["scale"])
    b = xs.fwd_fp8(q, k, v, (2 * dq, dk, 2 * dv), 7, inp["scale"] / 2)
    torch.cuda.synchronize()
    assert torch.equal((a * 2).view(torch.int16), b.view(torch.int16))


def test_fp8_negative_scale(gpu):
    w = workloads.custom(2, 333, 2, 64, 3, dtype="fp8", index=4200)
    inp = workloads.make_inputs(w)
    scale = -0.0883883461356163
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], 3, scale, inp["descales"])
    out = run(inp, 3, gpu, scale=scale)
    assert_gate(f64(out), ref, "fp8", f"fp8 scale={scale}")


def test_fp8_peaked_softmax_within_rounding_bound(gpu):
    # At scale 0.25, D=64 a few keys dominate each row and the e4m3 rounding of P
    # no longer averages out: each output is held to the rounding bound of its
    # encoding of P (fp8_bounds), with and without the log-sum-exp output.  The
    # relative-L2 gate of the fp8 workloads still applies.
    w = workloads.custom(2, 333, 2, 64, 3, dtype="fp8", index=4200)
    inp = workloads.make_inputs(w)
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], 3, 0.25, inp["descales"])
    bound_l, bound = fp8_bounds(inp, 3, 0.25)
    q, k, v = to_gpu(inp, gpu)
    _say("fp8 peaked softmax, scale 0.25")
    out = xs.fwd_fp8(q, k, v, inp["descales"], 3, 0.25)
    out_l, _ = xs.fwd_fp8(q, k, v, inp["descales"], 3, 0.25, lse=True)
    torch.cuda.synchronize()
    for name, o, bd in (("O", out, bound), ("O with lse", out_l, bound_l)):
        got = f64(o)
        worst = float((np.abs(got - ref) / bd).max())
        print(f"  fp8 scale=0.25 {name}: worst error / bound = {worst:.3f}", flush=True)
        assert worst <= 1.0, name
        assert gate(got, ref, "fp8")[1] <= TOL["fp8"][1], name


def test_fp8_constant_v_gives_constant_output(gpu):
    # Without the log-sum-exp output O is normalised by the sum of the same
    # quantised probabilities that weight V, so a constant V comes back exactly
    # (1.5 * 0.5 = 0.75 is exact in bf16).  With it, O is normalised by the fp32
    # sum of the unquantised probabilities, within the e4m3 rounding of P.
    w = workloads.custom(2, 1000, 2, 128, 8, dtype="fp8", index=4300)
    inp = workloads.make_inputs(w)
    q, k, _ = to_gpu(inp, gpu)
    v = torch.full_like(q, 1.5)
    dq, dk, _ = inp["descales"]
    _say("fp8 constant V")
    out = xs.fwd_fp8(q, k, v, (dq, dk, 0.5), 8, inp["scale"])
    out_l, _ = xs.fwd_fp8(q, k, v, (dq, dk, 0.5), 8, inp["scale"], lse=True)
    torch.cuda.synchronize()
    assert torch.all(out.float() == 0.75)
    assert float((out_l.float() - 0.75).abs().max()) <= 0.75 * 2.0 ** -4


def test_fp8_canaries_and_full_write(gpu):
    B, S, H, D, P = 2, 130, 2, 64, 2
    w = workloads.custom(B, S, H, D, P, dtype="fp8", index=4300)
    inp = workloads.make_inputs(w)
    q, k, v = to_gpu(inp, gpu)
    n = P * B * (S // P) * H * D
    pad = 2048
    big = torch.full((n + 2 * pad,), float("nan"), dtype=torch.bfloat16, device=gpu)
    big[:pad] = 5.0
    big[pad + n:] = -9.0
    out = big[pad:pad + n].view(P, B, S // P, H, D)
    _say("fp8 canary", B, S, H, D, P)
    xs.fwd_fp8(q, k, v, inp["descales"], P, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any()
    assert torch.all(big[:pad] == 5.0) and torch.all(big[pad + n:] == -9.0)
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], P, inp["scale"], inp["descales"])
    assert_gate(f64(out), ref, "fp8", "fp8 canary case")


# ------------------------------------------------------------------ split-key schedule
def test_split_and_unsplit_agree_with_the_oracle(gpu):
    # the image share: 54 tiles of 256 rows on a 256-CU GPU -> the key range is split
    w = workloads.WORKLOADS["image"]
    inp = workloads.make_inputs(w)
    assert xs.split_count(w.B, w.S, w.H, w.D) > 1
    q, k, v = to_gpu(inp, gpu)
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], w.P, inp["scale"])
    _say("image split vs unsplit")
    split = xs.fwd(q, k, v, w.P, inp["scale"])
    whole = xs.fwd(q, k, v, w.P, inp["scale"], workspace=None)
    torch.cuda.synchronize()
    assert_gate(f64(split), ref, "bf16", "image split")
    assert_gate(f64(whole), ref, "bf16", "image unsplit")
    assert float((split.float() - whole.float()).abs().max()) <= 2e-3


def test_split_fp8_agrees_with_the_oracle(gpu):
    w = workloads.custom(1, 4608, 3, 128, 8, dtype="fp8", index=4400)
    inp = workloads.make_inputs(w)
    assert xs.split_count(w.B, w.S, w.H, w.D) > 1
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], w.P, inp["scale"], inp["descales"])
    out = run(inp, w.P, gpu)
    assert_gate(f64(out), ref, "fp8", "fp8 split")


def test_explicit_workspace_reused_twice(gpu):
    w = workloads.custom(2, 1000, 3, 64, 8, index=4500)
    inp = workloads.make_inputs(w)
    q, k, v = to_gpu(inp, gpu)
    n = xs.workspace_size(2, 1000, 3, 64)
    assert n > 0
    ws = torch.full((n,), 255, dtype=torch.uint8, device=gpu)  # stale contents must not matter
    _say("explicit workspace")
    a = xs.fwd(q, k, v, 8, workspace=ws)
    b = xs.fwd(q, k, v, 8, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], 8, inp["scale"])
    assert_gate(f64(a), ref, "bf16", "explicit workspace")
    small = torch.empty(n - 16, dtype=torch.uint8, device=gpu)
    with pytest.raises(xs.XsAttnError):
        xs.fwd(q, k, v, 8, workspace=small)


@pytest.mark.parametrize("B,S,H,D", [(1, 2048, 7, 128), (3, 700, 5, 64), (1, 4672, 2, 128),
                                     (2, 1000, 3, 128), (1, 8256, 1, 64)])
def test_persistent_schedule_cut_tiles(gpu, B, S, H, D):
    # shapes whose schedule cuts tiles at varied offsets (odd block counts,
    # several pieces per tile, shares starting on and off tile boundaries):
    # the merged result meets the bar and stays close to the uncut schedule
    w = workloads.custom(B, S, H, D, 1, index=4600 + S + H)
    inp = workloads.make_inputs(w)
    _say(f"schedule B={B} S={S} H={H} D={D} pieces<={xs.split_count(B, S, H, D)}")
    q, k, v = to_gpu(inp, gpu)
    cut = xs.fwd(q, k, v, 1, inp["scale"])
    whole = xs.fwd(q, k, v, 1, inp["scale"], workspace=None)
    again = xs.fwd(q, k, v, 1, inp["scale"])
    torch.cuda.synchronize()
    assert torch.equal(cut.view(torch.int16), again.view(torch.int16))  # deterministic
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], 1, inp["scale"])
    assert_gate(f64(cut), ref, "bf16", "cut schedule")
    assert_gate(f64(whole), ref, "bf16", "uncut schedule")
    assert float((cut.float() - whole.float()).abs().max()) <= 2e-3


# ------------------------------------------------------------------ a call on a stream other than the current one
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_side_stream_with_auto_workspace(gpu, dtype):
    # The image share (its plan cuts every tile, so the call allocates a
    # workspace, the output and the log-sum-exp itself) on a side stream, while
    # the current stream allocates and overwrites memory of the same sizes right
    # after the call is enqueued: the call's buffers must come from the side
    # stream's pool, so that nothing freed on return is reused before the side
    # stream's kernels are done with it.
    w = workloads.WORKLOADS["image"].with_(dtype=dtype, index=8300 + (dtype == "fp8"))
    inp = workloads.make_inputs(w)
    assert xs.split_count(w.B, w.S, w.H, w.D) > 1
    q, k, v = to_gpu(inp, gpu)
    ref, ref_l = oracle.attention_packed(inp["q"], inp["k"], inp["v"], w.P, inp["scale"],
                                         inp["descales"], with_lse=True)
    side = torch.cuda.Stream(gpu)
    side.wait_stream(torch.cuda.current_stream(gpu))
    ws_bytes = xs.workspace_size(w.B, w.S, w.H, w.D)
    results = []
    _say(f"side stream {dtype} image share, workspace {ws_bytes} B")
    for _ in range(3):
        if dtype == "fp8":
            out, lse = xs.fwd_fp8(q, k, v, inp["descales"], w.P, inp["scale"], stream=side,
                                  workspace="auto", lse=True)
        else:
            out, lse = xs.fwd(q, k, v, w.P, inp["scale"], stream=side, workspace="auto", lse=True)
        # the current stream allocates and fills blocks of the workspace's size
        junk = [torch.full((ws_bytes // 4,), -7.0, device=gpu) for _ in range(2)]
        results.append((out, lse))
        del junk
    torch.cuda.current_stream(gpu).wait_stream(side)
    torch.cuda.synchronize()
    for out, lse in results:
        assert_gate(f64(out), ref, dtype, f"{dtype} side stream")
        assert float(np.abs(f64(lse) - ref_l).max()) <= 5e-3


# ------------------------------------------------------------------ fp8: running max moving inside a block (lse path)
def _fp8_block_spikes(B, S, H, D, lo, hi, index):
    """fp8 inputs whose large scores sit only in keys lo..hi-1 of every 64-key
    block: q[..., 0] = 1 and k[:, j, :, 0] = (j // 64) * 16 sqrt(D) there, else 0,
    then requantised to e4m3 with fresh per-tensor descales.  Each block's spike
    exceeds the previous block's max by about 16 * 1.44 = 23 (log2 units), so the
    kernel's probabilities computed with the running max overflow in exactly
    those keys and the max moves every block."""
    w = workloads.custom(B, S, H, D, 1, dtype="fp8", index=index)
    inp = workloads.make_inputs(w)
    dq, dk, dv = inp["descales"]
    q = inp["q"].to(torch.float32) * dq
    k = inp["k"].to(torch.float32) * dk
    j = torch.arange(S)
    inb = (j % 64 >= lo) & (j % 64 < hi)
    spike = torch.where(inb, (j // 64).to(torch.float32) * 16.0 * D ** 0.5, 0.0)
    q[..., 0] = 1.0
    k[..., 0] = spike.view(1, S, 1)
    dq, dk = float(q.abs().max()) / 448.0, float(k.abs().max()) / 448.0
    inp["q"] = (q / dq).to(torch.float8_e4m3fn)
    inp["k"] = (k / dk).to(torch.float8_e4m3fn)
    inp["descales"] = (dq, dk, dv)
    return w, inp


@pytest.mark.parametrize("lo,hi", [(16, 32), (48, 64)])
def test_fp8_running_max_moves_mid_block_with_lse(gpu, lo, hi):
    # Keys 0..31 of a block have their probabilities computed under the P V of
    # the block before, keys 32..63 under the block's own QK^T; with the
    # log-sum-exp requested the kernel takes no per-block max and finds the
    # overflow from the lane's sum of the new probabilities.  Spikes in either
    # half must move the running max before any of the block enters P V.
    B, S, H, D, P = 2, 1000, 2, 128, 8
    w, inp = _fp8_block_spikes(B, S, H, D, lo, hi, 4700 + lo)
    scale = inp["scale"]
    _say(f"fp8 spikes in keys {lo}..{hi - 1} of every block B={B} S={S} H={H} D={D} P={P}")
    ref, ref_l = oracle.attention_packed(inp["q"], inp["k"], inp["v"], P, scale, inp["descales"],
                                         with_lse=True)
    dq, dk, dv = inp["descales"]
    qf, kf = inp["q"].to(torch.float64) * dq, inp["k"].to(torch.float64) * dk
    bound_l, bound = fp8_bounds(inp, P, scale)  # rounding bounds of the two encodings of P
    # log-sum-exp bar: 5e-3 plus the e4m3 matrix core's score accumulation
    sabs = torch.einsum("bqhd,bkhd->bhqk", qf.abs(), kf.abs()).amax(-1).numpy() * scale
    bar = 5e-3 + 2.0 ** -11 * sabs
    q, k, v = to_gpu(inp, gpu)
    for ws in (None, "auto"):
        out, lse = xs.fwd_fp8(q, k, v, inp["descales"], P, scale, lse=True, workspace=ws)
        plain = xs.fwd_fp8(q, k, v, inp["descales"], P, scale, workspace=ws)
        torch.cuda.synchronize()
        for name, o, bd in (("O with lse", out, bound_l), ("O", plain, bound)):
            got = f64(o)
            worst = float((np.abs(got - ref) / bd).max())
            print(f"  workspace={ws} {name}: worst error / bound = {worst:.3f}", flush=True)
            assert np.isfinite(got).all() and worst <= 1.0, name
        d = np.abs(f64(lse) - ref_l)
        print(f"  workspace={ws} lse max_abs={d.max():.3e}", flush=True)
        assert np.isfinite(d).all() and (d <= bar).all()
