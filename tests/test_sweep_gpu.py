"""Seeded sweep of shapes through the C ABI against the oracle, every element.

Shapes, dtypes, schedules (with or without the split-key workspace) and input
layouts are drawn once from a fixed seed, so the list is the same on every run.
They cover what the fixed cases leave to chance: every residue of the key count
modulo the 64-key block and of the block count modulo the four-stage LDS ring
(so every tail length of a piece), pieces that start and end anywhere in a
tile, destination slices that straddle tiles, and B, H, P combinations.  Bars
as in the parity tests: max-abs 1e-2 / 5e-2 (fp8: or the per-element bound of its
encoding of P, where larger) and rel-L2 1e-2 / 8e-2 on O, 5e-3 on the log-sum-exp.
"""
import os

import numpy as np
import pytest
import torch

import sequence_attention_amd as xs
import workloads
from fp8_bounds import fp8_bounds
from oracle import oracle

pytestmark = pytest.mark.gpu

TOL = {"bf16": (1e-2, 1e-2), "fp8": (5e-2, 8e-2)}


def _cases(n=40, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 4))
        H = int(rng.integers(1, 4))
        nblk = int(rng.integers(1, 13))                    # key blocks: 1 .. 12
        S = max(1, 64 * (nblk - 1) + int(rng.integers(1, 65)))
        divisors = [p for p in range(1, min(S, 16) + 1) if S % p == 0]
        P = int(rng.choice(divisors))
        dtype = "fp8" if rng.random() < 0.3 else "bf16"
        split = bool(rng.random() < 0.6)
        chunked = bool(rng.random() < 0.3) and (B == 1 or P == 1 or (S // P) % 64 == 0)
        out.append((i, dtype, B, S, H, D, P, split, chunked))
    return out


# XS_SWEEP_CASES widens the sweep (same seed: the first 40 cases are always these)
@pytest.mark.parametrize("i,dtype,B,S,H,D,P,split,chunked",
                         _cases(int(os.environ.get("XS_SWEEP_CASES", "40"))))
def test_sweep(gpu, i, dtype, B, S, H, D, P, split, chunked):
    w = workloads.custom(B, S, H, D, P, dtype=dtype, index=6000 + i)
    inp = workloads.make_inputs(w)
    layout = "chunked" if chunked else "bshd"
    print(f"[case] sweep {i}: {dtype} B={B} S={S} H={H} D={D} P={P} split={split} "
          f"layout={layout} pieces={xs.split_count(B, S, H, D)}", flush=True)
    ref_o, ref_l = oracle.attention_packed(inp["q"], inp["k"], inp["v"], P, inp["scale"],
                                           inp["descales"], with_lse=True)
    q, k, v = (inp[n] for n in "qkv")
    if chunked:
        q, k, v = (xs.chunk(t, P) for t in (q, k, v))
    q, k, v = (t.to(gpu) for t in (q, k, v))
    ws = "auto" if split else None
    if dtype == "fp8":
        out, lse = xs.fwd_fp8(q, k, v, inp["descales"], P, inp["scale"], workspace=ws, lse=True,
                              in_layout=layout)
        plain = xs.fwd_fp8(q, k, v, inp["descales"], P, inp["scale"], workspace=ws,
                           in_layout=layout)
    else:
        out, lse = xs.fwd(q, k, v, P, inp["scale"], workspace=ws, lse=True, in_layout=layout)
        plain = xs.fwd(q, k, v, P, inp["scale"], workspace=ws, in_layout=layout)
    torch.cuda.synchronize()
    ta, tr = TOL[dtype]
    # fp8: the flat max-abs bar is stated for the workloads' |O| (outputs averaged
    # over thousands of keys); a row over a handful of keys is held to the larger
    # of that bar and the per-element bound derived from P's encoding
    bars = {"O": ta, "O with lse": ta}
    if dtype == "fp8":
        b_lse, b_plain = fp8_bounds(inp, P, inp["scale"])
        bars = {"O": np.maximum(ta, b_plain), "O with lse": np.maximum(ta, b_lse)}
    for name, o in (("O", plain), ("O with lse", out)):
        got = o.float().cpu().numpy().astype(np.float64)
        err = np.abs(got - ref_o)
        rel = float(np.linalg.norm(got - ref_o) / np.linalg.norm(ref_o))
        worst = float((err / bars[name]).max())
        print(f"  {name}: max_abs={err.max():.3e} rel_l2={rel:.3e} worst error / bar={worst:.3f}",
              flush=True)
        assert np.isfinite(got).all() and worst <= 1.0 and rel <= tr, name
    if dtype == "bf16":  # the log-sum-exp output does not change O
        assert torch.equal(out.view(torch.int16), plain.view(torch.int16))
    d = float(np.abs(lse.cpu().numpy().astype(np.float64) - ref_l).max())
    print(f"  lse max_abs={d:.3e}", flush=True)
    assert d <= 5e-3
