"""Seeded synthetic inputs for the attention share: the named workloads and a
generic generator for test shapes.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no attention arithmetic: it only draws q, k, v on the CPU from a seeded
generator and, for the fp8 workload, quantises them to OCP e4m3 with
per-tensor scales.  The same bytes feed the CPU oracle and the GPU library.

Recipe (the pages fix no distribution; these are the workload definitions):
  * torch.Generator('cpu').manual_seed(seed); draw q, k, v in that order as
    torch.randn(B, S, H, D, float32) * sigma, then round to bf16 (RNE).
  * fp8: the same fp32 draws; descale_x = amax(|x|) / 448 in fp32;
    x8 = clamp(x / descale_x, -448, 448) converted to float8_e4m3fn (RNE).
  * scale = float32(1 / sqrt(D)).
  * seed = 20260728 + the workload's index.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

SEED_BASE = 20260728
FP8_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    S: int
    H: int
    D: int
    P: int
    sigma: float = 1.0
    dtype: str = "bf16"  # "bf16" or "fp8"
    note: str = ""

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index

    @property
    def flops(self) -> float:
        """4*B*H*S^2*D: the two contractions QK^T and PV."""
        return 4.0 * self.B * self.H * self.S * self.S * self.D

    @property
    def algorithmic_bytes(self) -> float:
        """Read q, k, v once and write the bf16 output once."""
        elems = self.B * self.S * self.H * self.D
        in_bytes = 1 if self.dtype == "fp8" else 2
        return 3.0 * elems * in_bytes + 2.0 * elems

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 0, B=1, S=256, H=2, D=64, P=2,
                 note="P=2 sequence slices of 128 rows"),
        Workload("image", 1, B=1, S=4608, H=3, D=128, P=8,
                 note="DiT image share: 4096 image-patch + 512 text tokens, 24 heads / P=8"),
        Workload("video", 2, B=1, S=32768, H=5, D=128, P=8,
                 note="DiT video share: 40 heads / P=8"),
        Workload("long", 3, B=1, S=131072, H=3, D=128, P=8, sigma=0.5,
                 note="long-sequence share, N(0, 0.5^2)"),
        Workload("fp8", 4, B=2, S=32768, H=4, D=128, P=8, dtype="fp8",
                 note="e4m3 inputs with per-tensor fp32 scales"),
    ]
}


def softmax_scale(D: int) -> float:
    """float32(1/sqrt(D)) as a Python float."""
    return float(np.float32(1.0 / math.sqrt(D)))


def _draw(B, S, H, D, sigma, gen):
    x = torch.randn((B, S, H, D), generator=gen, dtype=torch.float32)
    if sigma != 1.0:
        x = x * sigma
    return x


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor OCP e4m3 quantisation: returns (codes, descale) with x ~ codes * descale."""
    amax = float(x.abs().max())
    descale = float(np.float32(amax / FP8_MAX)) if amax > 0 else 1.0
    q = (x / descale).clamp_(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q, descale


def make_inputs(w: Workload, seed: int | None = None):
    """Return dict(q, k, v, scale, descales, workload) with CPU tensors."""
    gen = torch.Generator("cpu")
    gen.manual_seed(w.seed if seed is None else seed)
    xs = [_draw(w.B, w.S, w.H, w.D, w.sigma, gen) for _ in range(3)]
    out = {"workload": w, "scale": softmax_scale(w.D)}
    if w.dtype == "fp8":
        qs = [quantize_e4m3(x) for x in xs]
        out["q"], out["k"], out["v"] = (t for t, _ in qs)
        out["descales"] = tuple(d for _, d in qs)
    else:
        out["q"], out["k"], out["v"] = (x.to(torch.bfloat16) for x in xs)
        out["descales"] = (1.0, 1.0, 1.0)
    return out


def custom(B, S, H, D, P, dtype="bf16", sigma=1.0, index=100, name="custom") -> Workload:
    return Workload(name, index, B=B, S=S, H=H, D=D, P=P, sigma=sigma, dtype=dtype)


def sample_rows(w: Workload, n: int, seed: int = 0) -> np.ndarray:
    """A deterministic (n, 3) sample of (b, s, h) rows that touches every
    destination slice, every head and the first/last rows."""
    rng = np.random.default_rng(seed + w.index)
    T = w.S // w.P
    rows = []
    for p in range(w.P):  # first and last row of every slice
        rows.append((0, p * T, p % w.H))
        rows.append((w.B - 1, p * T + T - 1, (p + 1) % w.H))
    while len(rows) < n:
        rows.append((int(rng.integers(w.B)), int(rng.integers(w.S)), int(rng.integers(w.H))))
    return np.asarray(rows[:max(n, 2 * w.P)], dtype=np.int64)
