"""xs_attn_fwd_noalloc (through the C ABI) against xs_attn_fwd_ws, the entry
point it is a variant of: the same schedule and kernels with the split-key
partials in the library's static device scratch instead of a caller workspace.

Two calls in a row, the second with a smaller input (so it runs on whatever the
first left in the scratch); each output must equal xs_attn_fwd_ws's bit for bit
and meet the oracle bar (max-abs 1e-2, relative L2 1e-2) on every element.
"""
import numpy as np
import pytest
import torch

import sequence_attention_amd as xs
import workloads
from oracle import oracle
from sequence_attention_amd import _lib

pytestmark = pytest.mark.gpu


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_noalloc_matches_workspace_entry_two_calls(gpu):
    L = _lib.lib()
    stream = torch.cuda.current_stream(gpu).cuda_stream
    shapes = [(1, 4608, 3, 128, 8), (2, 1000, 3, 64, 8)]  # the image share, then a smaller one
    for i, (B, S, H, D, P) in enumerate(shapes):
        w = workloads.custom(B, S, H, D, P, index=8400 + i)
        inp = workloads.make_inputs(w)
        q, k, v = (inp[n].to(gpu) for n in "qkv")
        need = xs.workspace_size(B, S, H, D)
        print(f"[case] noalloc call {i}: B={B} S={S} H={H} D={D} P={P}, partials {need} B",
              flush=True)
        assert 0 < need <= 68157440, "the shape must cut tiles and fit the scratch"
        out_na = torch.full((P, B, S // P, H, D), float("nan"), dtype=torch.bfloat16, device=gpu)
        rc = L.xs_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out_na.data_ptr(),
                                   B, S, H, D, P, inp["scale"], stream)
        assert rc == 0, xs.xs_attn_strerror(rc)
        ws = torch.empty(need, dtype=torch.uint8, device=gpu)
        out_ws = torch.full_like(out_na, float("nan"))
        rc = L.xs_attn_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), out_ws.data_ptr(), B, S, H,
                              D, P, inp["scale"], ws.data_ptr(), need, stream)
        assert rc == 0, xs.xs_attn_strerror(rc)
        torch.cuda.synchronize()
        assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16)), f"call {i}"
        ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], P, inp["scale"])
        got = _f64(out_na)
        max_abs = float(np.abs(got - ref).max())
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        print(f"  max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
        assert np.isfinite(got).all() and max_abs <= 1e-2 and rel <= 1e-2
