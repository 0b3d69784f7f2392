"""HIP-graph capture of the library call (through the C ABI, via the binding).

The path launches kernels only -- the attention kernel and, when the plan cuts
tiles, the merge kernel; no memset, no allocation, no host synchronisation
inside the call -- so a captured call replays.  Every replay must equal an
eager call on the inputs current at replay time, bit for bit (same kernels,
same schedule, same workspace), with eager work and synchronisations between
the replays.
"""
import pytest
import torch

import sequence_attention_amd as xs
import workloads

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("dtype,B,S,H,D,P", [
    ("bf16", 1, 4608, 3, 128, 8),   # the image share: cut tiles, two kernels per call
    ("bf16", 2, 576, 2, 64, 3),
    ("fp8", 2, 1024, 2, 128, 8),
])
def test_graph_replay_matches_eager(gpu, dtype, B, S, H, D, P):
    w = workloads.custom(B, S, H, D, P, dtype=dtype, index=5000 + S + D)
    inp = workloads.make_inputs(w)
    q, k, v = [inp[n].to(gpu) for n in "qkv"]
    out = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device=gpu)
    nbytes = xs.workspace_size(B, S, H, D)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=gpu) if nbytes else None
    _say(f"graph {dtype} B={B} S={S} H={H} D={D} P={P} split={xs.split_count(B, S, H, D)}")

    def call(o):
        if dtype == "fp8":
            xs.fwd_fp8(q, k, v, inp["descales"], P, inp["scale"], out=o, workspace=ws)
        else:
            xs.fwd(q, k, v, P, inp["scale"], out=o, workspace=ws)

    # warm up on a side stream, then capture (torch's capture recipe)
    side = torch.cuda.Stream(gpu)
    side.wait_stream(torch.cuda.current_stream(gpu))
    with torch.cuda.stream(side):
        call(out)
    torch.cuda.current_stream(gpu).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out)
    torch.cuda.synchronize()

    gen = torch.Generator().manual_seed(7)
    ref = torch.empty_like(out)
    for r in range(4):
        if r:  # eager work between replays: fresh query values, written in place
            src = torch.randn(tuple(q.shape), generator=gen) * 0.7
            if dtype == "fp8":
                src = (src / inp["descales"][0]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
            else:
                src = src.to(torch.bfloat16)
            q.copy_(src.to(gpu))
        call(ref)  # eager reference on the same inputs and workspace
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {r}"
