"""Fused Ulysses-share attention forward for MI355X (gfx950).

Thin Python binding over libxs_attn.so (include/xs_attn.h).  Every step of the
computation runs in the library's HIP kernels; this module only checks tensor
metadata, allocates the output with torch and passes pointers and the current
HIP stream.  There is no CPU or PyTorch fallback: if the library is missing,
the calls raise.

    out_packed = fwd(q, k, v, P)            # bf16 q/k/v [B][S][H][D] on the GPU
    out_packed = fwd_fp8(q8, k8, v8, descales, P)
    o = unpack(out_packed, S)               # back to [B][S][H][D] (a torch view)
    out_packed, lse = fwd(q, k, v, P, lse=True)          # + [B][H][S] fp32 log-sum-exp
    out_packed = fwd(qc, kc, vc, P, in_layout="chunked")  # inputs [P][B][S/P][H][D]

By default the calls use the split-key schedule when it fills the GPU better,
with a workspace allocated from torch's caching allocator (pass a tensor of
at least workspace_size(...) bytes to reuse one, or workspace=None to run
unsplit).  The call runs on `stream` (a torch stream or a raw hipStream_t
handle; default the current stream), and the buffers it allocates come from
that stream's pool.  A caller-provided out, lse or workspace that another
stream uses must be ordered by the caller (events or record_stream).
"""
from __future__ import annotations

import contextlib
import math

import numpy as np
import torch

from ._lib import XsAttnError, check, declared_functions, lib, strerror

__all__ = ["fwd", "fwd_fp8", "unpack", "chunk", "workspace_size", "split_count", "xs_attn_fwd",
           "xs_attn_fwd_fp8", "xs_attn_fwd_ws", "xs_attn_fwd_fp8_ws", "xs_attn_fwd_ex",
           "xs_attn_fwd_fp8_ex", "xs_attn_workspace_size", "xs_attn_split_count",
           "xs_attn_schedule", "xs_attn_fwd_noalloc",
           "xs_attn_strerror", "xs_attn_version", "XsAttnError", "default_scale",
           "LAYOUT_BSHD", "LAYOUT_CHUNKED", "ONE_LAUNCH"]

LAYOUT_BSHD, LAYOUT_CHUNKED = 0, 1  # include/xs_attn.h XS_LAYOUT_*
ONE_LAUNCH = 0x100  # include/xs_attn.h XS_ONE_LAUNCH, OR-ed into the layout code


def default_scale(D: int) -> float:
    """float32(1/sqrt(D))."""
    return float(np.float32(1.0 / math.sqrt(D)))


def _alloc_on(s, out, lse, workspace):
    """Context in which the call's own buffers are allocated: the call's stream
    when anything is to be allocated (nothing to switch otherwise)."""
    if out is None or lse is True or isinstance(workspace, str):
        return torch.cuda.stream(s)
    return contextlib.nullcontext()


def _stream(t: torch.Tensor, stream) -> torch.cuda.Stream:
    """The stream the call runs on, as a torch stream: the current one by
    default; a raw hipStream_t handle (int) is wrapped, not copied."""
    if stream is None:
        return torch.cuda.current_stream(t.device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=t.device)


def _check_inputs(q, k, v, dtype, P, in_layout):
    """Validate q/k/v metadata; returns (B, S, H, D, layout code)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a GPU tensor")
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.shape != q.shape or t.device != q.device:
            raise ValueError("q, k, v must share shape and device")
    if in_layout == "bshd":
        if q.dim() != 4:
            raise ValueError("bshd inputs must be [B][S][H][D]")
        B, S, H, D = q.shape
        return B, S, H, D, LAYOUT_BSHD
    if in_layout == "chunked":
        if q.dim() != 5 or q.shape[0] != P:
            raise ValueError("chunked inputs must be [P][B][S/P][H][D]")
        _, B, T, H, D = q.shape
        return B, P * T, H, D, LAYOUT_CHUNKED
    raise ValueError("in_layout must be 'bshd' or 'chunked'")


def _lse(q, B, S, H, lse):
    """Resolve the lse argument to a tensor or None."""
    if lse is None or lse is False:
        return None
    if lse is True:
        return torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if (not isinstance(lse, torch.Tensor) or not lse.is_cuda or lse.dtype != torch.float32
            or tuple(lse.shape) != (B, H, S) or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 GPU tensor of shape {(B, H, S)}")
    return lse


def _out(q, B, S, H, D, P, out):
    if S % P:
        raise ValueError(f"S={S} is not a multiple of P={P}")
    shape = (P, B, S // P, H, D)
    if out is None:
        return torch.empty(shape, dtype=torch.bfloat16, device=q.device)
    if out.shape != shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bf16 tensor of shape {shape}")
    return out


def xs_attn_fwd(q, k, v, out_packed, B, S, H_local, D, P, scale, stream) -> int:
    """Raw C-ABI call: pointers (ints or tensors), sizes, scale, stream handle. Returns the status."""
    ptr = lambda x: x.data_ptr() if isinstance(x, torch.Tensor) else x
    return lib().xs_attn_fwd(ptr(q), ptr(k), ptr(v), ptr(out_packed), B, S, H_local, D, P,
                             float(scale), stream)


def xs_attn_fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, out_packed, B, S, H_local, D, P,
                    scale, stream) -> int:
    ptr = lambda x: x.data_ptr() if isinstance(x, torch.Tensor) else x
    return lib().xs_attn_fwd_fp8(ptr(q8), ptr(k8), ptr(v8), float(q_descale), float(k_descale),
                                 float(v_descale), ptr(out_packed), B, S, H_local, D, P,
                                 float(scale), stream)


def xs_attn_fwd_ws(q, k, v, out_packed, B, S, H_local, D, P, scale, workspace, workspace_bytes,
                   stream) -> int:
    ptr = lambda x: x.data_ptr() if isinstance(x, torch.Tensor) else x
    return lib().xs_attn_fwd_ws(ptr(q), ptr(k), ptr(v), ptr(out_packed), B, S, H_local, D, P,
                                float(scale), ptr(workspace), int(workspace_bytes), stream)


def xs_attn_fwd_fp8_ws(q8, k8, v8, q_descale, k_descale, v_descale, out_packed, B, S, H_local, D,
                       P, scale, workspace, workspace_bytes, stream) -> int:
    ptr = lambda x: x.data_ptr() if isinstance(x, torch.Tensor) else x
    return lib().xs_attn_fwd_fp8_ws(ptr(q8), ptr(k8), ptr(v8), float(q_descale), float(k_descale),
                                    float(v_descale), ptr(out_packed), B, S, H_local, D, P,
                                    float(scale), ptr(workspace), int(workspace_bytes), stream)


def xs_attn_fwd_ex(q, k, v, in_layout, out_packed, lse, B, S, H_local, D, P, scale, workspace,
                   workspace_bytes, stream) -> int:
    ptr = lambda x: x.data_ptr() if isinstance(x, torch.Tensor) else x
    return lib().xs_attn_fwd_ex(ptr(q), ptr(k), ptr(v), int(in_layout), ptr(out_packed), ptr(lse),
                                B, S, H_local, D, P, float(scale), ptr(workspace),
                                int(workspace_bytes), stream)


def xs_attn_fwd_fp8_ex(q8, k8, v8, in_layout, q_descale, k_descale, v_descale, out_packed, lse, B,
                       S, H_local, D, P, scale, workspace, workspace_bytes, stream) -> int:
    ptr = lambda x: x.data_ptr() if isinstance(x, torch.Tensor) else x
    return lib().xs_attn_fwd_fp8_ex(ptr(q8), ptr(k8), ptr(v8), int(in_layout), float(q_descale),
                                    float(k_descale), float(v_descale), ptr(out_packed), ptr(lse),
                                    B, S, H_local, D, P, float(scale), ptr(workspace),
                                    int(workspace_bytes), stream)


def xs_attn_fwd_noalloc(q, k, v, out_packed, B, S, H_local, D, P, scale, stream) -> int:
    ptr = lambda x: x.data_ptr() if isinstance(x, torch.Tensor) else x
    return lib().xs_attn_fwd_noalloc(ptr(q), ptr(k), ptr(v), ptr(out_packed), B, S, H_local, D,
                                     P, float(scale), stream)


def xs_attn_workspace_size(B, S, H_local, D) -> int:
    return int(lib().xs_attn_workspace_size(B, S, H_local, D))


def xs_attn_split_count(B, S, H_local, D) -> int:
    return int(lib().xs_attn_split_count(B, S, H_local, D))


def xs_attn_schedule(B, S, H_local, D, with_workspace=True, fp8=False) -> dict:
    """The schedule the library runs for this shape on the current device:
    {"groups", "whole_rounds", "pieces", "half_tiles"} (pieces = most pieces a tile is
    cut into; half_tiles = 128-row tiles of a second launch; fp8 calls are scheduled alike)."""
    import ctypes

    g, r, p, h = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    check(lib().xs_attn_schedule_ex(B, S, H_local, D, int(bool(with_workspace)), int(bool(fp8)),
                                    ctypes.byref(g), ctypes.byref(r), ctypes.byref(p),
                                    ctypes.byref(h)))
    return {"groups": g.value, "whole_rounds": r.value, "pieces": p.value,
            "half_tiles": h.value}


workspace_size = xs_attn_workspace_size
split_count = xs_attn_split_count


def _workspace(q, B, S, H, D, workspace):
    """Resolve the workspace argument to (pointer-or-tensor, bytes)."""
    if workspace is None:
        return None, 0
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be a tensor, None or 'auto'")
        n = xs_attn_workspace_size(B, S, H, D)
        if n == 0:
            return None, 0
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
        raise TypeError("workspace must be a GPU tensor")
    return workspace, workspace.numel() * workspace.element_size()


def xs_attn_strerror(status: int) -> str:
    return strerror(status)


def xs_attn_version() -> int:
    return int(lib().xs_attn_version())


def fwd(q, k, v, P: int, scale: float | None = None, out=None, stream=None,
        workspace="auto", lse=None, in_layout: str = "bshd"):
    """Attention over bf16 inputs; returns bf16 out_packed [P][B][S/P][H][D].

    q, k, v are [B][S][H][D] (in_layout="bshd") or [P][B][S/P][H][D]
    (in_layout="chunked", what the pre-attention All-to-All delivers).  With
    lse=True (or a [B][H][S] float32 tensor) the rows' natural-log log-sum-exp is
    written too and (out_packed, lse) is returned."""
    B, S, H, D, code = _check_inputs(q, k, v, torch.bfloat16, P, in_layout)
    s = _stream(q, stream)
    # Buffers allocated here come from the caching allocator's pool of the stream
    # the kernels run on, so a block freed on return is not handed to another
    # stream's allocation while those kernels may still write it.
    with _alloc_on(s, out, lse, workspace):
        out = _out(q, B, S, H, D, P, out)
        lse_t = _lse(q, B, S, H, lse)
        ws, nbytes = _workspace(q, B, S, H, D, workspace)
    scale = default_scale(D) if scale is None else float(scale)
    check(xs_attn_fwd_ex(q, k, v, code, out, lse_t, B, S, H, D, P, scale, ws, nbytes,
                         s.cuda_stream))
    return (out, lse_t) if lse_t is not None else out


def fwd_fp8(q8, k8, v8, descales, P: int, scale: float | None = None, out=None,
            stream=None, workspace="auto", lse=None, in_layout: str = "bshd"):
    """Attention over e4m3 inputs with per-tensor descales (x = x8 * d); layouts,
    lse and the return value as for fwd."""
    B, S, H, D, code = _check_inputs(q8, k8, v8, torch.float8_e4m3fn, P, in_layout)
    s = _stream(q8, stream)
    with _alloc_on(s, out, lse, workspace):  # the pool of the call's stream (see fwd)
        out = _out(q8, B, S, H, D, P, out)
        lse_t = _lse(q8, B, S, H, lse)
        ws, nbytes = _workspace(q8, B, S, H, D, workspace)
    scale = default_scale(D) if scale is None else float(scale)
    dq, dk, dv = (float(d) for d in descales)
    check(xs_attn_fwd_fp8_ex(q8, k8, v8, code, dq, dk, dv, out, lse_t, B, S, H, D, P, scale, ws,
                             nbytes, s.cuda_stream))
    return (out, lse_t) if lse_t is not None else out


def chunk(x: torch.Tensor, P: int) -> torch.Tensor:
    """[B][S][H][D] -> contiguous [P][B][S/P][H][D] (the chunk layout; a torch copy)."""
    B, S, H, D = x.shape
    assert S % P == 0
    raw = x.view(torch.uint8) if x.element_size() == 1 else x.view(torch.int16)
    y = raw.reshape(B, P, S // P, H, D).permute(1, 0, 2, 3, 4).contiguous()
    return y.view(x.dtype)


def unpack(out_packed: torch.Tensor, S: int) -> torch.Tensor:
    """View a [P][B][S/P][H][D] buffer as [B][S][H][D] (torch permute/reshape)."""
    P, B, T, H, D = out_packed.shape
    assert P * T == S
    return out_packed.permute(1, 0, 2, 3, 4).reshape(B, S, H, D)
