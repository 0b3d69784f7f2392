"""ctypes wrapper around the fp64 CPU oracle (``xs_oracle.c``).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import this module.  It
imports nothing from the HIP library's package and the HIP library imports
nothing from here.

The oracle computes, in fp64 from the exact decoded input values, the plain
definition of attention, softmax(scale * Q K^T) V with a two-pass (exact max,
then exp/sum) softmax, and writes the result into the destination-ordered
buffer [P][B][S/P][H][D] an all-to-all over P sequence slices delivers (X-Stage
paper: catalyzex.com abstract; gist.science explainer, "Zentrale Beitraege",
"FlashAttention-A2A (Piggybacking)").  It also returns the rows' log-sum-exp
(natural log) on request, and reads inputs either as [B][S][H][D] or in the
same chunk layout [in_P][B][S/in_P][H][D] (what the pre-attention All-to-All
delivers).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "xs_oracle.c")
_LIB = os.path.join(_HERE, "libxs_oracle.so")

F64, BF16, E4M3 = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O3, no -ffast-math) into oracle/libxs_oracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O3", "-march=native", "-std=c11", "-Wall", "-shared", "-fPIC",
               "-pthread", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, dbl, vp, ci = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        lib.xs_oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.xs_oracle_decode_bf16.restype = dbl
        lib.xs_oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
        lib.xs_oracle_decode_e4m3.restype = dbl
        lib.xs_oracle_packed_offset.argtypes = [i64] * 9
        lib.xs_oracle_packed_offset.restype = i64
        lib.xs_oracle_pack.argtypes = [vp, i64, i64, i64, i64, i64, vp]
        lib.xs_oracle_pack.restype = ci
        lib.xs_oracle_attention_rows.argtypes = [ci, vp, vp, vp, dbl, dbl, dbl, i64, i64, i64, i64,
                                                 dbl, vp, i64, vp, ci]
        lib.xs_oracle_attention_rows.restype = ci
        lib.xs_oracle_attention_packed.argtypes = [ci, vp, vp, vp, dbl, dbl, dbl, i64, i64, i64,
                                                   i64, i64, dbl, vp, ci]
        lib.xs_oracle_attention_packed.restype = ci
        lib.xs_oracle_attention_rows_ex.argtypes = [ci, vp, vp, vp, dbl, dbl, dbl, i64, i64, i64,
                                                    i64, i64, dbl, vp, i64, vp, vp, ci]
        lib.xs_oracle_attention_rows_ex.restype = ci
        lib.xs_oracle_attention_packed_ex.argtypes = [ci, vp, vp, vp, dbl, dbl, dbl, i64, i64, i64,
                                                      i64, i64, i64, dbl, vp, vp, ci]
        lib.xs_oracle_attention_packed_ex.restype = ci
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _as_input(x):
    """Return (dtype code, contiguous CPU tensor kept alive) for q/k/v."""
    if not isinstance(x, torch.Tensor):
        x = torch.as_tensor(np.asarray(x, dtype=np.float64))
    x = x.detach().to("cpu").contiguous()
    if x.dtype == torch.bfloat16:
        return BF16, x
    if x.dtype == torch.float8_e4m3fn:
        return E4M3, x
    if x.dtype == torch.float64:
        return F64, x
    raise TypeError(f"oracle takes float64, bfloat16 or float8_e4m3fn inputs, got {x.dtype}")


def _problem(q, k, v, in_P: int = 0):
    """(dtype code, q, k, v, (B, S, H, D)) for [B][S][H][D] inputs (in_P = 0) or
    inputs in the chunk layout [in_P][B][S/in_P][H][D]."""
    (cq, q), (ck, k), (cv, v) = _as_input(q), _as_input(k), _as_input(v)
    if not (cq == ck == cv):
        raise TypeError("q, k, v must share one dtype")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one shape")
    if in_P:
        if q.dim() != 5 or q.shape[0] != in_P:
            raise ValueError("chunk-layout inputs must be [in_P][B][S/in_P][H][D]")
        _, B, T, H, D = q.shape
        shape = (B, in_P * T, H, D)
    else:
        if q.dim() != 4:
            raise ValueError("q, k, v must all be [B][S][H][D]")
        shape = tuple(q.shape)
    return cq, q, k, v, shape


def attention_packed(q, k, v, P: int, scale: float, descales=(1.0, 1.0, 1.0),
                     nthreads: int | None = None, in_P: int = 0, with_lse: bool = False):
    """Full oracle: fp64 out_packed of shape [P][B][S/P][H][D] (and, with
    with_lse, the fp64 log-sum-exp [B][H][S])."""
    code, q, k, v, (B, S, H, D) = _problem(q, k, v, in_P)
    if P < 1 or S % P:
        raise ValueError("S must be a multiple of P")
    out = np.empty((P, B, S // P, H, D), dtype=np.float64)
    lse = np.empty((B, H, S), dtype=np.float64) if with_lse else None
    rc = _load().xs_oracle_attention_packed_ex(
        code, q.data_ptr(), k.data_ptr(), v.data_ptr(), *map(float, descales), in_P, B, S, H, D,
        P, float(scale), out.ctypes.data, lse.ctypes.data if with_lse else None,
        nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle failed with status {rc}")
    return (out, lse) if with_lse else out


def attention_rows(q, k, v, rows, scale: float, descales=(1.0, 1.0, 1.0),
                   nthreads: int | None = None, in_P: int = 0, with_lse: bool = False):
    """Oracle rows O[b, s, h, :] for an (n, 3) array of (b, s, h); returns (n, D)
    fp64 (and, with with_lse, the rows' log-sum-exp, shape (n,))."""
    code, q, k, v, (B, S, H, D) = _problem(q, k, v, in_P)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    out = np.empty((rows.shape[0], D), dtype=np.float64)
    lse = np.empty(rows.shape[0], dtype=np.float64) if with_lse else None
    rc = _load().xs_oracle_attention_rows_ex(
        code, q.data_ptr(), k.data_ptr(), v.data_ptr(), *map(float, descales), in_P, B, S, H, D,
        float(scale), rows.ctypes.data, rows.shape[0], out.ctypes.data,
        lse.ctypes.data if with_lse else None, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle failed with status {rc}")
    return (out, lse) if with_lse else out


def pack(o, P: int) -> np.ndarray:
    """Relayout an fp64 [B][S][H][D] array into [P][B][S/P][H][D]."""
    o = np.ascontiguousarray(np.asarray(o, dtype=np.float64))
    B, S, H, D = o.shape
    if P < 1 or S % P:
        raise ValueError("S must be a multiple of P")
    out = np.empty((P, B, S // P, H, D), dtype=np.float64)
    rc = _load().xs_oracle_pack(o.ctypes.data, B, S, H, D, P, out.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle pack failed with status {rc}")
    return out


def packed_offset(B, S, H, D, P, b, s, h, d) -> int:
    return int(_load().xs_oracle_packed_offset(B, S, H, D, P, b, s, h, d))


def decode_bf16(bits: int) -> float:
    return float(_load().xs_oracle_decode_bf16(bits))


def decode_e4m3(code: int) -> float:
    return float(_load().xs_oracle_decode_e4m3(code))
