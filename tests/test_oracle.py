"""Pins of the fp64 CPU oracle against things other than itself: hand-derived
closed forms (tests/golden), library routines (torch's bf16/fp8 decoders, torch
SDPA in float64), invariants the definition fixes, and special cases with exact
answers.  Each pin is chosen so a plausible mistake in the oracle fails it:

  dropped or doubled scale           -> golden closed forms, two-key logistic form
  wrong max / missing normalisation  -> constant-V, uniform-mean, golden
  Q/K swapped or transposed K        -> one-hot selection with a non-involutive permutation
  V row/column mix-up                -> golden (two value columns), one-hot, SDPA
  head/batch indexing                -> SDPA at B, H > 1; permutation tests per head
  bf16 / e4m3 decode                 -> all codes vs torch's decoders
  pack layout                        -> hand-derived golden layouts, numpy split/stack
  log-sum-exp: dropped max / log     -> golden values, score-shift invariance, torch.logsumexp
  chunk-layout inputs (index math)   -> numpy reshape/transpose of [B][S][H][D] inputs
  anything in the core formula       -> Python-loop brute force (S <= 64), rows sum to 1
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def _rand(shape, seed, scale=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64) * scale


def _unpacked(q, k, v, scale, descales=(1.0, 1.0, 1.0)):
    """Oracle O in [B][S][H][D] (P = 1 is the identity layout)."""
    out = oracle.attention_packed(q, k, v, 1, scale, descales)
    return out[0]


# ---------------------------------------------------------------- decoders
def test_bf16_decode_matches_torch_for_every_code():
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    ref = codes.to(torch.float64).numpy()
    got = np.array([oracle.decode_bf16(c) for c in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_decode_matches_torch_for_every_code():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = codes.to(torch.float64).numpy()
    got = np.array([oracle.decode_e4m3(c) for c in range(256)])
    nan = np.isnan(ref)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


# ---------------------------------------------------------------- golden closed forms
def _golden_value(x):
    if isinstance(x, str):
        return {"ln2": math.log(2.0), "ln3": math.log(3.0), "ln4": math.log(4.0),
                "ln6": math.log(6.0)}[x]
    return float(x)


def _golden_array(a, shape):
    flat = np.array([_golden_value(x) for x in np.asarray(a, dtype=object).ravel()])
    return flat.reshape(shape)


def test_golden_closed_forms():
    cases = json.load(open(os.path.join(GOLDEN, "attention_closed_form.json")))["cases"]
    for c in cases:
        shape = (c["B"], c["S"], c["H"], c["D"])
        q, k, v = (_f64(_golden_array(c[n], shape)) for n in "qkv")
        got = _unpacked(q, k, v, c["scale"])
        want = _golden_array(c["O"], shape)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-14, err_msg=c["name"])


def test_golden_log_sum_exp():
    cases = json.load(open(os.path.join(GOLDEN, "attention_closed_form.json")))["cases"]
    for c in cases:
        shape = (c["B"], c["S"], c["H"], c["D"])
        q, k, v = (_f64(_golden_array(c[n], shape)) for n in "qkv")
        _, lse = oracle.attention_packed(q, k, v, 1, c["scale"], with_lse=True)
        want = _golden_array(c["lse"], (c["B"], c["H"], c["S"]))
        np.testing.assert_allclose(lse, want, rtol=0, atol=1e-14, err_msg=c["name"])


def test_two_key_logistic_closed_form():
    # softmax over two keys is the logistic function of the score difference
    B, S, H, D = 2, 2, 3, 16
    q, k, v = _rand((B, 1, H, D), 1).expand(B, S, H, D).contiguous(), _rand((B, S, H, D), 2), _rand((B, S, H, D), 3)
    scale = 0.37
    got = _unpacked(q, k, v, scale)
    qn, kn, vn = q.numpy(), k.numpy(), v.numpy()
    for b in range(B):
        for h in range(H):
            delta = scale * (qn[b, 0, h] @ kn[b, 0, h] - qn[b, 0, h] @ kn[b, 1, h])
            a = 1.0 / (1.0 + math.exp(-delta))
            want = a * vn[b, 0, h] + (1.0 - a) * vn[b, 1, h]
            for s in range(S):
                np.testing.assert_allclose(got[b, s, h], want, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- invariants / special cases
def test_constant_v_gives_constant_output():
    B, S, H, D = 1, 97, 2, 8
    q, k = _rand((B, S, H, D), 4, 3.0), _rand((B, S, H, D), 5, 3.0)
    v = torch.full((B, S, H, D), -1.75, dtype=torch.float64)
    got = _unpacked(q, k, v, 0.9)
    np.testing.assert_allclose(got, -1.75, rtol=0, atol=1e-14)


def test_zero_keys_give_mean_of_values():
    B, S, H, D = 2, 64, 2, 8
    q = _rand((B, S, H, D), 6)
    k = torch.zeros((B, S, H, D), dtype=torch.float64)
    g = torch.Generator("cpu").manual_seed(7)
    v = torch.randint(-8, 9, (B, S, H, D), generator=g).to(torch.float64)
    got = _unpacked(q, k, v, 0.125)
    want = v.mean(dim=1, keepdim=True).expand(B, S, H, D).numpy()  # exact: small ints / 64
    np.testing.assert_array_equal(got, want)


def test_one_hot_selection_follows_query_to_key_map():
    # K_j = 16 e_j, Q_i = 16 e_pi(i), scale 1/8: the score gap is 32, so O_i = V_pi(i)
    # up to 63 e^-32 of the value range.  pi has no fixed points and is not an
    # involution, so swapping the roles of Q and K (pi^-1) or transposing fails.
    S = D = 64
    pi = np.array([(3 * i + 5) % S for i in range(S)])
    assert not np.array_equal(pi[pi], np.arange(S))
    k = torch.zeros((1, S, 1, D), dtype=torch.float64)
    q = torch.zeros((1, S, 1, D), dtype=torch.float64)
    for j in range(S):
        k[0, j, 0, j] = 16.0
    for i in range(S):
        q[0, i, 0, pi[i]] = 16.0
    v = _rand((1, S, 1, D), 8)
    got = _unpacked(q, k, v, 0.125)
    want = v.numpy()[0, pi, 0, :]
    np.testing.assert_allclose(got[0, :, 0, :], want, rtol=0, atol=1e-11)
    inv = np.argsort(pi)
    assert not np.allclose(got[0, :, 0, :], v.numpy()[0, inv, 0, :], atol=1e-3)


def test_single_key_returns_values():
    q, k, v = _rand((2, 1, 3, 16), 9), _rand((2, 1, 3, 16), 10), _rand((2, 1, 3, 16), 11)
    got = _unpacked(q, k, v, 5.0)
    np.testing.assert_array_equal(got, v.numpy())


def test_large_scale_tends_to_hard_argmax():
    B, S, H, D = 1, 40, 1, 8
    q, k, v = _rand((B, S, H, D), 12), _rand((B, S, H, D), 13), _rand((B, S, H, D), 14)
    got = _unpacked(q, k, v, 1e4)
    scores = q.numpy()[0, :, 0] @ k.numpy()[0, :, 0].T
    top2 = np.sort(scores, axis=1)[:, -2:]
    assert np.all(top2[:, 1] - top2[:, 0] > 5e-3)  # margins make exp(-1e4*gap) negligible
    want = v.numpy()[0, scores.argmax(axis=1), 0]
    np.testing.assert_allclose(got[0, :, 0], want, rtol=0, atol=1e-12)


def test_zero_scale_gives_uniform_mean():
    B, S, H, D = 1, 33, 2, 4
    q, k, v = _rand((B, S, H, D), 15), _rand((B, S, H, D), 16), _rand((B, S, H, D), 17)
    got = _unpacked(q, k, v, 0.0)
    want = v.mean(dim=1, keepdim=True).expand(B, S, H, D).numpy()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def test_key_value_row_permutation_leaves_output_unchanged():
    B, S, H, D = 2, 50, 2, 16
    q, k, v = _rand((B, S, H, D), 18), _rand((B, S, H, D), 19), _rand((B, S, H, D), 20)
    perm = torch.randperm(S, generator=torch.Generator("cpu").manual_seed(21))
    a = _unpacked(q, k, v, 0.25)
    b = _unpacked(q, k[:, perm], v[:, perm], 0.25)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_query_row_permutation_permutes_output_rows():
    B, S, H, D = 1, 50, 2, 16
    q, k, v = _rand((B, S, H, D), 22), _rand((B, S, H, D), 23), _rand((B, S, H, D), 24)
    perm = torch.randperm(S, generator=torch.Generator("cpu").manual_seed(25))
    a = _unpacked(q, k, v, 0.25)
    b = _unpacked(q[:, perm], k, v, 0.25)
    np.testing.assert_array_equal(a[:, perm.numpy()], b)


def _brute_force(q, k, v, scale):
    """softmax(scale q k^T) v written out with Python loops and math.exp."""
    B, S, H, D = q.shape
    q, k, v = q.tolist(), k.tolist(), v.tolist()
    out = [[[[0.0] * D for _ in range(H)] for _ in range(S)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(S):
                s = [scale * sum(q[b][i][h][d] * k[b][j][h][d] for d in range(D)) for j in range(S)]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                tot = sum(e)
                for d in range(D):
                    out[b][i][h][d] = sum(e[j] * v[b][j][h][d] for j in range(S)) / tot
    return np.array(out)


@pytest.mark.parametrize("S", [1, 5, 33, 64])
def test_brute_force_small_sequences(S):
    B, H, D = 2, 2, 16
    q, k, v = _rand((B, S, H, D), 40 + S, 1.5), _rand((B, S, H, D), 41 + S), _rand((B, S, H, D), 42 + S)
    np.testing.assert_allclose(_unpacked(q, k, v, 0.4), _brute_force(q, k, v, 0.4), rtol=0, atol=1e-13)


@pytest.mark.parametrize("S", [3, 64])
def test_softmax_rows_sum_to_one(S):
    # with V the identity (value row j = e_j) O is the weight matrix itself: each
    # row must be a probability vector equal to the brute-force softmax row
    B, H, D = 1, 2, 64
    q, k = _rand((B, S, H, D), 50 + S), _rand((B, S, H, D), 51 + S)
    v = torch.zeros((B, S, H, D), dtype=torch.float64)
    for j in range(S):
        v[:, j, :, j] = 1.0
    w = _unpacked(q, k, v, 0.3)
    np.testing.assert_allclose(w[..., :S].sum(-1), 1.0, rtol=0, atol=1e-14)
    assert (w[..., :S] > 0).all() and (w[..., S:] == 0).all()
    np.testing.assert_allclose(w, _brute_force(q, k, v, 0.3), rtol=0, atol=1e-14)


@pytest.mark.parametrize("B,S,H,D", [(1, 1, 1, 8), (2, 17, 3, 64), (1, 64, 2, 128), (2, 130, 1, 32)])
def test_matches_torch_sdpa_float64(B, S, H, D):
    q, k, v = _rand((B, S, H, D), 26), _rand((B, S, H, D), 27), _rand((B, S, H, D), 28)
    scale = 1.0 / math.sqrt(D)
    got = _unpacked(q, k, v, scale)
    # torch SDPA takes [B][H][S][D]
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), scale=scale).transpose(1, 2)
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- reduced-precision inputs
def test_bf16_inputs_equal_fp64_of_decoded_values():
    w = workloads.custom(2, 40, 2, 64, 4)
    inp = workloads.make_inputs(w, seed=3)
    a = oracle.attention_packed(inp["q"], inp["k"], inp["v"], 4, inp["scale"])
    b = oracle.attention_packed(inp["q"].double(), inp["k"].double(), inp["v"].double(), 4, inp["scale"])
    np.testing.assert_array_equal(a, b)


def test_e4m3_inputs_equal_fp64_of_dequantised_values():
    w = workloads.custom(1, 48, 2, 32, 2, dtype="fp8")
    inp = workloads.make_inputs(w, seed=4)
    dq = [t.to(torch.float64) * d for t, d in zip((inp["q"], inp["k"], inp["v"]), inp["descales"])]
    a = oracle.attention_packed(inp["q"], inp["k"], inp["v"], 2, inp["scale"], inp["descales"])
    b = oracle.attention_packed(*dq, 2, inp["scale"])
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------- relayout
def test_pack_golden_layouts():
    cases = json.load(open(os.path.join(GOLDEN, "pack_layout.json")))["cases"]
    for c in cases:
        B, S, H, D, P = c["B"], c["S"], c["H"], c["D"], c["P"]
        b, s, h, d = np.meshgrid(np.arange(B), np.arange(S), np.arange(H), np.arange(D), indexing="ij")
        o = eval(c["tag"], {}, {"b": b, "s": s, "h": h, "d": d}).astype(np.float64)
        got = oracle.pack(o, P).ravel()
        np.testing.assert_array_equal(got, np.asarray(c["out_packed"], dtype=np.float64), err_msg=c["name"])


@pytest.mark.parametrize("B", [1, 2, 3])
@pytest.mark.parametrize("P", [1, 2, 4, 8])
@pytest.mark.parametrize("H", [1, 3])
def test_pack_is_the_all_to_all_chunk_split(B, P, H):
    S, D = 8 * 3, 4
    o = np.arange(B * S * H * D, dtype=np.float64).reshape(B, S, H, D)  # index tags, exact
    got = oracle.pack(o, P)
    want = np.stack(np.split(o, P, axis=1))  # chunk p = rows p*T..p*T+T-1 of every batch
    np.testing.assert_array_equal(got, want)
    assert np.array_equal(np.sort(got.ravel()), o.ravel())  # a permutation
    for _ in range(20):
        idx = tuple(int(np.random.default_rng(B * 100 + P).integers(n)) for n in (B, S, H, D))
        assert got.ravel()[oracle.packed_offset(B, S, H, D, P, *idx)] == o[idx]


def test_packed_attention_equals_pack_of_unpacked():
    B, S, H, D, P = 2, 24, 3, 8, 4
    q, k, v = _rand((B, S, H, D), 29), _rand((B, S, H, D), 30), _rand((B, S, H, D), 31)
    o = _unpacked(q, k, v, 0.3)
    np.testing.assert_array_equal(oracle.attention_packed(q, k, v, P, 0.3), oracle.pack(o, P))


def test_rows_entry_matches_packed_entry():
    w = workloads.custom(2, 64, 3, 32, 4)
    inp = workloads.make_inputs(w, seed=5)
    full = oracle.attention_packed(inp["q"], inp["k"], inp["v"], 1, inp["scale"])[0]
    rows = workloads.sample_rows(w, 30)
    got = oracle.attention_rows(inp["q"], inp["k"], inp["v"], rows, inp["scale"])
    for r, (b, s, h) in enumerate(rows):
        np.testing.assert_array_equal(got[r], full[b, s, h])


def test_thread_count_does_not_change_results():
    w = workloads.custom(1, 70, 2, 16, 2)
    inp = workloads.make_inputs(w, seed=6)
    a = oracle.attention_packed(inp["q"], inp["k"], inp["v"], 2, inp["scale"], nthreads=1)
    b = oracle.attention_packed(inp["q"], inp["k"], inp["v"], 2, inp["scale"], nthreads=5)
    np.testing.assert_array_equal(a, b)


def test_rejects_s_not_multiple_of_p():
    q = _rand((1, 10, 1, 4), 32)
    with pytest.raises(ValueError):
        oracle.attention_packed(q, q, q, 3, 1.0)


# ---------------------------------------------------------------- log-sum-exp
def test_log_sum_exp_matches_torch_logsumexp_float64():
    B, S, H, D = 2, 37, 3, 16
    q, k, v = _rand((B, S, H, D), 40), _rand((B, S, H, D), 41), _rand((B, S, H, D), 42)
    scale = 0.61
    _, lse = oracle.attention_packed(q, k, v, 1, scale, with_lse=True)
    s = torch.matmul(q.permute(0, 2, 1, 3), k.permute(0, 2, 3, 1).contiguous()) * scale
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-13)


def test_log_sum_exp_zero_keys_is_log_of_key_count():
    B, S, H, D = 1, 53, 2, 8
    q, v = _rand((B, S, H, D), 43, 4.0), _rand((B, S, H, D), 44)
    k = torch.zeros((B, S, H, D), dtype=torch.float64)
    _, lse = oracle.attention_packed(q, k, v, 1, 0.8, with_lse=True)
    np.testing.assert_allclose(lse, math.log(S), rtol=0, atol=1e-14)


def test_log_sum_exp_of_one_key_is_its_score():
    q, k, v = _rand((2, 1, 2, 8), 45), _rand((2, 1, 2, 8), 46), _rand((2, 1, 2, 8), 47)
    _, lse = oracle.attention_packed(q, k, v, 1, 0.3, with_lse=True)
    want = 0.3 * (q.numpy() * k.numpy()).sum(-1)          # [B][1][H]
    np.testing.assert_allclose(lse, want.transpose(0, 2, 1), rtol=0, atol=1e-14)


def test_log_sum_exp_shifts_with_a_common_score_offset():
    # an extra dimension with q = 1, k = c / scale adds c to every score: the
    # softmax (and O) is unchanged and the log-sum-exp moves by exactly c
    B, S, H, D = 1, 40, 2, 8
    q, k, v = _rand((B, S, H, D), 48), _rand((B, S, H, D), 49), _rand((B, S, H, D), 50)
    scale, c = 0.5, 7.25
    q2 = torch.cat([q, torch.ones((B, S, H, 1), dtype=torch.float64)], dim=-1)
    k2 = torch.cat([k, torch.full((B, S, H, 1), c / scale, dtype=torch.float64)], dim=-1)
    v2 = torch.cat([v, torch.zeros((B, S, H, 1), dtype=torch.float64)], dim=-1)
    o1, l1 = oracle.attention_packed(q, k, v, 1, scale, with_lse=True)
    o2, l2 = oracle.attention_packed(q2, k2, v2, 1, scale, with_lse=True)
    np.testing.assert_allclose(l2, l1 + c, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o2[..., :D], o1, rtol=0, atol=1e-13)


def test_rows_entry_log_sum_exp_matches_packed_entry():
    B, S, H, D = 2, 19, 2, 8
    q, k, v = _rand((B, S, H, D), 51), _rand((B, S, H, D), 52), _rand((B, S, H, D), 53)
    _, lse = oracle.attention_packed(q, k, v, 1, 0.4, with_lse=True)
    rows = [(b, s, h) for b in range(B) for s in range(S) for h in range(H)]
    _, got = oracle.attention_rows(q, k, v, rows, 0.4, with_lse=True)
    want = np.array([lse[b, h, s] for b, s, h in rows])
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- chunk-layout inputs
def _chunked(x, P):
    """[B][S][H][D] -> [P][B][S/P][H][D] by numpy reshape/transpose (not oracle.pack)."""
    B, S, H, D = x.shape
    return torch.as_tensor(np.ascontiguousarray(
        np.asarray(x).reshape(B, P, S // P, H, D).transpose(1, 0, 2, 3, 4)))


@pytest.mark.parametrize("B,S,P", [(1, 12, 3), (2, 12, 2), (3, 16, 4), (2, 18, 6)])
def test_chunk_layout_inputs_give_the_same_attention(B, S, P):
    H, D = 2, 8
    q, k, v = _rand((B, S, H, D), 54), _rand((B, S, H, D), 55), _rand((B, S, H, D), 56)
    want, want_lse = oracle.attention_packed(q, k, v, P, 0.45, with_lse=True)
    got, got_lse = oracle.attention_packed(_chunked(q, P), _chunked(k, P), _chunked(v, P), P, 0.45,
                                           in_P=P, with_lse=True)
    assert np.array_equal(got, want) and np.array_equal(got_lse, want_lse)
    rows = [(b, s, h) for b in range(B) for s in range(S) for h in range(H)][::3]
    r_want = oracle.attention_rows(q, k, v, rows, 0.45)
    r_got = oracle.attention_rows(_chunked(q, P), _chunked(k, P), _chunked(v, P), rows, 0.45, in_P=P)
    assert np.array_equal(r_got, r_want)


def test_chunk_layout_hand_indexed_case():
    # B = 2, S = 4, P = 2 (T = 2), H = D = 1: chunk p holds rows 2p, 2p+1 of
    # batch 0 then of batch 1.  Keys are zero, so each O row is the mean of its
    # batch's values: batch 0 values (1, 2, 3, 4) -> 2.5; batch 1 (10, 20, 30, 40) -> 25.
    v_chunks = _f64([[[[[1.0]], [[2.0]]], [[[10.0]], [[20.0]]]],
                     [[[[3.0]], [[4.0]]], [[[30.0]], [[40.0]]]]])   # [P][B][T][H][D]
    q = torch.ones_like(v_chunks)
    k = torch.zeros_like(v_chunks)
    out = oracle.attention_packed(q, k, v_chunks, 1, 1.0, in_P=2)    # [1][B][S][H][D]
    np.testing.assert_allclose(out[0, 0, :, 0, 0], 2.5, rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[0, 1, :, 0, 0], 25.0, rtol=0, atol=1e-15)
