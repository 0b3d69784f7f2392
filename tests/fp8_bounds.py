"""Per-element error bounds of the fp8 path, derived from its two encodings of P
(shared by the parity tests and the seeded sweep).  Test infrastructure: it calls
the oracle, never the HIP path."""
import numpy as np
import torch

from oracle import oracle

# Per-element rounding bounds of the fp8 path, from its two encodings of P.
#  * With the log-sum-exp output, P is 2^(s c - m) rounded to e4m3 (unit roundoff
#    u = 2^-4 for normal values, absolute 2^-10 below 2^-6) and O is normalised by
#    the fp32 sum of the unrounded values: |O' - O| <= u / (1 - u) (sum_j w_j |v_j|
#    + |O|) + 2^-8 |O| (bf16 output) + 2^-9 max|v| (weights in the subnormal range).
#  * Without it, P is the e4m3 code round(8 (y + 7)) of y = s c - m + 4.75: the
#    value 2^e (1 + f) (e + f = y) is 2^y times a factor in [1, 1.0614], and the
#    rounding of the code moves it by at most half a mantissa step (1/16 of it),
#    so p'_j = K 2^(y_j) g_j with g_j in [a, b] = [15/16, 1.0614 * 17/16], and O is
#    normalised by the sum of the same p'_j: O' - O = sum_j w_j (g_j - g) v_j / g
#    with g = sum_j w_j g_j in [a, b], so |O' - O| <= (b - a)/a sum_j w_j |v_j|.
#    Keys more than 10.75 octaves below the row's largest score are subnormal or
#    zero codes: their error is at most twice their share, 2 sum_(small j) w_j |v_j|.
#    Plus 2^-8 |O| for the bf16 output.
CODE_SPREAD = (1.0614 * 17 / 16 - 15 / 16) / (15 / 16)


def fp8_bounds(inp, P, scale):
    """(bound with the log-sum-exp output, bound without it), both [P][B][T][H][D]."""
    dq, dk, dv = inp["descales"]
    qf = inp["q"].to(torch.float64) * dq
    kf = inp["k"].to(torch.float64) * dk
    vabs = inp["v"].to(torch.float64).abs() * dv
    ref = oracle.attention_packed(inp["q"], inp["k"], inp["v"], P, scale, inp["descales"])
    ref_abs = oracle.attention_packed(qf, kf, vabs, P, scale)  # sum_j w_j |v_j|
    # keys below 2^-10.75 of the row's largest weight (softmax weights in fp64)
    s = torch.matmul(qf.permute(0, 2, 1, 3), kf.permute(0, 2, 3, 1).contiguous()) * scale
    w = torch.exp(s - s.amax(-1, keepdim=True))  # [B][H][S][S]
    small = (w < 2.0 ** -10.75).to(torch.float64)
    sub = torch.matmul(w * small, vabs.permute(0, 2, 1, 3).contiguous()) / w.sum(-1, keepdim=True)
    sub = oracle.pack(sub.permute(0, 2, 1, 3).numpy(), P)
    u = 2.0 ** -4
    with_lse = u / (1 - u) * (ref_abs + np.abs(ref)) + 2.0 ** -8 * np.abs(ref) \
        + 2.0 ** -9 * float(vabs.max())
    without = CODE_SPREAD * ref_abs + 2.0 ** -8 * np.abs(ref) + 2.0 * sub
    return with_lse, without
