"""Exact-arithmetic brute force used to pin the oracle.

Nothing here calls the oracle or the GPU library.  Values are carried as exact
rationals (``fractions.Fraction``) and rounded to IEEE binary32 by an explicit
round-to-nearest-even routine written from the format's definition, so a slip
in the oracle's C code (a fused multiply-add, a wrong association, round-to-even
instead of half-away, a dropped or transposed term) shows up as a mismatch.
Only for tiny inputs: everything is pure Python.
"""
from __future__ import annotations

import math
from fractions import Fraction

import mpmath
import numpy as np

F32_MIN_EXP = -126          # exponent of the smallest normal binary32
F32_MANT = 23               # fraction bits of binary32
F32_MAX = Fraction((2 ** 24 - 1) * 2 ** (127 - 23))


def f32_round(v: Fraction) -> float:
    """Round an exact rational to binary32, nearest, ties to even."""
    if v == 0:
        return 0.0
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix e so that 2^e <= a < 2^(e+1) exactly
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, F32_MIN_EXP) - F32_MANT)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r > F32_MAX:
        return sign * math.inf
    return float(sign * r)


def fr(x) -> Fraction:
    return Fraction(float(x))


def f32(x) -> float:
    """Check that x is a binary32 value and return it as a Python float."""
    xf = float(np.float32(x))
    assert xf == float(x)
    return xf


def half_away(v: Fraction) -> int:
    """Round to the nearest integer, halves away from zero."""
    a = abs(v)
    n = math.floor(a + Fraction(1, 2))
    return n if v >= 0 else -n


def quantize_row(x) -> tuple[list[int], float]:
    """Per-token quantisation by brute force: s = RN(amax / 127), q = clamp(half_away(RN(x / s)))."""
    xs = [fr(v) for v in np.asarray(x, np.float32).tolist()]
    amax = max((abs(v) for v in xs), default=Fraction(0))
    s = f32_round(amax / 127)
    if s == 0:
        return [0] * len(xs), 0.0
    q = []
    for v in xs:
        r = half_away(Fraction(f32_round(v / fr(s))))
        q.append(max(-127, min(127, r)))
    return q, s


def epilogue(acc: int, ws, a_scale) -> float:
    """RN( RN(acc) * RN(ws * as) ) evaluated exactly then rounded."""
    c = f32_round(Fraction(acc))
    sc = f32_round(fr(ws) * fr(a_scale))
    return f32_round(fr(c) * fr(sc))


def gemv(W, ws, q, a_scale) -> list[float]:
    W = np.asarray(W, np.int64)
    qv = np.asarray(q, np.int64)
    acc = W @ qv
    return [epilogue(int(acc[n]), ws[n], a_scale) for n in range(W.shape[0])]


def stack_token(weights, scales, x, act: int = 0) -> tuple[list[float], list[list[float]]]:
    """One token through the stack, composed from the brute-force pieces.

    Returns the final activation and, per layer, the seven projection outputs
    concatenated (q, k, v, o, gate, up, down).  act 1: the down projection reads
    quantise(silu(gate) * up)."""
    h = [float(v) for v in np.asarray(x, np.float32)]
    per_layer = []
    for wl, sl in zip(weights, scales):
        a, sa = quantize_row(np.array(h, np.float32))
        outs = [gemv(wl[j], sl[j], a, sa) for j in range(6)]
        din = outs[5]
        if act:
            din = [f32_round(fr(silu(g)) * fr(u)) for g, u in zip(outs[4], outs[5])]
        b, sb = quantize_row(np.array(din, np.float32))
        down = gemv(wl[6], sl[6], b, sb)
        per_layer.append(sum(outs, []) + down)
        h = down
    return h, per_layer


def seq_sum_products(w, x) -> float:
    """acc = 0; for k ascending acc = RN(acc + RN(w_k * x_k))."""
    acc = 0.0
    for a, b in zip(w, x):
        p = f32_round(fr(a) * fr(b))
        acc = f32_round(fr(acc) + fr(p))
    return acc


def exp_cr(x: float) -> float:
    """Correctly rounded binary32 exp via 80-digit mpmath then exact rounding."""
    if x == -math.inf:
        return 0.0
    with mpmath.workdps(80):
        y = mpmath.exp(mpmath.mpf(x))
        # exact rational of the 80-digit value (its error is far below any
        # binary32 rounding boundary distance for these inputs)
        man, exp = mpmath.mpf(y).man_exp
    v = Fraction(int(man)) * (Fraction(2) ** int(exp))
    return f32_round(v)


def silu(g) -> float:
    """silu(g) = RN(g / RN(1 + exp_cr(-g))), each step rounded exactly."""
    g = f32(g)
    e = exp_cr(-g)
    if math.isinf(e):
        return -0.0 if g < 0 else 0.0            # g / inf, with g's sign
    d = f32_round(1 + fr(e))
    q = f32_round(fr(g) / fr(d))
    return -0.0 if (q == 0 and g < 0) else q


def softmax_topk(logits, k, renorm: bool = False) -> tuple[list[int], list[float], list[float]]:
    """Brute-force softmax + top-k: returns (ids, weights, all p); renorm:
    weights divided by their sum taken in rank order."""
    ls = [float(v) for v in np.asarray(logits, np.float32)]
    m = max(ls)
    z = [exp_cr(f32_round(fr(v) - fr(m))) for v in ls]
    S = 0.0
    for v in z:
        S = f32_round(fr(S) + fr(v))
    p = [f32_round(fr(v) / fr(S)) for v in z]
    order = sorted(range(len(p)), key=lambda e: (-p[e], e))[:k]
    w = [p[e] for e in order]
    if renorm:
        T = 0.0
        for v in w:
            T = f32_round(fr(T) + fr(v))
        w = [f32_round(fr(v) / fr(T)) for v in w]
    return order, w, p


def dot_seq(a, b) -> float:
    """acc = 0; for i ascending acc = RN(acc + RN(a_i * b_i))."""
    acc = 0.0
    for x, y in zip(a, b):
        acc = f32_round(fr(acc) + fr(f32_round(fr(x) * fr(y))))
    return acc


def attend(q, K, V, t, n_heads) -> list[float]:
    """Causal attention of one token over rows 0..t of K and V (each a list of
    H floats): per head scores RN(dot * c), c = RN(1 / RN(sqrt(d))), softmax
    with the correctly rounded exp and an ascending sum, then the ascending
    sum of RN(p_j * V[j][i])."""
    H = len(q)
    d = H // n_heads
    root = f32_round(_sqrt_fraction(d))
    c = f32_round(1 / fr(root))
    out = [0.0] * H
    for hd in range(n_heads):
        cols = range(hd * d, hd * d + d)
        s = [f32_round(fr(dot_seq([q[i] for i in cols], [K[j][i] for i in cols])) * fr(c))
             for j in range(t + 1)]
        m = max(s)
        z = [exp_cr(f32_round(fr(v) - fr(m))) for v in s]
        S = 0.0
        for v in z:
            S = f32_round(fr(S) + fr(v))
        p = [f32_round(fr(v) / fr(S)) for v in z]
        for i in cols:
            o = 0.0
            for j in range(t + 1):
                o = f32_round(fr(o) + fr(f32_round(fr(p[j]) * fr(V[j][i]))))
            out[i] = o
    return out


def _sqrt_fraction(d: int) -> Fraction:
    """sqrt(d) to 80 digits as an exact rational (its binary32 rounding is then
    the correctly rounded square root)."""
    with mpmath.workdps(80):
        man, exp = mpmath.mpf(mpmath.sqrt(d)).man_exp
    return Fraction(int(man)) * (Fraction(2) ** int(exp))


def stack_attn(weights, scales, x, n_heads, act: int = 0):
    """The stack with causal attention, layer by layer over all tokens, from the
    brute-force pieces.  Returns (y, kv, per-layer projection rows)."""
    P = len(x)
    hs = [[float(v) for v in np.asarray(row, np.float32)] for row in x]
    L = len(weights)
    kv = [[[None] * P, [None] * P] for _ in range(L)]
    proj = [[None] * P for _ in range(L)]
    for l, (wl, sl) in enumerate(zip(weights, scales)):
        outs = []
        for t in range(P):
            a, sa = quantize_row(np.array(hs[t], np.float32))
            o = {j: gemv(wl[j], sl[j], a, sa) for j in (0, 1, 2, 4, 5)}
            kv[l][0][t], kv[l][1][t] = o[1], o[2]
            outs.append(o)
        for t in range(P):
            o = outs[t]
            att = attend(o[0], kv[l][0], kv[l][1], t, n_heads)
            ao, so = quantize_row(np.array(att, np.float32))
            o[3] = gemv(wl[3], sl[3], ao, so)
            din = o[5]
            if act:
                din = [f32_round(fr(silu(g)) * fr(u)) for g, u in zip(o[4], o[5])]
            b, sb = quantize_row(np.array(din, np.float32))
            o[6] = gemv(wl[6], sl[6], b, sb)
            proj[l][t] = sum((o[j] for j in range(7)), [])
            hs[t] = o[6]
    return hs, kv, proj
