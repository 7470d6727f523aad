"""Pins of the oracle's variants (CPU only): the gated SiLU between the gate/up
and down products (stack and experts) and top-k weights renormalised over the
chosen experts.

The pages name gate, up and down projections and a softmax top-10 but give
neither formula; the variants are the gated-SiLU feed-forward and the
renormalised routing weights of the model families the pages run.  Their
arithmetic is fixed step by step (each step one binary32 rounding), so an exact
brute force written from the same definitions pins them: silu(g) =
RN(g / RN(1 + exp_cr(-g))), r = RN(silu(g) * u); T = the chosen p summed in rank
order, w = RN(p / T).
"""
import math
import os

import numpy as np
import pytest

import exact
import oracle
import prefill_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [p.strip() for p in line.split("|")]


# --- silu -------------------------------------------------------------------------------

def test_silu_special_values():
    s = oracle.silu(np.float32([0.0, -0.0, 17.0, 30.0, 1e30, -89.0, -1e30, -200.0]))
    # silu(0) = 0 / 2 with the sign of the zero
    assert s[0] == 0.0 and not np.signbit(s[0])
    assert s[1] == 0.0 and np.signbit(s[1])
    # exp(-g) < 2^-25 for g >= 17.33: 1 + exp(-g) rounds to 1 and silu(g) = g exactly
    assert s[2] == np.float32(17.0) and s[3] == np.float32(30.0) and s[4] == np.float32(1e30)
    # exp(-g) overflows to +inf for g < -88.73: silu(g) = g / inf = -0
    assert np.all(s[5:] == 0.0) and np.all(np.signbit(s[5:]))


def test_silu_exact_brute_force():
    rng = np.random.default_rng(41)
    g = np.concatenate([rng.standard_normal(300), rng.uniform(-100, 100, 200),
                        rng.standard_normal(100) * 1e-3, [-88.7, -88.72, -88.73, -88.75, 16.5, 17.3,
                                                         0.6931472, -0.6931472, 1.0, -1.0]]).astype(np.float32)
    got = oracle.silu(g)
    for gi, si in zip(g.tolist(), got.tolist()):
        want = exact.silu(gi)
        assert si == want and math.copysign(1, si) == math.copysign(1, want), gi


def test_silu_close_to_textbook():
    """silu(g) = g * sigmoid(g): within 3 units in the last place of the float64
    value wherever that is a normal binary32 number (a sign or argument slip in
    the exponent would be far off)."""
    g = np.linspace(-80, 80, 20001).astype(np.float32)
    got = oracle.silu(g).astype(np.float64)
    ref = g.astype(np.float64) / (1.0 + np.exp(-g.astype(np.float64)))
    ok = np.abs(ref) > 1e-37
    ulp = np.spacing(np.abs(ref[ok]).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got[ok] - ref[ok]) <= 3 * ulp)


# --- the stack with the gated SiLU ------------------------------------------------------

def test_stack_swiglu_exact_brute_force():
    st = prefill_inputs.stack(L=2, H=64, F=128, P=3, seed=61)
    y, proj = oracle.stack(st["weights"], st["scales"], st["x"], return_proj=True, act=oracle.ACT_SWIGLU)
    for t in range(3):
        h, per_layer = exact.stack_token(st["weights"], st["scales"], st["x"][t], act=1)
        np.testing.assert_array_equal(y[t], np.array(h, np.float32))
        for l in range(2):
            np.testing.assert_array_equal(proj[l, t], np.array(per_layer[l], np.float32))


def test_stack_swiglu_differs_and_first_products_agree():
    """The variant changes only what feeds down: q..up of layer 0 are the plain
    stack's, down differs."""
    st = prefill_inputs.stack(L=2, H=64, F=128, P=4, seed=62)
    _, p0 = oracle.stack(st["weights"], st["scales"], st["x"], return_proj=True)
    _, p1 = oracle.stack(st["weights"], st["scales"], st["x"], return_proj=True, act=oracle.ACT_SWIGLU)
    H, F = 64, 128
    np.testing.assert_array_equal(p0[0, :, :4 * H + 2 * F], p1[0, :, :4 * H + 2 * F])
    assert not np.array_equal(p0[0, :, 4 * H + 2 * F:], p1[0, :, 4 * H + 2 * F:])


# --- renormalised top-k -------------------------------------------------------------------

def test_softmax_topk_renorm_golden():
    for name, E, k, rule, ids, ws in _rows("softmax_topk_renorm.txt"):
        E, k = int(E), int(k)
        if rule.startswith("all"):
            logits = np.full(E, float(rule.split()[1]), np.float32)
        else:
            logits = np.full(E, -200.0, np.float32)
            logits[int(rule.split()[2].rstrip(","))] = 0.0
        got_ids, got_w = oracle.softmax_topk(logits, k, renorm=True)
        np.testing.assert_array_equal(got_ids[0], np.array([int(v) for v in ids.split()]))
        np.testing.assert_array_equal(got_w[0], np.array([float(v) for v in ws.split()], np.float32))


def test_softmax_topk_renorm_brute_force_and_sum():
    rng = np.random.default_rng(13)
    for E, k, scale in ((16, 4, 1.0), (64, 10, 3.0), (512, 10, 1.0), (40, 10, 0.01)):
        logits = (rng.standard_normal((3, E)) * scale).astype(np.float32)
        logits[1, 5] = logits[1, 9]                     # a tie
        ids, w = oracle.softmax_topk(logits, k, renorm=True)
        ids0, w0 = oracle.softmax_topk(logits, k)
        np.testing.assert_array_equal(ids, ids0)        # the same experts, the same order
        for t in range(3):
            eids, ew, _ = exact.softmax_topk(logits[t], k, renorm=True)
            np.testing.assert_array_equal(ids[t], np.array(eids))
            np.testing.assert_array_equal(w[t], np.array(ew, np.float32))
            assert abs(float(np.sum(w[t].astype(np.float64))) - 1.0) <= 2 * k * 2.0 ** -24


# --- experts with the variants ------------------------------------------------------------

@pytest.mark.parametrize("act,renorm", [(1, 0), (0, 1), (1, 1)])
def test_moe_variants_brute_force_tiny(act, renorm):
    m = prefill_inputs.moe(E=8, top_k=3, H=64, I=64, T=3, seed=7)
    m["activation"], m["renormalize"] = act, renorm
    ids, w, out = oracle.moe(m, m["x"])
    for t in range(3):
        xq, xs = exact.quantize_row(m["x"][t])
        logits = [exact.seq_sum_products(m["W_router"][e], m["x"][t]) for e in range(8)]
        eids, ew, _ = exact.softmax_topk(np.array(logits, np.float32), 3, renorm=bool(renorm))
        np.testing.assert_array_equal(ids[t], eids)
        np.testing.assert_array_equal(w[t], np.array(ew, np.float32))
        acc = [0.0] * 64
        for e in sorted(eids):
            g = exact.gemv(m["W_gate"][e], m["s_gate"][e], xq, xs)
            u = exact.gemv(m["W_up"][e], m["s_up"][e], xq, xs)
            if act:
                r = [exact.f32_round(exact.fr(exact.silu(a)) * exact.fr(b)) for a, b in zip(g, u)]
            else:
                r = [exact.f32_round(exact.fr(a) * exact.fr(b)) for a, b in zip(g, u)]
            hq, hs = exact.quantize_row(np.array(r, np.float32))
            y = exact.gemv(m["W_down"][e], m["s_down"][e], hq, hs)
            np.testing.assert_array_equal(oracle.expert(m, e, np.array(xq, np.int8), xs),
                                          np.array(y, np.float32))
            we = ew[eids.index(e)]
            acc = [exact.f32_round(exact.fr(a) + exact.fr(exact.f32_round(exact.fr(we) * exact.fr(b))))
                   for a, b in zip(acc, y)]
        np.testing.assert_array_equal(out[t], np.array(acc, np.float32))
