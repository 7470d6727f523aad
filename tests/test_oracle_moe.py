"""Pins of the oracle's router, exp, softmax/top-k and expert path (CPU only)."""
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


# --- router -------------------------------------------------------------------

def test_router_golden_order():
    for w, x, expect in _rows("router_order.txt"):
        w = np.array([float(v) for v in w.split()], np.float32)
        x = np.array([float(v) for v in x.split()], np.float32)
        assert float(oracle.router(w[None, :], x)[0, 0]) == float(expect)


def test_router_exact_on_small_integers():
    # Small-integer weights and inputs keep every partial sum an exact integer
    # below 2^24, so the f32 result equals the integer dot product.
    rng = np.random.default_rng(2)
    Wr = rng.integers(-50, 51, (9, 300)).astype(np.float32)
    x = rng.integers(-50, 51, (3, 300)).astype(np.float32)
    np.testing.assert_array_equal(oracle.router(Wr, x),
                                  (x.astype(np.int64) @ Wr.astype(np.int64).T).astype(np.float32))


def test_router_unit_vectors():
    # x = e_j selects column j of the router weight: l[e] = Wr[e, j].
    rng = np.random.default_rng(4)
    Wr = rng.standard_normal((6, 32)).astype(np.float32)
    for j in (0, 7, 31):
        x = np.zeros(32, np.float32)
        x[j] = 1
        np.testing.assert_array_equal(oracle.router(Wr, x)[0], Wr[:, j])


def test_router_brute_force_and_error_bound():
    rng = np.random.default_rng(6)
    E, H = 5, 96
    Wr = (rng.standard_normal((E, H)) / math.sqrt(H)).astype(np.float32)
    x = rng.standard_normal((2, H)).astype(np.float32)
    got = oracle.router(Wr, x)
    u = 2.0 ** -24
    gamma = H * u / (1 - H * u)
    for t in range(2):
        for e in range(E):
            assert float(got[t, e]) == exact.seq_sum_products(Wr[e], x[t])
            exact64 = float(np.dot(Wr[e].astype(np.float64), x[t].astype(np.float64)))
            bound = gamma * float(np.abs(Wr[e].astype(np.float64) * x[t]).sum())
            assert abs(float(got[t, e]) - exact64) <= bound


# --- exp ------------------------------------------------------------------------

def test_expf_special_values():
    assert float(oracle.expf_cr(np.float32(0.0))) == 1.0
    assert float(oracle.expf_cr(np.float32(-np.inf))) == 0.0
    assert float(oracle.expf_cr(np.float32(-200.0))) == 0.0
    # the smallest subnormal 2^-149 is exp(x) for x near -103.28
    assert float(oracle.expf_cr(np.float32(-103.28))) == 2.0 ** -149


def test_expf_matches_mpmath_sample():
    rng = np.random.default_rng(8)
    xs = np.concatenate([
        -rng.exponential(3.0, 3000).astype(np.float32),
        rng.uniform(-104, 0, 2000).astype(np.float32),
        -np.float32(2.0) ** -np.arange(1, 40, dtype=np.float32),
        np.float32([-87.33654, -87.33655, -88.0, -100.0, -103.97, -1e-8, -0.5, -0.6931472]),
    ]).astype(np.float32)
    got = oracle.expf_cr(xs)
    for x, g in zip(xs.tolist(), got.tolist()):
        assert g == exact.exp_cr(x), x


@pytest.mark.slow
@pytest.mark.parametrize("lo_x,hi_x", [(-0.0, -104.0), (0.0, 89.0)])
def test_expf_exhaustive(lo_x, hi_x):
    """Every binary32 x in [-104, 0] (the softmax's arguments) and in [0, 89]
    (the gated SiLU's exp(-g) for g < 0; exp overflows past 88.72): the
    oracle's exp equals RN(exp(x)).

    float64 exp has error below one double ulp, so its binary32 rounding is the
    correct rounding except when exp(x) lies within ~2^-52 (relative) of a
    binary32 midpoint; those few inputs are recomputed with mpmath at 80 digits.
    """
    top = int(np.array(hi_x, np.float32).view(np.uint32))
    start = int(np.array(lo_x, np.float32).view(np.uint32))  # +-0: bits 0 or 0x80000000
    step = 1 << 24
    flagged = 0
    for lo in range(start, top + 1, step):
        bits = np.arange(lo, min(lo + step, top + 1), dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        got = oracle.expf_cr(x)
        d = np.exp(x.astype(np.float64))
        r = d.astype(np.float32)
        # midpoint between r and its neighbour on d's side
        nb = np.where(d > r.astype(np.float64), np.nextafter(r, np.float32(np.inf)),
                      np.nextafter(r, np.float32(-np.inf)))
        mid = (r.astype(np.float64) + nb.astype(np.float64)) / 2
        close = np.abs(d - mid) <= np.abs(d) * 2.0 ** -50
        ok = (got == r) | close
        assert ok.all(), x[~ok][:5]
        for xi, gi in zip(x[close].tolist(), got[close].tolist()):
            flagged += 1
            assert gi == exact.exp_cr(xi), xi
    assert flagged < 200


# --- softmax / top-k -----------------------------------------------------------

def test_softmax_topk_golden():
    for name, E, k, rule, ids, ws in _rows("softmax_topk.txt"):
        E, k = int(E), int(k)
        if rule.startswith("all"):
            logits = np.full(E, float(rule.split()[1]), np.float32)
        elif rule.startswith("0 at"):
            logits = np.full(E, -200.0, np.float32)
            logits[int(rule.split()[2].rstrip(","))] = 0.0
        else:
            logits = np.array([float(v) for v in rule.split()], np.float32)
        got_ids, got_w = oracle.softmax_topk(logits, k)
        np.testing.assert_array_equal(got_ids[0], np.array([int(v) for v in ids.split()]))
        if ws != "*":
            np.testing.assert_array_equal(got_w[0], np.array([float(v) for v in ws.split()], np.float32))


def test_softmax_topk_brute_force():
    rng = np.random.default_rng(12)
    for E, k, scale in ((16, 4, 1.0), (64, 10, 3.0), (40, 10, 0.01)):
        logits = (rng.standard_normal((3, E)) * scale).astype(np.float32)
        # plant exact ties
        logits[1, 5] = logits[1, 9]
        ids, w = oracle.softmax_topk(logits, k)
        for t in range(3):
            eids, ew, p = exact.softmax_topk(logits[t], k)
            np.testing.assert_array_equal(ids[t], np.array(eids))
            np.testing.assert_array_equal(w[t], np.array(ew, np.float32))
            # probabilities close to the exact softmax (relative error bound)
            with_mp = [float(v) for v in np.exp(logits[t].astype(np.float64) - logits[t].max())]
            tot = sum(with_mp)
            for j, e in enumerate(eids):
                ref = with_mp[e] / tot
                assert abs(float(w[t, j]) - ref) <= (E + 4) * 2.0 ** -24 * ref + 1e-45


# --- experts -------------------------------------------------------------------

def _tiny_moe(seed=3, T=4):
    return prefill_inputs.moe(E=8, top_k=3, H=64, I=64, T=T, seed=seed)


def test_moe_brute_force_tiny():
    m = _tiny_moe()
    ids, w, out = oracle.moe(m, m["x"])
    for t in range(m["x"].shape[0]):
        xq, xs = exact.quantize_row(m["x"][t])
        logits = [exact.seq_sum_products(m["W_router"][e], m["x"][t]) for e in range(8)]
        eids, ew, _ = exact.softmax_topk(np.array(logits, np.float32), 3)
        np.testing.assert_array_equal(ids[t], eids)
        np.testing.assert_array_equal(w[t], np.array(ew, np.float32))
        acc = [0.0] * 64
        for e in sorted(eids):
            g = exact.gemv(m["W_gate"][e], m["s_gate"][e], xq, xs)
            u = exact.gemv(m["W_up"][e], m["s_up"][e], xq, xs)
            r = [exact.f32_round(exact.fr(a) * exact.fr(b)) for a, b in zip(g, u)]
            hq, hs = exact.quantize_row(np.array(r, np.float32))
            y = exact.gemv(m["W_down"][e], m["s_down"][e], hq, hs)
            np.testing.assert_array_equal(oracle.expert(m, e, np.array(xq, np.int8), xs),
                                          np.array(y, np.float32))
            we = ew[eids.index(e)]
            acc = [exact.f32_round(exact.fr(a) + exact.fr(exact.f32_round(exact.fr(we) * exact.fr(b))))
                   for a, b in zip(acc, y)]
        np.testing.assert_array_equal(out[t], np.array(acc, np.float32))


def test_moe_token_independence_and_threads():
    m = _tiny_moe(T=7, seed=9)
    ids, w, out = oracle.moe(m, m["x"], threads=1)
    ids2, w2, out2 = oracle.moe(m, m["x"][::-1], threads=3)
    np.testing.assert_array_equal(ids2[::-1], ids)
    np.testing.assert_array_equal(w2[::-1], w)
    np.testing.assert_array_equal(out2[::-1], out)
