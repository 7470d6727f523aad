"""Pins of the oracle's quantiser and GEMV (CPU only).

The oracle is checked against hand-derived cases (tests/golden), closed forms
and exact-rational brute force (tests/exact.py), never against itself.
"""
import os

import numpy as np
import pytest

import exact
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_quantize():
    rows = []
    with open(os.path.join(GOLDEN, "quantize_halfaway.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            xs, qs, s = (p.strip() for p in line.split("|"))
            rows.append((np.array([float(v) for v in xs.split()], np.float32),
                         np.array([int(v) for v in qs.split()], np.int8), float(s)))
    return rows


@pytest.mark.parametrize("x,q_expected,s_expected", _golden_quantize())
def test_quantize_golden(x, q_expected, s_expected):
    q, s = oracle.quantize(x[None, :])
    assert float(s[0]) == s_expected
    np.testing.assert_array_equal(q[0], q_expected)


def test_quantize_brute_force_random():
    rng = np.random.default_rng(7)
    for K in (1, 3, 64, 257):
        x = rng.standard_normal((6, K)).astype(np.float32) * rng.uniform(1e-3, 1e3, (6, 1)).astype(np.float32)
        q, s = oracle.quantize(x)
        for t in range(6):
            qe, se = exact.quantize_row(x[t])
            assert float(s[t]) == se
            np.testing.assert_array_equal(q[t], np.array(qe, np.int8))


def test_quantize_exact_halves():
    # amax = 127 * 2^j gives an exact scale 2^j; x = (n + 1/2) * 2^j are exact
    # halves, which round away from zero (round-to-even would differ for even n).
    for j in (-6, 0, 3):
        s = 2.0 ** j
        n = np.arange(-126, 126)
        x = np.concatenate([[127 * s], (n + 0.5) * s]).astype(np.float32)
        q, sq = oracle.quantize(x[None, :])
        assert float(sq[0]) == s
        expect = np.concatenate([[127], np.where(n + 0.5 > 0, n + 1, n)])
        np.testing.assert_array_equal(q[0].astype(np.int64), expect)


def test_quantize_invariants():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((50, 300)).astype(np.float32)
    q, s = oracle.quantize(x)
    assert np.abs(q.astype(np.int32)).max() <= 127
    am = np.argmax(np.abs(x), axis=1)
    for t in range(50):
        assert int(q[t, am[t]]) == (127 if x[t, am[t]] > 0 else -127)
        # sign is kept wherever the code is nonzero
        nz = q[t] != 0
        assert np.all(np.sign(q[t][nz]) == np.sign(x[t][nz]))


def test_quantize_rejects_nonfinite():
    with pytest.raises(ValueError):
        oracle.quantize(np.array([[1.0, np.inf]], np.float32))
    with pytest.raises(ValueError):
        oracle.quantize(np.array([[np.nan, 1.0]], np.float32))


# --- GEMV / per-token linear -------------------------------------------------

def test_gemv_closed_form_ones():
    # W = 1, q = 1 -> acc = K; scales powers of two -> y = K * 2^-10 * 2^-3 exactly.
    N, K = 5, 192
    W = np.ones((N, K), np.int8)
    ws = np.full(N, 2.0 ** -10, np.float32)
    y = oracle.gemv(W, ws, np.ones(K, np.int8), 2.0 ** -3)
    np.testing.assert_array_equal(y, np.full(N, K * 2.0 ** -13, np.float32))


def test_gemv_closed_form_identity():
    # W = I picks q[n]; with unit scales y = q exactly.
    K = 128
    rng = np.random.default_rng(3)
    q = rng.integers(-127, 128, K).astype(np.int8)
    y = oracle.gemv(np.eye(K, dtype=np.int8), np.ones(K, np.float32), q, 1.0)
    np.testing.assert_array_equal(y, q.astype(np.float32))


def test_gemv_closed_form_extreme():
    # The largest accepted K with every product 127*127: acc = 16129 * 131072,
    # still inside int32 and exactly representable in binary32.
    K = 131072
    W = np.full((2, K), 127, np.int8)
    W[1] = -127
    y = oracle.gemv(W, np.ones(2, np.float32), np.full(K, 127, np.int8), 1.0)
    assert y[0] == 16129.0 * K and y[1] == -16129.0 * K
    with pytest.raises(ValueError):
        oracle.gemv(np.ones((1, K + 64), np.int8), np.ones(1, np.float32),
                    np.ones(K + 64, np.int8), 1.0)


def test_gemv_int_to_float_rounding():
    # acc = 2^24 + 1 is not a binary32 value: the conversion rounds to even, 2^24.
    # 2^24 + 1 = 1040 * 127*127 + 127*24 + 9*1.
    K = 1088
    W = np.zeros((1, K), np.int8)
    q = np.zeros(K, np.int8)
    W[0, :1040] = 127
    q[:1040] = 127
    W[0, 1040], q[1040] = 127, 24
    W[0, 1041], q[1041] = 9, 1
    y = oracle.gemv(W, np.ones(1, np.float32), q, 1.0)
    assert float(y[0]) == 2.0 ** 24


@pytest.mark.parametrize("N,K,M", [(1, 64, 1), (7, 64, 3), (70, 128, 5), (33, 256, 17), (16, 192, 40)])
def test_linear_brute_force(N, K, M):
    rng = np.random.default_rng(N * 1000 + K + M)
    W = rng.integers(-127, 128, (N, K)).astype(np.int8)
    ws = rng.uniform(0.001, 0.01, N).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    q, s = oracle.quantize(x)
    y = oracle.linear(W, ws, q, s)
    for t in range(M):
        np.testing.assert_array_equal(y[t], np.array(exact.gemv(W, ws, q[t], s[t]), np.float32))
        # the per-token entry point gives the same bytes as the per-row loop
        np.testing.assert_array_equal(oracle.gemv(W, ws, q[t], s[t]), y[t])


def test_linear_not_transposed():
    # A non-square W with one nonzero entry: y[t, n] must read W[n, k] * q[t, k].
    N, K, M = 3, 64, 2
    W = np.zeros((N, K), np.int8)
    W[2, 5] = 7
    q = np.zeros((M, K), np.int8)
    q[1, 5] = -3
    y = oracle.linear(W, np.ones(N, np.float32), q, np.ones(M, np.float32))
    expect = np.zeros((M, N), np.float32)
    expect[1, 2] = -21
    np.testing.assert_array_equal(y, expect)


def test_epilogue_association():
    # (float)acc * (ws * as) and ((float)acc * ws) * as round differently for some
    # inputs; find such inputs by exact arithmetic and check the oracle takes the
    # first association.
    rng = np.random.default_rng(5)
    K = 64
    found = 0
    for _ in range(400):
        c = int(rng.integers(1, 127))
        ws = np.float32(rng.uniform(0.001, 0.01))
        a = np.float32(rng.uniform(0.001, 0.05))
        acc = c * 127 * K
        right = exact.epilogue(acc, ws, a)
        left = exact.f32_round(exact.fr(exact.f32_round(exact.fr(float(acc)) * exact.fr(ws))) * exact.fr(a))
        if right == left:
            continue
        found += 1
        W = np.full((1, K), 127, np.int8)
        q = np.full(K, c, np.int8)
        assert float(oracle.gemv(W, np.array([ws]), q, a)[0]) == right
    assert found >= 20
