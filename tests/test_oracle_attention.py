"""Pins of the oracle's stack with causal attention and a KV cache (CPU only).

"Batched Prefill", What Stays Sequential: attention is sequential over
positions and runs per position inside each chunk.  "Single-pass prefill", The
fix: position i attends over the K/V history kv_[layer][0..i], already written
because every earlier position went first.  The arithmetic (a reading; the
pages give no formula) is fixed step by step: f32 dot products in ascending
index, scale c = RN(1 / RN(sqrt(d))), softmax with the correctly rounded exp and
an ascending sum, the probability-weighted sum of v rows in ascending position.
"""
import numpy as np
import pytest

import exact
import oracle
import prefill_inputs


def _small(L=2, H=16, F=32, P=5, seed=81):
    return prefill_inputs.stack(L=L, H=H, F=F, P=P, seed=seed)


@pytest.mark.parametrize("n_heads,act", [(2, 0), (1, 0), (4, 1)])
def test_stack_attn_exact_brute_force(n_heads, act):
    st = _small()
    y, kv, proj = oracle.stack_attn(st["weights"], st["scales"], st["x"], n_heads, return_proj=True,
                                    act=act)
    ye, kve, proje = exact.stack_attn(st["weights"], st["scales"], st["x"], n_heads, act=act)
    np.testing.assert_array_equal(y, np.array(ye, np.float32))
    for l in range(2):
        for t in range(5):
            np.testing.assert_array_equal(kv[l, 0, t], np.array(kve[l][0][t], np.float32))
            np.testing.assert_array_equal(kv[l, 1, t], np.array(kve[l][1][t], np.float32))
            np.testing.assert_array_equal(proj[l, t], np.array(proje[l][t], np.float32))


def test_first_position_attends_to_itself_only():
    """At position 0 the softmax has one term: p = 1, so the attention output is
    v_0 itself and o = gemv(W_o, quantise(v_0))."""
    st = _small(P=3)
    _, kv, proj = oracle.stack_attn(st["weights"], st["scales"], st["x"], 2, return_proj=True)
    H = 16
    for l in range(2):
        ao, so = oracle.quantize(kv[l, 1, 0][None, :])
        o = oracle.gemv(st["weights"][l][3], st["scales"][l][3], ao[0], so[0])
        np.testing.assert_array_equal(proj[l, 0, 3 * H:4 * H], o)


def test_equal_keys_average_the_values():
    """With every key of a head equal, all scores tie, p_j = RN(1 / n) for n
    positions, and the output is the ascending sum of RN(p * v_j) (checked in
    exact arithmetic on a hand-built cache)."""
    rng = np.random.default_rng(5)
    H, t = 8, 6
    q = rng.standard_normal(H).astype(np.float32)
    K = np.tile(rng.standard_normal(H).astype(np.float32), (t + 1, 1))
    V = rng.standard_normal((t + 1, H)).astype(np.float32)
    out = exact.attend(q.tolist(), K.tolist(), V.tolist(), t, 2)
    p = exact.f32_round(exact.Fraction(1, t + 1))
    for i in range(H):
        acc = 0.0
        for j in range(t + 1):
            acc = exact.f32_round(exact.fr(acc) + exact.fr(exact.f32_round(exact.fr(p) * exact.fr(V[j, i]))))
        assert out[i] == acc


def test_causality():
    """Changing tokens after position t changes nothing at positions <= t (the
    cache rows and projections of every layer)."""
    st = _small(P=6, seed=83)
    y0, kv0, p0 = oracle.stack_attn(st["weights"], st["scales"], st["x"], 2, return_proj=True)
    x2 = st["x"].copy()
    x2[4:] = -x2[4:] * 1.5
    y1, kv1, p1 = oracle.stack_attn(st["weights"], st["scales"], x2, 2, return_proj=True)
    np.testing.assert_array_equal(kv0[:, :, :4], kv1[:, :, :4])
    np.testing.assert_array_equal(p0[:, :4], p1[:, :4])
    assert not np.array_equal(p0[:, 4:], p1[:, 4:])


def test_attention_close_to_float64():
    """The f32 attention as defined (the exact brute force, to which the oracle
    is pinned above) stays within the rounding error of a float64 softmax
    attention: a dropped scale, a wrong maximum or a transposed head in the
    definition would be far off."""
    rng = np.random.default_rng(6)
    H, nh, t = 64, 4, 40
    q = rng.standard_normal(H).astype(np.float32)
    K = rng.standard_normal((t + 1, H)).astype(np.float32)
    V = rng.standard_normal((t + 1, H)).astype(np.float32)
    got = np.array(exact.attend(q.tolist(), K.tolist(), V.tolist(), t, nh))
    d = H // nh
    for hd in range(nh):
        c = slice(hd * d, hd * d + d)
        s = (K[:, c].astype(np.float64) @ q[c].astype(np.float64)) / np.sqrt(d)
        p = np.exp(s - s.max())
        p /= p.sum()
        ref = p @ V[:, c].astype(np.float64)
        scale = np.abs(p[:, None] * V[:, c]).sum(axis=0)
        assert np.all(np.abs(got[c] - ref) <= (3 * d + 3 * t + 10) * 2.0 ** -24 * scale + 1e-30)


def test_without_attention_feeding_down_y_is_the_plain_stack():
    """The attention feeds o, which feeds nothing further: y equals or_stack's."""
    st = _small(P=7, seed=84)
    y, _ = oracle.stack_attn(st["weights"], st["scales"], st["x"], 4)
    np.testing.assert_array_equal(y, oracle.stack(st["weights"], st["scales"], st["x"]))
