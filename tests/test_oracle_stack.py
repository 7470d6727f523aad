"""Pins of the oracle's projection stack (CPU only).

A tiny stack is recomputed token by token with the exact-rational pieces of
tests/exact.py, composed here from the dataflow the oracle documents (all six
K = H projections read quantise(h); down reads quantise(up); next h = down).
Structural properties that hold for any correct implementation follow.
"""
import numpy as np
import pytest

import exact
import oracle
import prefill_inputs


def _tiny(L=2, H=64, F=128, P=5, seed=77):
    return prefill_inputs.stack(L, H, F, P, seed)


def test_stack_brute_force_tiny():
    st = _tiny()
    y, proj = oracle.stack(st["weights"], st["scales"], st["x"], return_proj=True)
    for t in range(st["x"].shape[0]):
        h, per_layer = exact.stack_token(st["weights"], st["scales"], st["x"][t])
        np.testing.assert_array_equal(y[t], np.array(h, np.float32))
        for l, outs in enumerate(per_layer):
            np.testing.assert_array_equal(proj[l, t], np.array(outs, np.float32))


def test_stack_single_layer_is_composition():
    st = _tiny(L=1, H=128, F=192, P=4, seed=5)
    (wq, wk, wv, wo, wg, wu, wd), (sq, sk, sv, so, sg, su, sd) = st["weights"][0], st["scales"][0]
    a, sa = oracle.quantize(st["x"])
    up = oracle.linear(wu, su, a, sa)
    b, sb = oracle.quantize(up)
    down = oracle.linear(wd, sd, b, sb)
    y, proj = oracle.stack(st["weights"], st["scales"], st["x"], return_proj=True)
    np.testing.assert_array_equal(y, down)
    H, F = 128, 192
    np.testing.assert_array_equal(proj[0, :, 0:H], oracle.linear(wq, sq, a, sa))
    np.testing.assert_array_equal(proj[0, :, 3 * H:4 * H], oracle.linear(wo, so, a, sa))
    np.testing.assert_array_equal(proj[0, :, 4 * H:4 * H + F], oracle.linear(wg, sg, a, sa))
    np.testing.assert_array_equal(proj[0, :, 4 * H + F:4 * H + 2 * F], up)
    np.testing.assert_array_equal(proj[0, :, 4 * H + 2 * F:], down)


def test_stack_token_independence():
    # Tokens do not interact: permuting the prompt permutes the output rows, and
    # any split of the prompt gives the same rows (the oracle itself has no chunk).
    st = _tiny(P=9)
    y = oracle.stack(st["weights"], st["scales"], st["x"])
    perm = np.random.default_rng(1).permutation(9)
    np.testing.assert_array_equal(oracle.stack(st["weights"], st["scales"], st["x"][perm]), y[perm])
    parts = [oracle.stack(st["weights"], st["scales"], st["x"][a:b]) for a, b in ((0, 4), (4, 5), (5, 9))]
    np.testing.assert_array_equal(np.concatenate(parts), y)


def test_stack_unconsumed_projections_do_not_feed_forward():
    # q, k, v, o and gate are computed but do not reach the next layer; up and
    # down do.  Changing q's weights moves q's output only.
    st = _tiny()
    y0, p0 = oracle.stack(st["weights"], st["scales"], st["x"], return_proj=True)
    w = [list(l) for l in st["weights"]]
    w[0][0] = (-w[0][0].astype(np.int16)).clip(-127, 127).astype(np.int8)
    y1, p1 = oracle.stack(w, st["scales"], st["x"], return_proj=True)
    np.testing.assert_array_equal(y0, y1)
    assert not np.array_equal(p0[0, :, :64], p1[0, :, :64])
    w = [list(l) for l in st["weights"]]
    w[0][5] = (-w[0][5].astype(np.int16)).clip(-127, 127).astype(np.int8)
    y2 = oracle.stack(w, st["scales"], st["x"])
    assert not np.array_equal(y0, y2)


def test_stack_threads_do_not_change_bytes():
    st = _tiny(P=11)
    a = oracle.stack(st["weights"], st["scales"], st["x"], threads=1)
    b = oracle.stack(st["weights"], st["scales"], st["x"], threads=4)
    np.testing.assert_array_equal(a, b)


def test_stack_scales_keep_activations_bounded():
    # The stack-scale recipe keeps a 16-layer chain finite and of order one.
    st = prefill_inputs.stack(16, 256, 512, 3, 9)
    y = oracle.stack(st["weights"], st["scales"], st["x"])
    assert np.all(np.isfinite(y))
    assert 0.05 < float(np.sqrt(np.mean(y.astype(np.float64) ** 2))) < 20.0
