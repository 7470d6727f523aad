"""GPU parity of pf_moe_chunk against the per-token oracle (bit-exact ids,
weights and outputs)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import prefill_inputs
import int8_weight_gemm_amd as pf

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def to_moe(m):
    return pf.Moe(m["n_experts"], m["top_k"], *[dev(m[n]) for n in (
        "W_router", "W_gate", "W_up", "W_down", "s_gate", "s_up", "s_down")])


def check(m, T=None):
    x = m["x"] if T is None else m["x"][:T]
    moe = to_moe(m)
    ws = pf.workspace(moe.workspace_bytes(x.shape[0]))
    ids, w, out = moe.chunk(dev(x), ws)
    ids_o, w_o, out_o = oracle.moe(m, x)
    np.testing.assert_array_equal(host(ids), ids_o)
    np.testing.assert_array_equal(host(w), w_o)
    np.testing.assert_array_equal(host(out), out_o)
    return host(out)


@pytest.mark.parametrize("E,k,H,I,T", [(8, 3, 64, 64, 5), (16, 4, 128, 192, 37), (64, 10, 256, 128, 100)])
def test_small_moe_matches_oracle(E, k, H, I, T):
    check(prefill_inputs.moe(E, k, H, I, T, seed=E + T))


# Shapes for the streaming expert kernel (K of 512, 1024 or 2048 in both
# products): expert groups over 32 tokens (150 tokens, top-2 of 8), a down
# projection whose 576 output rows end inside a 256-row band (its gate/up,
# K = 576, take the piecewise kernel), and K = 2048 in both products.
@pytest.mark.parametrize("E,k,H,I,T", [(16, 4, 512, 1024, 70), (8, 2, 1024, 512, 150),
                                       (8, 2, 576, 512, 40), (4, 1, 2048, 2048, 33)])
def test_streaming_expert_shapes_match_oracle(E, k, H, I, T):
    print(f"moe E={E} k={k} H={H} I={I} T={T}", file=sys.stderr, flush=True)
    check(prefill_inputs.moe(E, k, H, I, T, seed=100 + E + T))


def test_moe_many_pairs_grouping_from_memory():
    # 16000 (token, expert) pairs: the ids do not fit in LDS beside the bitmap,
    # so the grouping reads them from memory
    check(prefill_inputs.moe(16, 8, 64, 64, 2000, seed=9))


def test_moe_concentrated_routing():
    # A router with one dominant expert sends every token to the same experts:
    # groups larger than 32 tokens take the multi-group path.
    m = prefill_inputs.moe(32, 4, 128, 128, 90, seed=5)
    m["x"] = (m["x"] + np.float32(1.0)).astype(np.float32)
    m["W_router"][7] += np.float32(3.0)
    m["W_router"][3] += np.float32(2.5)
    check(m)


# The limits pf_moe_chunk takes: 1024 experts with top-32 over 2048 tokens
# (65536 pairs, the most a call may route), and 16384 tokens (the grouping
# bitmap's largest) with top-4; small experts keep the oracle quick.
@pytest.mark.parametrize("E,k,T", [(1024, 32, 2048), (16, 4, 16384)])
def test_moe_at_its_limits(E, k, T):
    print(f"moe limits E={E} k={k} T={T}", file=sys.stderr, flush=True)
    check(prefill_inputs.moe(E, k, 64, 64, T, seed=300 + E + k))


def test_moe512_matches_oracle():
    print("moe512: 512 experts, top-10, 512 tokens", file=sys.stderr, flush=True)
    m = prefill_inputs.workload("moe512")
    out = check(m)
    assert np.all(np.isfinite(out))


def test_moe512_repeatable_and_token_subsets():
    m = prefill_inputs.workload("moe512")
    moe = to_moe(m)
    x = dev(m["x"])
    ws = pf.workspace(moe.workspace_bytes(512))
    ids0, w0, o0 = [host(t) for t in moe.chunk(x, ws)]
    for _ in range(3):
        ids1, w1, o1 = [host(t) for t in moe.chunk(x, ws)]
        np.testing.assert_array_equal(ids1, ids0)
        np.testing.assert_array_equal(o1, o0)
    # tokens do not interact: a sub-chunk gives the same rows
    ws2 = pf.workspace(moe.workspace_bytes(77))
    ids2, w2, o2 = [host(t) for t in moe.chunk(x[100:177].contiguous(), ws2)]
    np.testing.assert_array_equal(ids2, ids0[100:177])
    np.testing.assert_array_equal(w2, w0[100:177])
    np.testing.assert_array_equal(o2, o0[100:177])
