"""GPU parity of the oracle-changing variants (bit-exact): the gated SiLU
between the gate/up and the down products, in the stack and in the experts,
and top-k weights renormalised over the chosen experts.  Also the GPU exp over
the positive arguments the gated SiLU gives it (exp(-g) for g < 0)."""
import os
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


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_stack(st, **kw):
    return pf.Stack([[dev(w) for w in wl] for wl in st["weights"]],
                    [[dev(s) for s in sl] for sl in st["scales"]], **kw)


@pytest.fixture(scope="module")
def swiglu_stack():
    st = prefill_inputs.stack(L=3, H=256, F=1024, P=200, seed=71)
    y_ref, proj_ref = oracle.stack(st["weights"], st["scales"], st["x"], return_proj=True,
                                   act=oracle.ACT_SWIGLU)
    return st, y_ref, proj_ref, to_stack(st, activation=pf.ACT_SWIGLU)


@pytest.mark.parametrize("chunk", [1, 7, 32, 64, 96, 160, 200])
def test_stack_swiglu_full_compare(swiglu_stack, chunk):
    st, y_ref, proj_ref, stack = swiglu_stack
    proj = torch.empty((3, 200, 5 * 256 + 2 * 1024), dtype=torch.float32, device="cuda")
    y = stack.prefill(dev(st["x"]), chunk, pf.workspace(stack.workspace_bytes(chunk)), proj=proj)
    np.testing.assert_array_equal(host(y), y_ref)
    np.testing.assert_array_equal(host(proj), proj_ref)
    assert np.all(np.isfinite(y_ref))


@pytest.mark.parametrize("chunk", [32, 96, 200])
def test_stack_swiglu_without_projection_rows(swiglu_stack, chunk):
    """No projection rows kept: q, k, v and o are not stored, gate is (the gated
    SiLU reads it); y is the same."""
    st, y_ref, _, stack = swiglu_stack
    y = stack.prefill(dev(st["x"]), chunk, pf.workspace(stack.workspace_bytes(chunk)))
    np.testing.assert_array_equal(host(y), y_ref)


def test_stack_swiglu_per_token_mode(swiglu_stack):
    st, y_ref, _, stack = swiglu_stack
    os.environ["PF_BATCHED_PREFILL"] = "0"
    try:
        y = stack.prefill(dev(st["x"][:40]), 32, pf.workspace(stack.workspace_bytes(32)))
    finally:
        del os.environ["PF_BATCHED_PREFILL"]
    np.testing.assert_array_equal(host(y), y_ref[:40])


def test_stack_swiglu_long_rows():
    """F = 20480: the gated rows exceed the register-held width and take the
    two-pass quantisation, which evaluates the gated row twice."""
    st = prefill_inputs.stack(L=1, H=256, F=20480, P=40, seed=72)
    y_ref = oracle.stack(st["weights"], st["scales"], st["x"], act=oracle.ACT_SWIGLU)
    stack = to_stack(st, activation=pf.ACT_SWIGLU)
    for chunk in (32, 40):
        y = stack.prefill(dev(st["x"]), chunk, pf.workspace(stack.workspace_bytes(chunk)))
        np.testing.assert_array_equal(host(y), y_ref)


def check_moe(m, x):
    moe = pf.Moe(m["n_experts"], m["top_k"], *[dev(m[n]) for n in (
        "W_router", "W_gate", "W_up", "W_down", "s_gate", "s_up", "s_down")],
        activation=m.get("activation", 0), renormalize=m.get("renormalize", 0))
    ids, w, out = moe.chunk(dev(x), pf.workspace(moe.workspace_bytes(x.shape[0])))
    ids_o, w_o, out_o = oracle.moe(m, x)
    np.testing.assert_array_equal(host(ids), ids_o)
    np.testing.assert_array_equal(host(w), w_o)
    np.testing.assert_array_equal(host(out), out_o)
    return ids_o, w_o, out_o


# streaming expert kernel (K 512 / 1024 / 2048) and the piecewise one (K 576)
@pytest.mark.parametrize("act,renorm", [(1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("E,k,H,I,T", [(16, 4, 512, 1024, 70), (8, 2, 576, 512, 40), (64, 10, 256, 128, 100)])
def test_moe_variants_match_oracle(act, renorm, E, k, H, I, T):
    m = prefill_inputs.moe(E, k, H, I, T, seed=300 + E + T)
    m["activation"], m["renormalize"] = act, renorm
    x = m["x"].copy()
    x[1] = 0.0                                  # an all-zero token: equal logits
    check_moe(m, x)


def test_moe512_swiglu_renormalised():
    say("moe512, gated SiLU and renormalised weights")
    m = prefill_inputs.workload("moe512")
    m["activation"], m["renormalize"] = 1, 1
    _, w, out = check_moe(m, m["x"])
    assert np.all(np.isfinite(out))
    assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - 1.0) <= 20 * 2.0 ** -24)


def test_expf_cr_positive_domain():
    """Every binary32 x in [0, 89] and a few beyond: the GPU exp equals the
    correctly rounded exp (float64 exp decides, near-midpoint cases the
    oracle)."""
    top = int(np.array(89.0, np.float32).view(np.uint32))
    step = 1 << 26
    for lo in range(0, top + 1, step):
        bits = np.arange(lo, min(lo + step, top + 1), dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        g = host(pf.expf_cr(dev(x)))
        with np.errstate(over="ignore"):
            d = np.exp(x.astype(np.float64))
            r = d.astype(np.float32)
        nb = np.where(d > r.astype(np.float64), np.nextafter(r, np.float32(np.inf)),
                      np.nextafter(r, np.float32(-np.inf)))
        mid = (r.astype(np.float64) + nb.astype(np.float64)) / 2
        close = np.abs(d - mid) <= np.abs(d) * 2.0 ** -50
        far_bad = (g != r) & ~close
        assert not far_bad.any(), x[far_bad][:5]
        if close.any():
            np.testing.assert_array_equal(g[close], oracle.expf_cr(x[close]))
    extra = np.float32([89.5, 100.0, 1e30, np.inf, 88.72283, 88.72284])
    np.testing.assert_array_equal(host(pf.expf_cr(dev(extra))), oracle.expf_cr(extra))


@pytest.fixture
def fused_experts(monkeypatch):
    """PF_MOE_FUSED=1: gate/up, quantise(r) and down as one launch."""
    monkeypatch.setenv("PF_MOE_FUSED", "1")


# the fused expert kernel (hidden and inter of 512, 1024 or 2048): groups of up
# to 32 pairs (E = 8, top-2 of 150 tokens: over 32 per expert), both orders of
# H and I, gated SiLU, and an all-zero token (its r rows are zero: scale 0)
@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("E,k,H,I,T", [(16, 4, 512, 1024, 70), (8, 2, 1024, 512, 150),
                                       (4, 1, 2048, 2048, 33), (32, 4, 2048, 512, 64)])
def test_moe_fused_experts_match_oracle(fused_experts, act, E, k, H, I, T):
    say(f"fused experts E={E} k={k} H={H} I={I} T={T} act={act}")
    m = prefill_inputs.moe(E, k, H, I, T, seed=400 + E + T)
    m["activation"] = act
    x = m["x"].copy()
    x[2] = 0.0
    check_moe(m, x)


def test_moe512_fused_experts_match_oracle(fused_experts):
    say("moe512 with the fused expert kernel")
    m = prefill_inputs.workload("moe512")
    check_moe(m, m["x"])
