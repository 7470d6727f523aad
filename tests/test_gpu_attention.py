"""GPU parity of the stack with causal attention over its K/V cache against the
oracle (bit-exact): y, every projection (o now from the attention) and the
cache itself, at chunk sizes that split the prompt in many ways (a chunk's
tokens attend to earlier chunks' cache rows written by other chunk groups),
in the per-token mode, and for the 350M-class stack with 16 heads."""
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


def run(st, n_heads, chunk, act=0, per_token=False, alt=False, keep_proj=True):
    wd = [[dev(w) for w in wl] for wl in st["weights"]]
    sd = [[dev(s) for s in sl] for sl in st["scales"]]
    altc = ([[w.clone() for w in wl] for wl in wd], [[s.clone() for s in sl] for sl in sd]) if alt else None
    stack = pf.Stack(wd, sd, alt=altc, activation=act, n_heads=n_heads)
    L, P, H = len(wd), st["x"].shape[0], stack.H
    proj = torch.empty((L, P, 5 * H + 2 * stack.F), dtype=torch.float32, device="cuda") if keep_proj else None
    kv = torch.full((L, 2, P, H), float("nan"), dtype=torch.float32, device="cuda")
    if per_token:
        os.environ["PF_BATCHED_PREFILL"] = "0"
    try:
        y = stack.prefill(dev(st["x"]), chunk, pf.workspace(stack.workspace_bytes(chunk)), proj=proj, kv=kv)
    finally:
        if per_token:
            del os.environ["PF_BATCHED_PREFILL"]
    return host(y), (host(proj) if keep_proj else None), host(kv)


@pytest.fixture(scope="module")
def small():
    st = prefill_inputs.stack(L=3, H=256, F=512, P=150, seed=91)
    ref = oracle.stack_attn(st["weights"], st["scales"], st["x"], 4, return_proj=True)
    return st, ref


@pytest.mark.parametrize("chunk", [1, 7, 32, 64, 96, 150, 200])
def test_attention_stack_matches_oracle(small, chunk):
    st, (y_ref, kv_ref, proj_ref) = small
    y, proj, kv = run(st, 4, chunk)
    np.testing.assert_array_equal(kv, kv_ref)
    np.testing.assert_array_equal(proj, proj_ref)
    np.testing.assert_array_equal(y, y_ref)


@pytest.mark.parametrize("chunk", [32, 96, 150])
def test_attention_without_projection_rows(small, chunk):
    """No projection rows kept: only q (read by the attention) and up (read by
    the down product's quantisation) are stored besides the cache; y and the
    cache are the same."""
    st, (y_ref, kv_ref, _) = small
    y, _, kv = run(st, 4, chunk, keep_proj=False)
    np.testing.assert_array_equal(kv, kv_ref)
    np.testing.assert_array_equal(y, y_ref)


def test_attention_stack_per_token_mode(small):
    st, (y_ref, kv_ref, proj_ref) = small
    y, proj, kv = run(st, 4, 32, per_token=True)
    np.testing.assert_array_equal(kv, kv_ref)
    np.testing.assert_array_equal(proj, proj_ref)


def test_attention_second_weight_copy(small):
    st, (y_ref, kv_ref, proj_ref) = small
    y, proj, kv = run(st, 4, 16, alt=True)
    np.testing.assert_array_equal(kv, kv_ref)
    np.testing.assert_array_equal(proj, proj_ref)


# head widths 128, 64, 16 (32 heads: more heads than waves) and 4
@pytest.mark.parametrize("H,n_heads,chunk", [(256, 2, 32), (512, 32, 32), (256, 64, 96), (1024, 16, 64)])
def test_attention_head_shapes(H, n_heads, chunk):
    st = prefill_inputs.stack(L=2, H=H, F=512, P=100, seed=92 + n_heads)
    y_ref, kv_ref, proj_ref = oracle.stack_attn(st["weights"], st["scales"], st["x"], n_heads,
                                                return_proj=True)
    y, proj, kv = run(st, n_heads, chunk)
    np.testing.assert_array_equal(kv, kv_ref)
    np.testing.assert_array_equal(proj, proj_ref)


def test_attention_with_gated_silu():
    st = prefill_inputs.stack(L=2, H=256, F=512, P=80, seed=97)
    y_ref, kv_ref, proj_ref = oracle.stack_attn(st["weights"], st["scales"], st["x"], 4,
                                                return_proj=True, act=oracle.ACT_SWIGLU)
    y, proj, kv = run(st, 4, 32, act=pf.ACT_SWIGLU)
    np.testing.assert_array_equal(y, y_ref)
    np.testing.assert_array_equal(proj, proj_ref)
    np.testing.assert_array_equal(kv, kv_ref)


def test_stack350m_attention_all_tokens():
    """16 layers, hidden 1024, 16 heads of 64, the 747-token prompt in 32-token
    chunks: every token, every projection and the whole cache."""
    say("stack350m with attention: oracle")
    st = prefill_inputs.workload("stack350m")
    y_ref, kv_ref, proj_ref = oracle.stack_attn(st["weights"], st["scales"], st["x"], 16,
                                                return_proj=True)
    say("stack350m with attention: GPU")
    y, proj, kv = run(st, 16, 32)
    np.testing.assert_array_equal(kv, kv_ref)
    np.testing.assert_array_equal(proj, proj_ref)
    np.testing.assert_array_equal(y, y_ref)


def test_attention_requires_cache():
    st = prefill_inputs.stack(L=1, H=256, F=512, P=10, seed=98)
    stack = pf.Stack([[dev(w) for w in wl] for wl in st["weights"]],
                     [[dev(s) for s in sl] for sl in st["scales"]], n_heads=4)
    with pytest.raises(pf.PrefillError) as e:
        stack.prefill(dev(st["x"]), 32, pf.workspace(stack.workspace_bytes(32)))
    assert e.value.status == pf.PF_EINVAL
