"""GPU parity of pf_prefill_stack against the per-token oracle (bit-exact).

Covers: a small stack compared in full (outputs and every projection), the
350M-class stack (16 layers, hidden 1024, 747 tokens in 32-token chunks plus an
11-token tail) on every token with chunk invariance and the per-token GEMV
mode, and the 7B-class stack (32 layers, hidden 4096, 2048 tokens in 512-token
chunks) on every token.
"""
import hashlib
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


def to_stack(st):
    return pf.Stack([[dev(w) for w in wl] for wl in st["weights"]],
                    [[dev(s) for s in sl] for sl in st["scales"]])


def run(stack, x, chunk, proj=None, per_token=False, stats=False):
    ws = pf.workspace(stack.workspace_bytes(chunk))
    old = os.environ.get("PF_BATCHED_PREFILL")
    if per_token:
        os.environ["PF_BATCHED_PREFILL"] = "0"
    try:
        out = stack.prefill(x, chunk, ws, proj=proj, stats=stats)
    finally:
        if per_token:
            if old is None:
                del os.environ["PF_BATCHED_PREFILL"]
            else:
                os.environ["PF_BATCHED_PREFILL"] = old
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("chunk", [1, 5, 32, 64, 75, 96, 128])
def test_small_stack_full_compare(chunk):
    st = prefill_inputs.stack(L=3, H=128, F=320, P=75, seed=21)
    y_ref, proj_ref = oracle.stack(st["weights"], st["scales"], st["x"], return_proj=True)
    stack = to_stack(st)
    x = dev(st["x"])
    proj = torch.empty((3, 75, 5 * 128 + 2 * 320), dtype=torch.float32, device="cuda")
    y = run(stack, x, chunk, proj=proj)
    np.testing.assert_array_equal(host(y), y_ref)
    np.testing.assert_array_equal(host(proj), proj_ref)
    y2 = run(stack, x, chunk)                      # without the projection copy
    np.testing.assert_array_equal(host(y2), y_ref)


@pytest.mark.parametrize("chunk", [96, 160])
def test_tiled_stack_full_compare(chunk):
    """Chunks over 64 tokens on the tiled path with a longer down product
    (F = 2048, 32 k-blocks) and a ragged last chunk."""
    st = prefill_inputs.stack(L=3, H=256, F=2048, P=300, seed=23)
    y_ref, proj_ref = oracle.stack(st["weights"], st["scales"], st["x"], return_proj=True)
    stack = to_stack(st)
    x = dev(st["x"])
    proj = torch.empty((3, 300, 5 * 256 + 2 * 2048), dtype=torch.float32, device="cuda")
    y = run(stack, x, chunk, proj=proj)
    np.testing.assert_array_equal(host(y), y_ref)
    np.testing.assert_array_equal(host(proj), proj_ref)


def test_small_stack_per_token_mode_identical():
    st = prefill_inputs.stack(L=2, H=256, F=512, P=40, seed=22)
    stack = to_stack(st)
    x = dev(st["x"])
    yb, sb = run(stack, x, 32, stats=True)
    yt, stt = run(stack, x, 32, per_token=True, stats=True)
    assert sb["per_token_mode"] == 0 and stt["per_token_mode"] == 1
    assert sb["chunks"] == 2 and sb["tail_tokens"] == 8
    np.testing.assert_array_equal(host(yb), host(yt))
    np.testing.assert_array_equal(host(yb), oracle.stack(st["weights"], st["scales"], st["x"]))


@pytest.fixture(scope="module")
def stack350m():
    st = prefill_inputs.workload("stack350m")
    return st, to_stack(st), dev(st["x"])


def _digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_stack350m_all_tokens_match_oracle(stack350m):
    """Every one of the 747 tokens (23 chunks of 32 and the 11-token tail)."""
    st, stack, x = stack350m
    say("stack350m chunk 32")
    y = host(run(stack, x, 32))
    ref = oracle.stack(st["weights"], st["scales"], st["x"])
    np.testing.assert_array_equal(y, ref)
    assert np.all(np.isfinite(y))


def test_stack350m_chunk_invariance_and_per_token(stack350m):
    st, stack, x = stack350m
    base = _digest(host(run(stack, x, 32)))
    for chunk in (7, 64, 96, 747):
        say("stack350m chunk", chunk)
        assert _digest(host(run(stack, x, chunk))) == base, chunk
    say("stack350m per-token GEMV mode")
    assert _digest(host(run(stack, x, 32, per_token=True))) == base


def test_stack350m_repeatable(stack350m):
    st, stack, x = stack350m
    ws = pf.workspace(stack.workspace_bytes(32))
    y0 = host(stack.prefill(x, 32, ws))
    for _ in range(5):
        np.testing.assert_array_equal(host(stack.prefill(x, 32, ws)), y0)


@pytest.fixture(scope="module")
def stack7b():
    say("stack7b: generating 6.5 GB of weights")
    st = prefill_inputs.workload("stack7b")
    stack = to_stack(st)
    x = dev(st["x"])
    say("stack7b chunk 512")
    y = host(run(stack, x, 512))
    return st, stack, x, y


def test_stack7b_chunk_invariance(stack7b):
    st, stack, x, y = stack7b
    assert np.all(np.isfinite(y))
    say("stack7b chunk 1000 (ragged tail 48), 64 and 32 (skinny paths)")
    np.testing.assert_array_equal(host(run(stack, x, 1000)), y)
    np.testing.assert_array_equal(host(run(stack, x[:256].contiguous(), 64)), y[:256])
    np.testing.assert_array_equal(host(run(stack, x[:80].contiguous(), 32)), y[:80])


# every token of the 2048-token prompt against the oracle, one 512-token chunk
# per test (the oracle takes ~12 s per chunk on 16 host cores)
@pytest.mark.parametrize("c", [0, 1, 2, 3])
def test_stack7b_chunk_matches_oracle(stack7b, c):
    st, stack, x, y = stack7b
    say(f"stack7b oracle on tokens {512 * c} .. {512 * c + 511}")
    ref = oracle.stack(st["weights"], st["scales"], st["x"][512 * c:512 * (c + 1)])
    np.testing.assert_array_equal(y[512 * c:512 * (c + 1)], ref)


@pytest.mark.parametrize("chunk", [16, 96])
def test_second_weight_copy_same_bytes(chunk):
    """Odd chunks reading a second copy of the weights (pf_stack layers_alt)
    give the same bytes, including the projections."""
    st = prefill_inputs.stack(L=3, H=256, F=1024, P=200, seed=27)
    y_ref, proj_ref = oracle.stack(st["weights"], st["scales"], st["x"], return_proj=True)
    wd = [[dev(w) for w in wl] for wl in st["weights"]]
    sd = [[dev(s) for s in sl] for sl in st["scales"]]
    alt = ([[w.clone() for w in wl] for wl in wd], [[s.clone() for s in sl] for sl in sd])
    stack = pf.Stack(wd, sd, alt=alt)
    proj = torch.empty((3, 200, 5 * 256 + 2 * 1024), dtype=torch.float32, device="cuda")
    y = stack.prefill(dev(st["x"]), chunk, pf.workspace(stack.workspace_bytes(chunk)), proj=proj)
    np.testing.assert_array_equal(host(y), y_ref)
    np.testing.assert_array_equal(host(proj), proj_ref)
