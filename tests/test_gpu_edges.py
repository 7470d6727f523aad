"""GPU parity on the method's own edge cases, against the oracle (bit-exact).

* Top-k ties: routers with equal rows give equal logits, so equal
  probabilities meet inside a token's top-k and at its boundary; the lower
  expert id must win ("Red Lite dev24", What changed item 2: ids and weights
  identical to the single-token routine).  An all-zero token has every logit 0,
  p = 1/E and ids 0..k-1.
* int32 accumulators above 2^24, where the int -> f32 conversion rounds: codes
  and weights of magnitude 126..127 at K >= 1088 give |acc| from 1.7e7 to
  1.8e8 with random low bits, through every product kernel (GEMV, the
  token-resident product split and unsplit, the streamed product, the piecewise
  product with split partials, the tiled product split and unsplit) and through
  the stack's rebuild of the down product from its split partials.
* All-zero tokens (scale 0, codes 0, outputs +0) through the stack's chunk-32
  and chunk-512 paths and the expert chunk.
* A prompt shorter than one chunk, with exactly the queried workspace.
"""
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


# --- top-k ties ------------------------------------------------------------------------

def tied_router(m, seed):
    """Router rows repeated: experts 2j and 2j+1 equal below 384, groups of four
    above, so every token's logits come in equal pairs or quadruples."""
    E, H = m["W_router"].shape
    rng = np.random.default_rng(seed)
    base = (rng.standard_normal((E, H), dtype=np.float32) / np.float32(np.sqrt(H))).astype(np.float32)
    e = np.arange(E)
    src = np.where(e < 3 * E // 4, e // 2, 3 * E // 8 + (e - 3 * E // 4) // 4)
    m["W_router"] = np.ascontiguousarray(base[src])
    return m


def check_moe(m, x):
    moe = pf.Moe(m["n_experts"], m["top_k"], *[dev(m[n]) for n in (
        "W_router", "W_gate", "W_up", "W_down", "s_gate", "s_up", "s_down")])
    ids, w, out = moe.chunk(dev(x), pf.workspace(moe.workspace_bytes(x.shape[0])))
    ids_o, w_o, out_o = oracle.moe(m, x)
    np.testing.assert_array_equal(host(ids), ids_o)
    np.testing.assert_array_equal(host(w), w_o)
    np.testing.assert_array_equal(host(out), out_o)
    return ids_o, w_o, out_o


def test_moe512_topk_ties_and_zero_tokens():
    say("moe512 with tied router rows and all-zero tokens")
    m = tied_router(prefill_inputs.workload("moe512"), seed=77)
    x = m["x"].copy()
    x[5] = 0.0
    x[300] = 0.0
    ids, w, out = check_moe(m, x)
    # the ties are really there: in most tokens equal weights sit side by side
    # in the top-10, the lower id first
    tied = (w[:, 1:] == w[:, :-1])
    assert tied.sum() > 1000
    assert np.all(ids[:, 1:][tied] > ids[:, :-1][tied])
    # all-zero token: p = 1/512 everywhere, ids 0..9, output +0
    for t in (5, 300):
        np.testing.assert_array_equal(ids[t], np.arange(10))
        assert np.all(w[t] == np.float32(1.0 / 512))
        assert np.all(out[t] == 0.0) and not np.signbit(out[t]).any()


def test_small_moe_ties_at_the_boundary():
    """Groups of equal logits straddling the k-th place: the lower ids of the
    group are taken, the higher ones dropped."""
    m = tied_router(prefill_inputs.moe(64, 5, 256, 128, 90, seed=31), seed=5)
    ids, w, _ = check_moe(m, m["x"])
    assert (w[:, -1] == w[:, -2]).any()


# --- accumulators above 2^24 -------------------------------------------------------------

def big_acc(N, K, M, seed):
    """Weights +-(126 or 127) per row sign, codes 126 or 127: |acc| between
    15876 K and 16129 K (above 2^24 from K = 1088) with random low bits.  Half
    of the rows and tokens have scale 1, so the output is the rounded
    accumulator itself."""
    rng = np.random.default_rng(seed)
    sign = np.where(rng.integers(0, 2, N) == 1, 1, -1).astype(np.int16)[:, None]
    W = (sign * (126 + rng.integers(0, 2, (N, K)))).astype(np.int8)
    q = (126 + rng.integers(0, 2, (M, K))).astype(np.int8)
    ws = rng.uniform(0.001, 0.01, N).astype(np.float32)
    ws[::2] = 1.0
    s = rng.uniform(0.001, 0.01, M).astype(np.float32)
    s[::2] = 1.0
    return W, ws, q, s


def _exact_rows_are_rounded(y, W, q, ws, s):
    """Where both scales are 1, y is the accumulator rounded to binary32, and
    some of those accumulators are not binary32 values."""
    acc = q[::2].astype(np.int64) @ W[::2].astype(np.int64).T
    assert np.abs(acc).min() > 2 ** 24
    np.testing.assert_array_equal(y[::2, ::2], acc.astype(np.float32))
    assert (acc.astype(np.float32).astype(np.int64) != acc).any()


@pytest.mark.parametrize("K", [1088, 4096, 11008])
def test_gemv_accumulators_above_2_24(K):
    W, ws, q, s = big_acc(96, K, 2, seed=K)
    for t in range(2):
        y = host(pf.gemv_i8(dev(W), dev(ws), dev(q[t]), dev(s[t:t + 1])))
        np.testing.assert_array_equal(y, oracle.gemv(W, ws, q[t], s[t]))
    # token 0 has scale 1: on rows of scale 1 the output is the rounded accumulator
    y0 = host(pf.gemv_i8(dev(W), dev(ws), dev(q[0]), dev(s[:1])))
    acc = W.astype(np.int64) @ q[0].astype(np.int64)
    assert np.abs(acc).min() > 2 ** 24
    np.testing.assert_array_equal(y0[::2], acc[::2].astype(np.float32))


# (N, K, M, workspace, output offset in floats): which kernel takes the product
CHUNK_CASES = {
    "token-resident split (4 x 16 k-blocks) + reduction": (1024, 4096, 32, True, 0),
    "token-resident split, 11008 = 11 x 16 k-blocks": (512, 11008, 17, True, 0),
    "streamed, whole K per tile (17 k-blocks)": (1024, 1088, 32, False, 0),
    "streamed, K 11008": (260, 11008, 9, False, 0),
    "piecewise split, unaligned output + reduction": (300, 4096, 33, True, 1),
    "tiled unsplit": (512, 4096, 256, False, 0),
    "tiled split + reduction": (512, 4096, 256, True, 0),
    "tiled unsplit, 11008": (300, 11008, 100, False, 0),
    "token-resident 65-128 tokens, 8-k-block slices + reduction": (392, 4096, 100, True, 0),
}


@pytest.mark.parametrize("case", sorted(CHUNK_CASES))
def test_chunk_product_accumulators_above_2_24(case):
    N, K, M, use_ws, off = CHUNK_CASES[case]
    say("product", case)
    W, ws, q, s = big_acc(N, K, M, seed=N + K + M)
    wsp = pf.workspace(pf.gemm_i8_chunk_workspace(N, K, M)) if use_ws else None
    if use_ws:
        assert pf.gemm_i8_chunk_workspace(N, K, M) > 0
    buf = torch.full((M * N + off,), -1.0, dtype=torch.float32, device="cuda")
    out = buf[off:].view(M, N)
    pf.gemm_i8_chunk(dev(W), dev(ws), dev(q), dev(s), ws=wsp, out=out)
    y = host(out)
    np.testing.assert_array_equal(y, oracle.linear(W, ws, q, s))
    _exact_rows_are_rounded(y, W, q, ws, s)


def big_down_stack(L, H, F, P, seed):
    """A stack whose up projection gives every output of a token the same value
    (identical rows, equal scales), so the down product's codes are all +-127,
    against down rows of +-(126 or 127): |acc| ~ 127 * 126.5 * F, above 2^24,
    through the split partials and their rebuild."""
    st = prefill_inputs.stack(L=L, H=H, F=F, P=P, seed=seed)
    rng = np.random.default_rng(seed)
    for l in range(L):
        row = rng.integers(-127, 128, H).astype(np.int8)
        st["weights"][l][5] = np.ascontiguousarray(np.broadcast_to(row, (F, H)))
        st["scales"][l][5] = np.full(F, st["scales"][l][5][0], np.float32)
        sign = np.where(rng.integers(0, 2, H) == 1, 1, -1).astype(np.int16)[:, None]
        st["weights"][l][6] = (sign * (126 + rng.integers(0, 2, (H, F)))).astype(np.int8)
    return st


def to_stack(st):
    return pf.Stack([[dev(w) for w in wl] for wl in st["weights"]],
                    [[dev(s) for s in sl] for sl in st["scales"]])


@pytest.mark.parametrize("chunk", [32, 96])
def test_stack_down_accumulators_above_2_24(chunk):
    st = big_down_stack(L=2, H=256, F=2048, P=150, seed=12)
    y_ref, proj_ref = oracle.stack(st["weights"], st["scales"], st["x"], return_proj=True)
    stack = to_stack(st)
    x = dev(st["x"])
    proj = torch.empty((2, 150, 5 * 256 + 2 * 2048), dtype=torch.float32, device="cuda")
    y = stack.prefill(x, chunk, pf.workspace(stack.workspace_bytes(chunk)), proj=proj)
    np.testing.assert_array_equal(host(y), y_ref)
    np.testing.assert_array_equal(host(proj), proj_ref)
    y2 = stack.prefill(x, chunk, pf.workspace(stack.workspace_bytes(chunk)))   # rebuilt, no proj
    np.testing.assert_array_equal(host(y2), y_ref)


# --- all-zero tokens ---------------------------------------------------------------------

@pytest.mark.parametrize("chunk", [32, 512])
def test_stack_all_zero_tokens(chunk):
    """Zero tokens stay +0 through every layer; a chunk made only of zero tokens
    (tokens 32..63) and scattered ones."""
    st = prefill_inputs.stack(L=3, H=256, F=1024, P=600, seed=44)
    x = st["x"].copy()
    x[[0, 7, 100, 599]] = 0.0
    x[32:64] = 0.0
    y_ref = oracle.stack(st["weights"], st["scales"], x)
    stack = to_stack(st)
    y = host(stack.prefill(dev(x), chunk, pf.workspace(stack.workspace_bytes(chunk))))
    np.testing.assert_array_equal(y, y_ref)
    z = y[[0, 7, 100, 599, 40]]
    assert np.all(z == 0.0) and not np.signbit(z).any()


def test_moe_all_zero_chunk_rows():
    m = prefill_inputs.moe(64, 10, 512, 512, 64, seed=8)
    x = m["x"].copy()
    x[::3] = 0.0
    _, _, out = check_moe(m, x)
    assert np.all(out[::3] == 0.0)


# --- a prompt shorter than one chunk -----------------------------------------------------

@pytest.mark.parametrize("P,chunk", [(40, 128), (64, 256), (3, 96)])
def test_short_prompt_with_queried_workspace(P, chunk):
    st = prefill_inputs.stack(L=3, H=256, F=1024, P=P, seed=50 + P)
    stack = to_stack(st)
    ws = torch.zeros(stack.workspace_bytes(chunk), dtype=torch.uint8, device="cuda")
    y = host(stack.prefill(dev(st["x"]), chunk, ws))
    np.testing.assert_array_equal(y, oracle.stack(st["weights"], st["scales"], st["x"]))
