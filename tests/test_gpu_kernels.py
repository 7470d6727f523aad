"""GPU parity of the single-kernel entry points against the oracle (bit-exact).

Every comparison is byte-for-byte: int8 codes identical, f32 outputs 0 ulp
(``assert_array_equal`` on the raw values).  Inputs come from prefill_inputs.
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


def test_init_reports_gfx950():
    pf.init()


# --- quantisation ----------------------------------------------------------------

# rows held in registers for every width up to 16384 values (1 to 16 pieces
# per thread), two passes beyond
@pytest.mark.parametrize("M,K", [(1, 64), (11, 1024), (32, 4096), (7, 11008), (512, 2048), (3, 1088),
                                 (5, 6144), (4, 16384), (3, 20480)])
def test_quantize_matches_oracle(M, K):
    x = prefill_inputs.activations(np.random.default_rng(M * 7 + K), (M, K))
    x[0, :5] = [0.0, -0.0, 2.5, -2.5, 1e-30]
    if M > 2:
        x[2] = 0.0                      # all-zero token
    q, s = pf.quantize_act(dev(x))
    qo, so = oracle.quantize(x)
    np.testing.assert_array_equal(host(s), so)
    np.testing.assert_array_equal(host(q), qo)


def test_quantize_exact_halves_and_golden():
    rows = []
    for j in (-6, 0, 3):
        n = np.arange(-126, 126)
        rows.append(np.concatenate([[127 * 2.0 ** j], (n + 0.5) * 2.0 ** j, np.zeros(3)]))
    x = np.array(rows, np.float32)
    q, s = pf.quantize_act(dev(x))
    qo, so = oracle.quantize(x)
    np.testing.assert_array_equal(host(q), qo)
    np.testing.assert_array_equal(host(s), so)


# --- GEMV and the chunk product ------------------------------------------------------

def _proj(N, K, M, seed):
    d = prefill_inputs.projection(N, K, M, seed)
    q, s = oracle.quantize(d["x"])
    return d["W"], d["w_scale"], q, s


@pytest.mark.parametrize("N,K", [(1024, 1024), (70, 128), (4096, 4096), (512, 2048)])
def test_gemv_matches_oracle(N, K):
    W, ws, q, s = _proj(N, K, 3, 100 + N)
    Wd, wsd = dev(W), dev(ws)
    for t in range(3):
        y = pf.gemv_i8(Wd, wsd, dev(q[t]), dev(s[t:t + 1]))
        np.testing.assert_array_equal(host(y), oracle.gemv(W, ws, q[t], s[t]))


@pytest.mark.parametrize("split", [False, True])
def test_proj1024_batched_equals_oracle_and_gemvs(split):
    """32 tokens against W [1024, 1024]: the chunk product, 32 per-token GEMVs and the
    oracle agree byte for byte ("Batched Prefill", §Correctness)."""
    d = prefill_inputs.workload("proj1024")
    W, ws, x = d["W"], d["w_scale"], d["x"]
    Wd, wsd = dev(W), dev(ws)
    q, s = pf.quantize_act(dev(x))
    qo, so = oracle.quantize(x)
    np.testing.assert_array_equal(host(q), qo)
    wsp = pf.workspace(pf.gemm_i8_chunk_workspace(1024, 1024, 32)) if split else None
    y = host(pf.gemm_i8_chunk(Wd, wsd, q, s, ws=wsp))
    np.testing.assert_array_equal(y, oracle.linear(W, ws, qo, so))
    for t in range(32):
        g = pf.gemv_i8(Wd, wsd, q[t].contiguous(), s[t:t + 1].contiguous())
        np.testing.assert_array_equal(host(g), y[t])


@pytest.mark.parametrize("M", list(range(1, 18)) + [31, 33, 48, 63, 64])
@pytest.mark.parametrize("split", [False, True])
def test_skinny_tails(M, split):
    N, K = 200, 1536                     # 200 rows: a ragged last band of 8 rows
    W, ws, q, s = _proj(N, K, M, 300 + M)
    wsp = pf.workspace(pf.gemm_i8_chunk_workspace(N, K, M)) if split else None
    if split:
        assert pf.gemm_i8_chunk_workspace(N, K, M) > 0
    y = pf.gemm_i8_chunk(dev(W), dev(ws), dev(q), dev(s), ws=wsp)
    np.testing.assert_array_equal(host(y), oracle.linear(W, ws, q, s))


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("M", [7, 33])
def test_skinny_unaligned_output(M, split):
    """Up to 64 tokens with an output that is only 4-byte aligned: the streamed
    kernel (unsplit) or the piecewise one (split), both with scalar stores."""
    N, K = 300, 1536
    W, ws, q, s = _proj(N, K, M, 800 + M)
    wsp = pf.workspace(pf.gemm_i8_chunk_workspace(N, K, M)) if split else None
    buf = torch.full((M * N + 1,), -1.0, dtype=torch.float32, device="cuda")
    out = buf[1:].view(M, N)
    pf.gemm_i8_chunk(dev(W), dev(ws), dev(q), dev(s), ws=wsp, out=out)
    np.testing.assert_array_equal(host(out), oracle.linear(W, ws, q, s))
    assert host(buf)[0] == -1.0


def test_skinny_many_tiles_long_k():
    """129 tiles of 64 rows (the last ragged) and 33 k-blocks: the whole K per
    tile in the streamed kernel, no split."""
    N, K, M = 8200, 2112, 37
    W, ws, q, s = _proj(N, K, M, 61)
    wsp = pf.workspace(pf.gemm_i8_chunk_workspace(N, K, M))
    y = pf.gemm_i8_chunk(dev(W), dev(ws), dev(q), dev(s), ws=wsp)
    np.testing.assert_array_equal(host(y), oracle.linear(W, ws, q, s))


def test_split_workspace_reused_with_garbage():
    # the split partials are overwritten each call: any workspace contents work
    N, K, M = 1024, 4096, 32
    W, ws, q, s = _proj(N, K, M, 41)
    nb = pf.gemm_i8_chunk_workspace(N, K, M)
    assert nb > 0
    wsp = torch.randint(0, 255, (nb,), dtype=torch.uint8, device="cuda")
    args = (dev(W), dev(ws), dev(q), dev(s))
    ref = oracle.linear(W, ws, q, s)
    for _ in range(5):
        np.testing.assert_array_equal(host(pf.gemm_i8_chunk(*args, ws=wsp)), ref)


@pytest.mark.parametrize("M", [65, 100, 128, 129, 300])
def test_tiled_matches_oracle(M):
    N, K = 392, 1024                     # ragged rows (392 = 3 * 128 + 8) and tokens
    W, ws, q, s = _proj(N, K, M, 500 + M)
    y = pf.gemm_i8_chunk(dev(W), dev(ws), dev(q), dev(s))
    np.testing.assert_array_equal(host(y), oracle.linear(W, ws, q, s))


@pytest.mark.parametrize("K", [64, 192, 256, 320, 1088])
@pytest.mark.parametrize("M", [65, 256])
def test_tiled_k_blocks_around_ring_depth(M, K):
    """k-block counts below, at and just above the stage ring's depth, and odd.
    522 rows (not a multiple of four) keep 65 tokens on the tiled kernel."""
    N = 522                              # two full 256-row tiles and 10 rows
    W, ws, q, s = _proj(N, K, M, 900 + M + K)
    y = pf.gemm_i8_chunk(dev(W), dev(ws), dev(q), dev(s))
    np.testing.assert_array_equal(host(y), oracle.linear(W, ws, q, s))


@pytest.mark.parametrize("M", [100, 200])
def test_tiled_unaligned_output(M):
    """An output that is only 4-byte aligned (the epilogue's 4-byte stores need no
    more) and whose rows are not a multiple of four floats apart."""
    N, K = 300, 512
    W, ws, q, s = _proj(N, K, M, 700 + M)
    buf = torch.full((M * N + 1,), -1.0, dtype=torch.float32, device="cuda")
    out = buf[1:].view(M, N)
    pf.gemm_i8_chunk(dev(W), dev(ws), dev(q), dev(s), out=out)
    np.testing.assert_array_equal(host(out), oracle.linear(W, ws, q, s))
    assert host(buf)[0] == -1.0


@pytest.mark.parametrize("N,K,M", [(520, 2048, 100), (300, 4096, 256), (1024, 1088, 300)])
def test_tiled_split_k_with_garbage_workspace(N, K, M):
    """Few tiles: the K range is split and the int32 partials are summed by a
    second launch; workspace contents on entry do not matter."""
    W, ws, q, s = _proj(N, K, M, 1300 + N + M)
    nb = pf.gemm_i8_chunk_workspace(N, K, M)
    assert nb > 0
    wsp = torch.randint(0, 255, (nb,), dtype=torch.uint8, device="cuda")
    args = (dev(W), dev(ws), dev(q), dev(s))
    ref = oracle.linear(W, ws, q, s)
    for _ in range(3):
        np.testing.assert_array_equal(host(pf.gemm_i8_chunk(*args, ws=wsp)), ref)


@pytest.mark.parametrize("K", [512, 1088, 4096])
@pytest.mark.parametrize("M", [65, 80, 113, 128])
def test_xres128_matches_oracle(M, K):
    """65 to 128 tokens on a small product (rows a multiple of four, aligned
    output): the token-resident kernel with eight 16-token blocks, tokens past M
    repeating row 0 and never stored.  K in one slice of at most 8 k-blocks
    (512), or split into slices with a ragged last one (1088: 8 + 8 + 1) or into
    eight (4096), the partials summed by the reduction.  Repeated calls on a
    workspace that starts as garbage."""
    N = 392                              # six 64-row tiles and 8 rows
    W, ws, q, s = _proj(N, K, M, 1700 + M + K)
    nb = pf.gemm_i8_chunk_workspace(N, K, M)
    if K > 512:
        assert nb >= 4 * M * N * ((K // 64 + 7) // 8)
    wsp = torch.randint(0, 255, (max(nb, 16),), dtype=torch.uint8, device="cuda")
    args = (dev(W), dev(ws), dev(q), dev(s))
    ref = oracle.linear(W, ws, q, s)
    for _ in range(2):
        np.testing.assert_array_equal(host(pf.gemm_i8_chunk(*args, ws=wsp)), ref)


def test_mfma_single_tiles_extreme_values():
    """One 16x16x64 and one 32x32x32 tile region with +-127 everywhere: operand
    layout and int32 range of the MFMA paths against exact integers."""
    rng = np.random.default_rng(9)
    for M in (16, 128):
        N, K = (16, 64) if M == 16 else (128, 128)
        W = rng.choice(np.array([-127, 127], np.int8), (N, K))
        q = rng.choice(np.array([-127, 127], np.int8), (M, K))
        ws = np.ones(N, np.float32)
        s = np.ones(M, np.float32)
        y = host(pf.gemm_i8_chunk(dev(W), dev(ws), dev(q), dev(s)))
        exact = (q.astype(np.int64) @ W.astype(np.int64).T).astype(np.float32)
        np.testing.assert_array_equal(y, exact)


def test_sweep4096_chunks_match_oracle_and_each_other():
    """W [4096, 4096]: chunk M in {1,...,512} uses the first M tokens; every M gives
    the oracle's bytes, so y_M equals the first M rows of y_512."""
    d = prefill_inputs.workload("sweep4096")
    W, ws, x = d["W"], d["w_scale"], d["x"]
    qo, so = oracle.quantize(x)
    ref = oracle.linear(W, ws, qo, so)
    Wd, wsd = dev(W), dev(ws)
    q, s = pf.quantize_act(dev(x))
    np.testing.assert_array_equal(host(q), qo)
    for M in prefill_inputs.WORKLOADS["sweep4096"]["chunks"]:
        say("sweep4096 M =", M)
        wsp = pf.workspace(pf.gemm_i8_chunk_workspace(4096, 4096, M))
        if M == 1:
            y = pf.gemv_i8(Wd, wsd, q[0].contiguous(), s[:1].contiguous())[None, :]
            np.testing.assert_array_equal(host(y), ref[:1])
        y = pf.gemm_i8_chunk(Wd, wsd, q[:M].contiguous(), s[:M].contiguous(), ws=wsp)
        np.testing.assert_array_equal(host(y), ref[:M])


@pytest.mark.parametrize("N,K,M", [(38400, 4096, 512), (16384, 16384, 320), (11008, 4096, 200)])
def test_large_tiled_products_equal_per_token_gemvs(N, K, M):
    """Products of hundreds of tiles (several rounds of workgroups per compute
    unit): every output of the chunk product equals the per-token GEMV's
    (both bit-exact definitions of the same arithmetic, "Batched Prefill",
    §Correctness), and sampled rows equal the oracle's."""
    say("large tiled", N, K, M)
    g = torch.Generator(device="cuda")
    g.manual_seed(N + K + M)
    W = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
    ws = torch.rand(N, device="cuda", generator=g) * 0.009 + 0.001
    x = torch.randn(M, K, device="cuda", generator=g)
    q, s = pf.quantize_act(x)
    wsp = pf.workspace(max(1, pf.gemm_i8_chunk_workspace(N, K, M)))
    y = pf.gemm_i8_chunk(W, ws, q, s, ws=wsp)
    y2 = pf.gemm_i8_chunk(W, ws, q, s, ws=wsp)            # the same call again
    per = torch.empty_like(y)
    for t in range(M):
        pf.gemv_i8(W, ws, q[t].contiguous(), s[t:t + 1].contiguous(), out=per[t])
    torch.cuda.synchronize()
    assert torch.equal(y, per)
    assert torch.equal(y, y2)
    rows = np.unique(np.concatenate([np.arange(0, N, 997), [N - 1]]))
    Wh = host(W)[rows]
    ref = oracle.linear(Wh, host(ws)[rows], host(q), host(s))
    np.testing.assert_array_equal(host(y)[:, rows], ref)


@pytest.mark.parametrize("M", [1, 32, 100])
def test_largest_accepted_product(M):
    """The largest weight matrix the entry points take: K at its maximum (131072)
    and N * K one row short of 2^32 bytes (the tiled copies address a matrix by
    32-bit offsets), through the GEMV (M = 1), the skinny path (32) and the tiled
    path (100); sampled rows, the last included, equal the oracle's.  (One row
    more is refused before any launch: test_abi.)"""
    K = 131072
    N = (1 << 32) // K - 1
    say("largest product", N, K, M)
    g = torch.Generator(device="cuda")
    g.manual_seed(M)
    W = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
    ws = torch.rand(N, device="cuda", generator=g) * 0.009 + 0.001
    q, s = pf.quantize_act(torch.randn(M, K, device="cuda", generator=g))
    if M == 1:
        y = pf.gemv_i8(W, ws, q[0].contiguous(), s[:1].contiguous())[None, :]
    else:
        wsp = pf.workspace(max(1, pf.gemm_i8_chunk_workspace(N, K, M)))
        y = pf.gemm_i8_chunk(W, ws, q, s, ws=wsp)
    rows = np.array([0, 1, 4097, N // 2, N - 2, N - 1])
    ref = oracle.linear(host(W[torch.from_numpy(rows).cuda()]), host(ws)[rows], host(q), host(s))
    np.testing.assert_array_equal(host(y)[:, rows], ref)
    del W
    torch.cuda.empty_cache()


def test_rejects_bad_arguments_without_launch():
    W = torch.zeros((64, 100), dtype=torch.int8, device="cuda")
    with pytest.raises(pf.PrefillError) as e:
        pf.gemm_i8_chunk(W, torch.ones(64, device="cuda"), torch.zeros((4, 100), dtype=torch.int8, device="cuda"),
                         torch.ones(4, device="cuda"))
    assert e.value.status == pf.PF_EINVAL


# --- exp -------------------------------------------------------------------------------

def test_expf_cr_whole_nonpositive_domain():
    """Every binary32 x in [-104, 0] (and a few beyond): the GPU exp equals the
    oracle's correctly rounded exp.  Where float64 exp decides the rounding the
    oracle is known to equal RN(float64 exp) (exhaustive CPU pin), elsewhere the
    oracle is called directly."""
    top = int(np.array(-104.0, np.float32).view(np.uint32))
    start = int(np.array(-0.0, np.float32).view(np.uint32))
    step = 1 << 26
    for lo in range(start, top + 1, step):
        bits = np.arange(lo, min(lo + step, top + 1), dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        g = host(pf.expf_cr(dev(x)))
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
    extra = np.float32([-104.5, -150.0, -1e30, -np.inf, 0.0, -0.0])
    np.testing.assert_array_equal(host(pf.expf_cr(dev(extra))), oracle.expf_cr(extra))
