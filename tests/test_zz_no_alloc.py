"""pf_gemm_i8_chunk_noalloc: the chunk product with its split partials in the
library's own device array instead of a workspace.  Its outputs must be the
bytes of pf_gemm_i8_chunk (with a workspace) on two calls in a row, the second
with a smaller input, whose partials overwrite the first call's in the shared
array; and a product whose split plan needs more than the array holds is
refused before any device work."""
import sys

import numpy as np
import pytest
import torch

import prefill_inputs
import int8_weight_gemm_amd as pf

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def operands(N, K, M, seed):
    d = prefill_inputs.projection(N, K, M, seed)
    W, ws = dev(d["W"]), dev(d["w_scale"])
    q, s = pf.quantize_act(dev(d["x"]))
    return W, ws, q, s


def with_workspace(W, ws, q, s):
    N, K = W.shape
    M = q.shape[0]
    nb = pf.gemm_i8_chunk_workspace(N, K, M)
    assert 0 < nb <= pf.NOALLOC_SCRATCH_BYTES
    return host(pf.gemm_i8_chunk(W, ws, q, s, ws=pf.workspace(nb)))


# (N, K, M) pairs, the second call smaller than the first; each needs split
# partials: the tiled product split four ways, then the token-resident product
# split into 16-k-block slices; the 65-128-token token-resident product, then
# the piecewise split product
@pytest.mark.parametrize("first,second", [((4096, 4096, 512), (1024, 4096, 32)),
                                          ((392, 4096, 100), (512, 2048, 17))])
def test_noalloc_equals_workspace_product_twice(first, second):
    pf.init()
    for i, (N, K, M) in enumerate((first, second)):
        print(f"noalloc call {i}: N={N} K={K} M={M}", file=sys.stderr, flush=True)
        W, ws, q, s = operands(N, K, M, 2000 + N + M)
        ref = with_workspace(W, ws, q, s)
        y = torch.full((M, N), -1.0, dtype=torch.float32, device="cuda")
        pf.gemm_i8_chunk_noalloc(W, ws, q, s, out=y)
        np.testing.assert_array_equal(host(y), ref)
