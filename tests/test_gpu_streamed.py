"""GPU parity of the host-streamed stack (weights in pinned host memory, a
device ring of layer slots fed by a copy stream) against the oracle, and its
prefetch counters ("Predictive prefetch": the backend changes the schedule,
never the result)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import prefill_inputs
import int8_weight_gemm_amd as pf

pytestmark = pytest.mark.gpu


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def pinned(a):
    return torch.from_numpy(np.ascontiguousarray(a)).pin_memory()


def host_stack(st, act=0):
    return pf.HostStack([[pinned(w) for w in wl] for wl in st["weights"]],
                        [[pinned(s) for s in sl] for sl in st["scales"]], activation=act)


@pytest.mark.parametrize("chunk,n_buffers", [(32, 2), (7, 3), (96, 2), (300, 4)])
def test_streamed_stack_matches_oracle(chunk, n_buffers):
    st = prefill_inputs.stack(L=5, H=256, F=1024, P=300, seed=101)
    ref = oracle.stack(st["weights"], st["scales"], st["x"])
    hs = host_stack(st)
    x = torch.from_numpy(st["x"]).cuda()
    ws = pf.workspace(hs.workspace_bytes(300, n_buffers))
    y, stats = hs.prefill(x, chunk, ws, n_buffers=n_buffers, stats=True)
    np.testing.assert_array_equal(host(y), ref)
    assert stats["layers_copied"] == 5
    assert stats["prefetch_hits"] + stats["prefetch_misses"] == 5
    assert stats["prefetch_misses"] >= 1                     # the first layer's copy
    # again on the same workspace (the ring holds the previous call's layers)
    np.testing.assert_array_equal(host(hs.prefill(x, chunk, ws, n_buffers=n_buffers)), ref)


def test_streamed_stack_gated_silu():
    st = prefill_inputs.stack(L=3, H=256, F=512, P=70, seed=102)
    ref = oracle.stack(st["weights"], st["scales"], st["x"], act=oracle.ACT_SWIGLU)
    hs = host_stack(st, act=pf.ACT_SWIGLU)
    y = hs.prefill(torch.from_numpy(st["x"]).cuda(), 32, pf.workspace(hs.workspace_bytes(70)))
    np.testing.assert_array_equal(host(y), ref)


def test_streamed_stack350m_matches_resident():
    """The 350M-class stack streamed from host memory gives the bytes of the
    resident stack and of the oracle on every token; the ring's counters are
    reported."""
    print("stack350m streamed from pinned host memory", file=sys.stderr, flush=True)
    st = prefill_inputs.workload("stack350m")
    hs = host_stack(st)
    x = torch.from_numpy(st["x"]).cuda()
    y, stats = hs.prefill(x, 32, pf.workspace(hs.workspace_bytes(747)), stats=True)
    y = host(y)
    np.testing.assert_array_equal(y, oracle.stack(st["weights"], st["scales"], st["x"]))
    dev_stack = pf.Stack([[torch.from_numpy(w).cuda() for w in wl] for wl in st["weights"]],
                         [[torch.from_numpy(s).cuda() for s in sl] for sl in st["scales"]])
    y2 = dev_stack.prefill(x, 32, pf.workspace(dev_stack.workspace_bytes(32)))
    np.testing.assert_array_equal(host(y2), y)
    print("ring:", stats, file=sys.stderr, flush=True)
    assert stats["prefetch_hits"] + stats["prefetch_misses"] == 16
