"""Plain CPU oracle of the batched int8-weight prefill path (ctypes binding).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library (``int8_weight_gemm_amd``) never imports it and shares no code with it.

The arithmetic lives in ``prefill_oracle.c`` (C11, libm, OpenMP over tokens),
compiled by :func:`build` with gcc and ``-ffp-contract=off``; this module only
marshals numpy arrays.  Every function is per token: the oracle has no notion of
a chunk, so chunk-invariance of the GPU path is a property the tests check.

Sources: "Batched Prefill" (cellm), §The Problem / §The Solution / §Correctness;
"Single-pass prefill" (SipLLM), "The fix"; "Red Lite dev24", "What changed".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "prefill_oracle.c")
_LIB = os.path.join(_HERE, "libprefill_oracle.so")

CFLAGS = ["-std=c11", "-O2", "-ftree-vectorize", "-mavx2", "-ffp-contract=off",
          "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build() -> str:
    """Compile the oracle with gcc into ``oracle/libprefill_oracle.so``."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        F = ctypes.c_float
        INT = ctypes.c_int
        sigs = {
            "or_quantize": [P, I64, I64, P, P],
            "or_gemv": [P, P, I64, I64, P, F, P],
            "or_linear_per_token": [P, P, I64, I64, P, P, I64, P, INT],
            "or_stack": [I64, I64, I64, P, P, P, I64, P, P, INT, INT],
            "or_stack_attn": [I64, I64, I64, I64, P, P, P, I64, P, P, P, INT, INT],
            "or_router": [P, I64, I64, P, P],
            "or_expf_cr_array": [P, I64, P, INT],
            "or_softmax_topk": [P, I64, I64, P, P, INT],
            "or_expert": [I64, I64, P, P, P, P, P, P, I64, P, F, P, INT],
            "or_moe": [I64, I64, I64, I64, P, P, P, P, P, P, P, P, I64, P, P, P, INT, INT, INT],
        }
        for name, args in sigs.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.or_expf_cr.argtypes = [F]
        lib.or_expf_cr.restype = F
        lib.or_silu.argtypes = [F]
        lib.or_silu.restype = F
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, name: str):
    if rc != 0:
        raise ValueError(f"{name} returned {rc}")


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def quantize(x: np.ndarray):
    """Per-token symmetric quantisation of x [M, K] -> (q int8 [M, K], s f32 [M])."""
    x = _c(np.atleast_2d(x), np.float32)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    _check(_load().or_quantize(_ptr(x), M, K, _ptr(q), _ptr(s)), "or_quantize")
    return q, s


def gemv(W: np.ndarray, w_scale: np.ndarray, q: np.ndarray, a_scale: float) -> np.ndarray:
    """One token: y[n] = (float)(W[n] . q) * (w_scale[n] * a_scale)."""
    W = _c(W, np.int8)
    N, K = W.shape
    ws = _c(w_scale, np.float32)
    q = _c(q, np.int8).reshape(K)
    y = np.empty(N, np.float32)
    _check(_load().or_gemv(_ptr(W), _ptr(ws), N, K, _ptr(q), float(np.float32(a_scale)),
                           _ptr(y)), "or_gemv")
    return y


def linear(W, w_scale, q, a_scale, threads: int | None = None) -> np.ndarray:
    """GEMV per token row of q [M, K] -> y [M, N] (token-major)."""
    W = _c(W, np.int8)
    N, K = W.shape
    q = _c(np.atleast_2d(q), np.int8)
    M = q.shape[0]
    assert q.shape[1] == K
    s = _c(a_scale, np.float32).reshape(M)
    y = np.empty((M, N), np.float32)
    _check(_load().or_linear_per_token(_ptr(W), _ptr(_c(w_scale, np.float32)), N, K, _ptr(q),
                                       _ptr(s), M, _ptr(y), threads or default_threads()),
           "or_linear_per_token")
    return y


ACT_NONE, ACT_SWIGLU = 0, 1


def stack(weights, scales, x, return_proj: bool = False, threads: int | None = None,
          act: int = ACT_NONE):
    """The projection stack token by token.

    weights[l] is the list (q, k, v, o, gate, up, down) of int8 arrays of layer l,
    scales[l] the matching f32 per-row scales.  x [P, H] -> y [P, H]; with
    ``return_proj`` also every projection output [L, P, 5H + 2F].  act selects
    the down projection's input: quantise(up), or quantise(silu(gate) * up).
    """
    L = len(weights)
    x = _c(np.atleast_2d(x), np.float32)
    P, H = x.shape
    F = weights[0][4].shape[0]
    keep = []
    wp = (ctypes.c_void_p * (7 * L))()
    sp = (ctypes.c_void_p * (7 * L))()
    for l in range(L):
        for j in range(7):
            w = _c(weights[l][j], np.int8)
            s = _c(scales[l][j], np.float32)
            keep += [w, s]
            wp[l * 7 + j] = w.ctypes.data
            sp[l * 7 + j] = s.ctypes.data
    y = np.empty((P, H), np.float32)
    proj = np.empty((L, P, 5 * H + 2 * F), np.float32) if return_proj else None
    rc = _load().or_stack(L, H, F, ctypes.cast(wp, ctypes.c_void_p), ctypes.cast(sp, ctypes.c_void_p),
                          _ptr(x), P, _ptr(y), _ptr(proj) if proj is not None else None,
                          threads or default_threads(), int(act))
    _check(rc, "or_stack")
    return (y, proj) if return_proj else y


def stack_attn(weights, scales, x, n_heads: int, return_proj: bool = False,
               threads: int | None = None, act: int = ACT_NONE):
    """The stack with causal attention (n_heads heads), layer by layer over the
    prompt.  Returns (y [P, H], kv [L, 2, P, H]) and, with ``return_proj``, also
    every projection output [L, P, 5H + 2F] (o from the attention)."""
    L = len(weights)
    x = _c(np.atleast_2d(x), np.float32)
    P, H = x.shape
    F = weights[0][4].shape[0]
    keep = []
    wp = (ctypes.c_void_p * (7 * L))()
    sp = (ctypes.c_void_p * (7 * L))()
    for l in range(L):
        for j in range(7):
            w = _c(weights[l][j], np.int8)
            s = _c(scales[l][j], np.float32)
            keep += [w, s]
            wp[l * 7 + j] = w.ctypes.data
            sp[l * 7 + j] = s.ctypes.data
    y = np.empty((P, H), np.float32)
    kv = np.empty((L, 2, P, H), np.float32)
    proj = np.empty((L, P, 5 * H + 2 * F), np.float32) if return_proj else None
    rc = _load().or_stack_attn(L, H, F, n_heads, ctypes.cast(wp, ctypes.c_void_p),
                               ctypes.cast(sp, ctypes.c_void_p), _ptr(x), P, _ptr(y),
                               _ptr(proj) if proj is not None else None, _ptr(kv),
                               threads or default_threads(), int(act))
    _check(rc, "or_stack_attn")
    return (y, kv, proj) if return_proj else (y, kv)


def expf_cr(x, threads: int | None = None) -> np.ndarray:
    """Correctly rounded binary32 exp, elementwise."""
    shape = np.shape(x)
    x = _c(x, np.float32).reshape(-1)
    out = np.empty_like(x)
    _check(_load().or_expf_cr_array(_ptr(x), x.size, _ptr(out), threads or default_threads()),
           "or_expf_cr_array")
    return out.reshape(shape)


def router(Wr, x) -> np.ndarray:
    """Router logits of token rows x [T, H] with Wr [E, H] -> [T, E]."""
    Wr = _c(Wr, np.float32)
    E, H = Wr.shape
    x = _c(np.atleast_2d(x), np.float32)
    out = np.empty((x.shape[0], E), np.float32)
    lib = _load()
    for t in range(x.shape[0]):
        _check(lib.or_router(_ptr(Wr), E, H, _ptr(x[t]), _ptr(out[t])), "or_router")
    return out


def silu(g):
    """silu(g) = g / (1 + expf_cr(-g)), each step rounded to binary32, elementwise."""
    g = np.asarray(g, np.float32)
    lib = _load()
    return np.array([lib.or_silu(float(v)) for v in g.reshape(-1)], np.float32).reshape(g.shape)


def softmax_topk(logits, top_k: int, renorm: bool = False):
    """Per row of logits [T, E]: (ids int32 [T, k], weights f32 [T, k]); renorm:
    weights renormalised over the chosen experts."""
    logits = _c(np.atleast_2d(logits), np.float32)
    T, E = logits.shape
    ids = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k), np.float32)
    lib = _load()
    for t in range(T):
        _check(lib.or_softmax_topk(_ptr(logits[t]), E, top_k, _ptr(ids[t]), _ptr(w[t]),
                                   int(renorm)), "or_softmax_topk")
    return ids, w


def expert(moe: dict, e: int, xq, xs) -> np.ndarray:
    """Expert e applied to one quantised token (xq int8 [H], xs f32); the
    activation is moe.get("activation", ACT_NONE)."""
    H, I = moe["hidden"], moe["inter"]
    y = np.empty(H, np.float32)
    xq = _c(xq, np.int8).reshape(H)
    rc = _load().or_expert(H, I, _ptr(moe["W_gate"]), _ptr(moe["W_up"]), _ptr(moe["W_down"]),
                           _ptr(moe["s_gate"]), _ptr(moe["s_up"]), _ptr(moe["s_down"]), e,
                           _ptr(xq), float(np.float32(xs)), _ptr(y), int(moe.get("activation", 0)))
    _check(rc, "or_expert")
    return y


def moe(moe: dict, x, threads: int | None = None):
    """Mixture-of-experts prefill of x [T, H] -> (ids [T, k], weights [T, k], out [T, H]).

    ``moe`` holds n_experts, top_k, hidden, inter, W_router [E, H] f32,
    W_gate / W_up [E, I, H] int8, W_down [E, H, I] int8, s_gate / s_up [E, I] and
    s_down [E, H] f32 (C-contiguous numpy arrays); optional "activation"
    (ACT_NONE or ACT_SWIGLU) and "renormalize" (0 or 1) select the variants.
    """
    E, k, H, I = moe["n_experts"], moe["top_k"], moe["hidden"], moe["inter"]
    x = _c(np.atleast_2d(x), np.float32)
    T = x.shape[0]
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    out = np.empty((T, H), np.float32)
    arrs = [_c(moe[n], dt) for n, dt in (("W_router", np.float32), ("W_gate", np.int8),
                                          ("W_up", np.int8), ("W_down", np.int8),
                                          ("s_gate", np.float32), ("s_up", np.float32),
                                          ("s_down", np.float32))]
    rc = _load().or_moe(E, k, H, I, *[_ptr(a) for a in arrs], _ptr(x), T, _ptr(ids), _ptr(w),
                        _ptr(out), threads or default_threads(), int(moe.get("activation", 0)),
                        int(moe.get("renormalize", 0)))
    _check(rc, "or_moe")
    return ids, w, out
