"""Python binding of libprefill (include/libprefill.h).

Argument marshalling only: every step of the prefill path runs in the HIP
kernels of ``libprefill.so``; PyTorch supplies device memory and the stream.
The names mirror the C entry points without their ``pf_`` prefix.

The library is loaded from this directory (build it with
``python int8_weight_gemm_amd/build.py`` or ``__graft_entry__.build()``); if it
is missing, importing works but every call raises ``LibraryMissing``.  There is
no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libprefill.so")

PF_OK, PF_EINVAL, PF_ENODEV, PF_ELAUNCH, PF_EWORKSPACE, PF_EINTERNAL = 0, -1, -2, -3, -4, -5
NPROJ = 7
NOALLOC_SCRATCH_BYTES = 64 << 20     # PF_NOALLOC_SCRATCH_BYTES
ACT_NONE, ACT_SWIGLU = 0, 1          # PF_ACT_NONE, PF_ACT_SWIGLU
PROJ_NAMES = ("q", "k", "v", "o", "gate", "up", "down")


class LibraryMissing(RuntimeError):
    pass


class PrefillError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} ({status})")


class _Layer(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p * NPROJ), ("w_scale", ctypes.c_void_p * NPROJ)]


class _Stack(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int64), ("hidden", ctypes.c_int64), ("ffn", ctypes.c_int64),
                ("layers", ctypes.POINTER(_Layer)), ("layers_alt", ctypes.POINTER(_Layer)),
                ("activation", ctypes.c_int64), ("n_heads", ctypes.c_int64)]


class StackStats(ctypes.Structure):
    _fields_ = [("time_kernels", ctypes.c_int), ("max_groups", ctypes.c_int),
                ("groups", ctypes.c_int), ("per_token_mode", ctypes.c_int),
                ("chunks", ctypes.c_int64), ("tail_tokens", ctypes.c_int64),
                ("launches", ctypes.c_int64), ("alg_bytes", ctypes.c_double),
                ("elapsed_ms", ctypes.c_double), ("product_launches", ctypes.c_int64),
                ("quant_launches", ctypes.c_int64), ("product_alg_bytes", ctypes.c_double),
                ("quant_alg_bytes", ctypes.c_double), ("product_ms", ctypes.c_double),
                ("quant_ms", ctypes.c_double), ("product_busy_ms", ctypes.c_double),
                ("quant_busy_ms", ctypes.c_double), ("overhead_bytes", ctypes.c_double),
                ("attn_launches", ctypes.c_int64), ("attn_alg_bytes", ctypes.c_double),
                ("attn_ms", ctypes.c_double)]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


class StreamStats(ctypes.Structure):
    _fields_ = [("n_buffers", ctypes.c_int64), ("layers_copied", ctypes.c_int64),
                ("prefetch_hits", ctypes.c_int64), ("prefetch_misses", ctypes.c_int64),
                ("bytes_copied", ctypes.c_double), ("elapsed_ms", ctypes.c_double)]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


class _Moe(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int64), ("top_k", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("inter", ctypes.c_int64), ("W_router", ctypes.c_void_p), ("W_gate", ctypes.c_void_p),
                ("W_up", ctypes.c_void_p), ("W_down", ctypes.c_void_p), ("s_gate", ctypes.c_void_p),
                ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
                ("activation", ctypes.c_int64), ("renormalize", ctypes.c_int64)]


_lib = None

_P, _I64, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "pf_init": ([], ctypes.c_int),
    "pf_workspace_clear": ([_P, _SZ, _P], ctypes.c_int),
    "pf_quantize_act": ([_P, _I64, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "pf_gemm_i8_chunk_workspace": ([_I64, _I64, _I64], _SZ),
    "pf_gemm_i8_chunk": ([_P, _P, _I64, _I64, _P, _P, _I64, _P, _P, _SZ, _P], ctypes.c_int),
    "pf_gemm_i8_chunk_noalloc": ([_P, _P, _I64, _I64, _P, _P, _I64, _P, _P], ctypes.c_int),
    "pf_gemv_i8": ([_P, _P, _I64, _I64, _P, _P, _P, _P], ctypes.c_int),
    "pf_prefill_stack_workspace": ([ctypes.POINTER(_Stack), _I64], _SZ),
    "pf_prefill_stack": ([ctypes.POINTER(_Stack), _P, _I64, _I64, _P, _P, _P, _P, _SZ,
                          ctypes.POINTER(StackStats), _P], ctypes.c_int),
    "pf_prefill_stack_streamed_workspace": ([ctypes.POINTER(_Stack), _I64, _I64], _SZ),
    "pf_prefill_stack_streamed": ([ctypes.POINTER(_Stack), _P, _I64, _I64, _P, _I64, _P, _SZ,
                                   ctypes.POINTER(StreamStats), _P], ctypes.c_int),
    "pf_moe_chunk_workspace": ([ctypes.POINTER(_Moe), _I64], _SZ),
    "pf_moe_chunk": ([ctypes.POINTER(_Moe), _P, _I64, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "pf_expf_cr": ([_P, _I64, _P, _P], ctypes.c_int),
    "pf_status_string": ([ctypes.c_int], ctypes.c_char_p),
}


def lib() -> ctypes.CDLL:
    """The loaded libprefill.so (raises LibraryMissing if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(f"{LIB_PATH} is not built; run int8_weight_gemm_amd/build.py")
        h = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = res
        _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().pf_status_string(status).decode()


def _check(fn: str, status: int):
    if status != PF_OK:
        raise PrefillError(fn, status)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dev(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def init() -> None:
    _check("pf_init", lib().pf_init())


def workspace(nbytes: int, device=None) -> torch.Tensor:
    """A zero-filled workspace of nbytes (at least 16) on the current device."""
    return torch.zeros(max(16, int(nbytes)), dtype=torch.uint8, device=device or "cuda")


def workspace_clear(ws: torch.Tensor) -> None:
    _check("pf_workspace_clear", lib().pf_workspace_clear(_ptr(ws), ws.numel(), _stream()))


def quantize_act(x: torch.Tensor, out: tuple | None = None):
    """x f32 [M, K] -> (xq int8 [M, K], a_scale f32 [M])."""
    _dev(x, torch.float32, "x")
    M, K = x.shape
    xq, s = out if out is not None else (torch.empty((M, K), dtype=torch.int8, device=x.device),
                                         torch.empty(M, dtype=torch.float32, device=x.device))
    _check("pf_quantize_act", lib().pf_quantize_act(_ptr(x), M, K, K, _ptr(xq), _ptr(s), _stream()))
    return xq, s


def gemm_i8_chunk_workspace(N: int, K: int, M: int) -> int:
    return int(lib().pf_gemm_i8_chunk_workspace(N, K, M))


def gemm_i8_chunk(W, w_scale, xq, a_scale, ws: torch.Tensor | None = None,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """y f32 [M, N] = int8 product of W [N, K] with the chunk xq [M, K]."""
    _dev(W, torch.int8, "W"); _dev(w_scale, torch.float32, "w_scale")
    _dev(xq, torch.int8, "xq"); _dev(a_scale, torch.float32, "a_scale")
    N, K = W.shape
    M = xq.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=W.device)
    _check("pf_gemm_i8_chunk", lib().pf_gemm_i8_chunk(
        _ptr(W), _ptr(w_scale), N, K, _ptr(xq), _ptr(a_scale), M, _ptr(y),
        _ptr(ws), ws.numel() if ws is not None else 0, _stream()))
    return y


def gemm_i8_chunk_noalloc(W, w_scale, xq, a_scale, out: torch.Tensor | None = None) -> torch.Tensor:
    """gemm_i8_chunk with the split partials in the library's own device array
    (no workspace; out must be given to avoid any allocation here)."""
    _dev(W, torch.int8, "W"); _dev(w_scale, torch.float32, "w_scale")
    _dev(xq, torch.int8, "xq"); _dev(a_scale, torch.float32, "a_scale")
    N, K = W.shape
    M = xq.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=W.device)
    _check("pf_gemm_i8_chunk_noalloc", lib().pf_gemm_i8_chunk_noalloc(
        _ptr(W), _ptr(w_scale), N, K, _ptr(xq), _ptr(a_scale), M, _ptr(y), _stream()))
    return y


def gemv_i8(W, w_scale, xq, a_scale, out: torch.Tensor | None = None) -> torch.Tensor:
    """y f32 [N] for one quantised token xq [K] with scale a_scale [1]."""
    _dev(W, torch.int8, "W"); _dev(w_scale, torch.float32, "w_scale")
    _dev(xq, torch.int8, "xq"); _dev(a_scale, torch.float32, "a_scale")
    N, K = W.shape
    y = out if out is not None else torch.empty(N, dtype=torch.float32, device=W.device)
    _check("pf_gemv_i8", lib().pf_gemv_i8(_ptr(W), _ptr(w_scale), N, K, _ptr(xq), _ptr(a_scale),
                                         _ptr(y), _stream()))
    return y


def expf_cr(x: torch.Tensor) -> torch.Tensor:
    _dev(x, torch.float32, "x")
    y = torch.empty_like(x)
    _check("pf_expf_cr", lib().pf_expf_cr(_ptr(x), x.numel(), _ptr(y), _stream()))
    return y


class Stack:
    """A projection stack resident in HBM: weights[l] = 7 int8 tensors (q, k, v, o,
    gate, up, down), scales[l] = 7 f32 tensors.  ``alt``, optional, is a second
    (weights, scales) copy of the same values that odd chunks read (pf_stack's
    layers_alt); activation: ACT_NONE or ACT_SWIGLU (pf_stack's activation);
    n_heads > 0: causal attention over a K/V cache (pf_stack's n_heads)."""

    def __init__(self, weights, scales, alt=None, activation: int = ACT_NONE, n_heads: int = 0):
        self.L = len(weights)
        self.H = weights[0][0].shape[1]
        self.F = weights[0][4].shape[0]
        self.weights, self.scales, self.alt = weights, scales, alt
        self._layers = self._table(weights, scales)
        self._alt = self._table(*alt) if alt is not None else None
        self._desc = _Stack(self.L, self.H, self.F, ctypes.cast(self._layers, ctypes.POINTER(_Layer)),
                            ctypes.cast(self._alt, ctypes.POINTER(_Layer)) if self._alt is not None
                            else None, int(activation), int(n_heads))
        self.n_heads = int(n_heads)

    def _table(self, weights, scales):
        tab = (_Layer * self.L)()
        for l in range(self.L):
            for j in range(NPROJ):
                _dev(weights[l][j], torch.int8, f"W[{l}][{j}]")
                _dev(scales[l][j], torch.float32, f"w_scale[{l}][{j}]")
                tab[l].W[j] = weights[l][j].data_ptr()
                tab[l].w_scale[j] = scales[l][j].data_ptr()
        return tab

    @property
    def weight_bytes(self) -> int:
        return sum(w.numel() for wl in self.weights for w in wl)

    def workspace_bytes(self, chunk: int) -> int:
        return int(lib().pf_prefill_stack_workspace(ctypes.byref(self._desc), chunk))

    def prefill(self, x: torch.Tensor, chunk: int, ws: torch.Tensor, y: torch.Tensor | None = None,
                proj: torch.Tensor | None = None, stats: bool = False, time_kernels: bool = False,
                kv: torch.Tensor | None = None, max_groups: int = 0):
        """x f32 [P, H] -> y f32 [P, H]; proj (optional) f32 [L, P, 5H + 2F]; kv,
        the K/V cache f32 [L, 2, P, H], required with n_heads > 0.  With stats
        (or time_kernels) also returns the call's statistics."""
        stats = stats or time_kernels or max_groups > 0
        _dev(x, torch.float32, "x")
        P = x.shape[0]
        if y is None:
            y = torch.empty((P, self.H), dtype=torch.float32, device=x.device)
        st = StackStats() if stats else None
        if st is not None:
            st.time_kernels = 1 if time_kernels else 0
            st.max_groups = int(max_groups)
        _check("pf_prefill_stack", lib().pf_prefill_stack(
            ctypes.byref(self._desc), _ptr(x), P, chunk, _ptr(y), _ptr(proj), _ptr(kv), _ptr(ws), ws.numel(),
            ctypes.byref(st) if st is not None else None, _stream()))
        return (y, st.as_dict()) if stats else y


class HostStack:
    """A projection stack whose weights stay in host memory (CPU tensors, pinned
    so that the copies run asynchronously), streamed layer by layer through a
    device ring by pf_prefill_stack_streamed."""

    def __init__(self, weights, scales, activation: int = ACT_NONE):
        self.L = len(weights)
        self.H = weights[0][0].shape[1]
        self.F = weights[0][4].shape[0]
        self.weights, self.scales = weights, scales
        self._layers = (_Layer * self.L)()
        for l in range(self.L):
            for j in range(NPROJ):
                for t, dt, n in ((weights[l][j], torch.int8, "W"), (scales[l][j], torch.float32, "w_scale")):
                    if t.is_cuda or t.dtype != dt or not t.is_contiguous():
                        raise TypeError(f"{n}[{l}][{j}] must be a contiguous host {dt} tensor")
                self._layers[l].W[j] = weights[l][j].data_ptr()
                self._layers[l].w_scale[j] = scales[l][j].data_ptr()
        self._desc = _Stack(self.L, self.H, self.F, ctypes.cast(self._layers, ctypes.POINTER(_Layer)),
                            None, int(activation), 0)

    def workspace_bytes(self, P: int, n_buffers: int = 2) -> int:
        return int(lib().pf_prefill_stack_streamed_workspace(ctypes.byref(self._desc), P, n_buffers))

    def prefill(self, x: torch.Tensor, chunk: int, ws: torch.Tensor, n_buffers: int = 2,
                y: torch.Tensor | None = None, stats: bool = False):
        """x f32 [P, H] on the device -> y f32 [P, H]; with stats also the ring's
        counters (the call then synchronises)."""
        _dev(x, torch.float32, "x")
        P = x.shape[0]
        if y is None:
            y = torch.empty((P, self.H), dtype=torch.float32, device=x.device)
        st = StreamStats() if stats else None
        _check("pf_prefill_stack_streamed", lib().pf_prefill_stack_streamed(
            ctypes.byref(self._desc), _ptr(x), P, chunk, _ptr(y), n_buffers, _ptr(ws), ws.numel(),
            ctypes.byref(st) if st is not None else None, _stream()))
        return (y, st.as_dict()) if stats else y


class Moe:
    """Mixture-of-experts layer resident in HBM (tensors as in pf_moe)."""

    def __init__(self, n_experts, top_k, W_router, W_gate, W_up, W_down, s_gate, s_up, s_down,
                 activation: int = ACT_NONE, renormalize: int = 0):
        E, I, H = W_gate.shape
        for n, t, dt in (("W_router", W_router, torch.float32), ("W_gate", W_gate, torch.int8),
                         ("W_up", W_up, torch.int8), ("W_down", W_down, torch.int8),
                         ("s_gate", s_gate, torch.float32), ("s_up", s_up, torch.float32),
                         ("s_down", s_down, torch.float32)):
            _dev(t, dt, n)
        self.E, self.k, self.H, self.I = n_experts, top_k, H, I
        self.tensors = (W_router, W_gate, W_up, W_down, s_gate, s_up, s_down)
        self._desc = _Moe(n_experts, top_k, H, I, *[t.data_ptr() for t in self.tensors],
                          int(activation), int(renormalize))

    @property
    def expert_weight_bytes(self) -> int:
        return sum(t.numel() for t in self.tensors[1:4])

    def workspace_bytes(self, T: int) -> int:
        return int(lib().pf_moe_chunk_workspace(ctypes.byref(self._desc), T))

    def chunk(self, x: torch.Tensor, ws: torch.Tensor, out=None):
        """x f32 [T, H] -> (ids int32 [T, k], weights f32 [T, k], out f32 [T, H])."""
        _dev(x, torch.float32, "x")
        T = x.shape[0]
        ids, w, o = out if out is not None else (
            torch.empty((T, self.k), dtype=torch.int32, device=x.device),
            torch.empty((T, self.k), dtype=torch.float32, device=x.device),
            torch.empty((T, self.H), dtype=torch.float32, device=x.device))
        _check("pf_moe_chunk", lib().pf_moe_chunk(ctypes.byref(self._desc), _ptr(x), T, _ptr(ids),
                                                  _ptr(w), _ptr(o), _ptr(ws), ws.numel(), _stream()))
        return ids, w, o
