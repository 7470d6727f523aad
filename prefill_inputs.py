"""Seeded synthetic inputs for the batched int8 prefill path.

This module holds no arithmetic of the method: it only draws random numbers.
Both the oracle (via the tests) and the GPU library consume what it produces;
neither side imports the other.

The pages' own models and prompts are not available, so inputs of their shapes
stand in for them ("Batched Prefill", §The Problem and §Results: a 350M model,
a 747-token prompt, 32-token chunks; "Red Lite dev24": 512 experts, top-10,
512-token chunks).  Every generator uses numpy's PCG64 with a fixed seed and
one independent sub-stream per (layer, projection) via SeedSequence.spawn, so
the same call always returns the same bytes.

Value recipes:
  * weights: int8 uniform on [-127, 127];
  * single-projection and expert scales: f32 uniform on [0.001, 0.01];
  * stack scales: u / (74 * sqrt(K)) with u uniform on [0.5, 1.5], which keeps
    the per-layer gain near one so that a 16- or 32-layer chain stays finite
    (74 ~ the RMS of a uniform int8 weight);
  * activations: f32 standard normal;
  * router weight: f32 standard normal / sqrt(hidden).
"""
from __future__ import annotations

import math

import numpy as np

PROJ_NAMES = ("q", "k", "v", "o", "gate", "up", "down")

# Named workloads (sizes only).
WORKLOADS = {
    "proj1024": dict(kind="projection", N=1024, K=1024, M=32, chunk=32, seed=1001),
    "stack350m": dict(kind="stack", L=16, H=1024, F=4096, P=747, chunk=32, seed=1002),
    "sweep4096": dict(kind="projection", N=4096, K=4096, M=512,
                      chunks=(1, 8, 16, 32, 64, 128, 256, 512), seed=1003),
    "stack7b": dict(kind="stack", L=32, H=4096, F=11008, P=2048, chunk=512, seed=1004),
    "moe512": dict(kind="moe", E=512, top_k=10, H=2048, I=512, T=512, seed=1005),
}


def _rngs(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def int8_weight(rng, shape) -> np.ndarray:
    return rng.integers(-127, 128, size=shape, dtype=np.int8)


def uniform_scale(rng, n, lo=0.001, hi=0.01) -> np.ndarray:
    return rng.uniform(lo, hi, size=n).astype(np.float32)


def normalised_scale(rng, n, K) -> np.ndarray:
    u = rng.uniform(0.5, 1.5, size=n)
    return (u / (74.0 * math.sqrt(K))).astype(np.float32)


def activations(rng, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def projection(N: int, K: int, M: int, seed: int) -> dict:
    """One projection: W int8 [N, K], w_scale f32 [N], x f32 [M, K]."""
    rw, rs, rx = _rngs(seed, 3)
    return dict(W=int8_weight(rw, (N, K)), w_scale=uniform_scale(rs, N),
                x=activations(rx, (M, K)))


def stack(L: int, H: int, F: int, P: int, seed: int) -> dict:
    """A projection stack: weights[l] = [q, k, v, o, gate, up, down] int8,
    scales[l] the per-row f32 scales, x f32 [P, H]."""
    rngs = _rngs(seed, 2 * 7 * L + 1)
    shapes = [(H, H), (H, H), (H, H), (H, H), (F, H), (F, H), (H, F)]
    weights, scales = [], []
    for l in range(L):
        wl, sl = [], []
        for j, (n, k) in enumerate(shapes):
            wl.append(int8_weight(rngs[2 * (7 * l + j)], (n, k)))
            sl.append(normalised_scale(rngs[2 * (7 * l + j) + 1], n, k))
        weights.append(wl)
        scales.append(sl)
    return dict(L=L, H=H, F=F, weights=weights, scales=scales, x=activations(rngs[-1], (P, H)))


def moe(E: int, top_k: int, H: int, I: int, T: int, seed: int) -> dict:
    """Experts with gate/up [I, H] and down [H, I] in int8 plus an f32 router."""
    r = _rngs(seed, 8)
    Wr = (r[0].standard_normal(size=(E, H), dtype=np.float32) / np.float32(math.sqrt(H)))
    return dict(n_experts=E, top_k=top_k, hidden=H, inter=I,
                W_router=Wr.astype(np.float32),
                W_gate=int8_weight(r[1], (E, I, H)), W_up=int8_weight(r[2], (E, I, H)),
                W_down=int8_weight(r[3], (E, H, I)),
                s_gate=uniform_scale(r[4], (E, I)), s_up=uniform_scale(r[5], (E, I)),
                s_down=uniform_scale(r[6], (E, H)),
                x=activations(r[7], (T, H)))


def workload(name: str) -> dict:
    """Inputs of a named workload at full size."""
    w = WORKLOADS[name]
    if w["kind"] == "projection":
        return projection(w["N"], w["K"], w["M"], w["seed"])
    if w["kind"] == "stack":
        return stack(w["L"], w["H"], w["F"], w["P"], w["seed"])
    return moe(w["E"], w["top_k"], w["H"], w["I"], w["T"], w["seed"])
