"""Seeded synthetic inputs for the hybrid-attention workloads.

Both the CPU oracle and the GPU path consume exactly these arrays; this module
holds none of the method's arithmetic (no pooling, scoring, selection or
attention), only random draws and their rounding to the stated input types.

Every tensor is drawn from its own stream: numpy PCG64 seeded by
SeedSequence([workload seed, crc32(tensor name)]), so any subset can be
regenerated independently.  bf16 tensors are returned as uint16 bit patterns
(round-to-nearest-even from the float32 draw).

Distributions (the workload definitions): Q, K, V, indexer queries and keys
N(0, 1); indexer head weights U(0, 1); compression pooling logits N(0, 0.1^2).
The 128K prefill plants correlated keys: in every 4096-token segment 41 seeded
positions (1%) carry keys at cosine ~0.5 to every query (see `_planted_rows`).
"""
from __future__ import annotations

import math
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Workload

_POOL = ThreadPoolExecutor(max_workers=8)


def rng(seed: int, name: str) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, zlib.crc32(name.encode())])))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, name: str, shape) -> np.ndarray:
    return bf16_bits(rng(seed, name).standard_normal(shape, dtype=np.float32))


def pool_logits(w: Workload, layer: str) -> dict:
    """Per-slot, per-channel pooling logits Z ~ N(0, 0.1^2), float32 [m, dim]."""
    m = w.m(layer)
    out = {
        "zk": (0.1 * rng(w.seed, f"{layer}.zk").standard_normal((m, w.d))).astype(np.float32),
        "zv": (0.1 * rng(w.seed, f"{layer}.zv").standard_normal((m, w.d))).astype(np.float32),
    }
    if layer == "csa":
        out["zi"] = (0.1 * rng(w.seed, f"{layer}.zi").standard_normal((m, w.d_I))).astype(np.float32)
    return out


# ----------------------------------------------------------------------------- planted structure

_RHO = math.sqrt(0.5)
_PLANT_SEG = 4096
_PLANT_PER_SEG = 41            # round(0.01 * 4096)


def _unit(seed, name, dim):
    g = rng(seed, name).standard_normal(dim)
    return g / np.linalg.norm(g)


def _planted_rows(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Rows sqrt(D) * (rho*u + sqrt(1-rho^2)*n), n = g's direction orthogonal to u."""
    D = u.shape[0]
    u = u.astype(np.float32)
    g = np.asarray(g, dtype=np.float32)
    g = g - (g @ u)[:, None] * u[None, :]
    g *= np.float32(math.sqrt(D) * math.sqrt(1 - _RHO ** 2)) / np.linalg.norm(g, axis=1, keepdims=True)
    g += np.float32(math.sqrt(D) * _RHO) * u[None, :]
    return g


def planted_positions(w: Workload, layer: str, T: int) -> np.ndarray:
    r = rng(w.seed, f"{layer}.plant.pos")
    pos = []
    for s0 in range(0, T, _PLANT_SEG):
        n = min(_PLANT_SEG, T - s0)
        cnt = min(n, _PLANT_PER_SEG)
        pos.append(s0 + np.sort(r.choice(n, size=cnt, replace=False)))
    return np.concatenate(pos) if pos else np.zeros(0, np.int64)


# ----------------------------------------------------------------------------- prefill

def _normal_rows(seed, name, T, inner, planted_u=None):
    """N(0,1) rows [T, *inner] as bf16 bits, generated in chunks."""
    n_inner = int(np.prod(inner))
    chunk = max(1, min(1 << 15, (1 << 22) // n_inner))
    out = np.empty((T, n_inner), np.uint16)
    g = rng(seed, name)
    # one stream per tensor: draw sequentially in chunks to bound memory
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        a = g.standard_normal((t1 - t0, n_inner), dtype=np.float32)
        if planted_u is not None:
            D = planted_u.shape[0]
            a = _planted_rows(a.reshape(-1, D), planted_u).reshape(t1 - t0, n_inner)
        out[t0:t1] = bf16_bits(a)
    return out.reshape((T,) + tuple(inner))


def prefill_layer(w: Workload, layer: str, T: int | None = None) -> dict:
    """Inputs of one prefill layer over tokens 0..T-1 (T defaults to the workload's)."""
    T = w.T if T is None else T
    s, H, d = w.seed, w.H, w.d
    u = _unit(s, f"{layer}.plant.u", d) if w.planted else None
    uI = _unit(s, f"{layer}.plant.uI", w.d_I) if w.planted else None
    jobs = {
        "q": _POOL.submit(_normal_rows, s, f"{layer}.q", T, (H, d), planted_u=u),
        "k": _POOL.submit(_normal_rows, s, f"{layer}.k", T, (d,)),
        "v": _POOL.submit(_normal_rows, s, f"{layer}.v", T, (d,)),
    }
    if layer == "csa":
        jobs["qi"] = _POOL.submit(_normal_rows, s, f"{layer}.qi", T, (w.H_I, w.d_I), planted_u=uI)
        jobs["ki"] = _POOL.submit(_normal_rows, s, f"{layer}.ki", T, (w.d_I,))
    out = {k: j.result() for k, j in jobs.items()}
    if layer == "csa":
        out["w"] = rng(s, f"{layer}.w").random((T, w.H_I), dtype=np.float32)
    if w.planted:
        pos = planted_positions(w, layer, T)
        out["planted_pos"] = pos
        rk = rng(s, f"{layer}.plant.k").standard_normal((len(pos), d), dtype=np.float32)
        out["k"][pos] = bf16_bits(_planted_rows(rk, u))
        if layer == "csa":
            ri = rng(s, f"{layer}.plant.ki").standard_normal((len(pos), w.d_I), dtype=np.float32)
            out["ki"][pos] = bf16_bits(_planted_rows(ri, uI))
    out.update(pool_logits(w, layer))
    return out


# ----------------------------------------------------------------------------- decode

def decode_request(w: Workload, layer: str, r: int, L: int | None = None,
                   extra_tokens: int = 1, n_queries: int = 1) -> dict:
    """Token history of request r: positions 0 .. L+extra_tokens-1 (K, V, and KI
    for CSA), and `n_queries` query rows for positions L, L+1, ...

    With the defaults this is one decode step: L cached tokens plus the new
    token at position L, whose query is row 0."""
    L = w.L if L is None else L
    s, H, d = w.seed, w.H, w.d
    n_tok = L + extra_tokens
    jobs = {
        "k": _POOL.submit(_normal_rows, s, f"{layer}.k.{r}", n_tok, (d,)),
        "v": _POOL.submit(_normal_rows, s, f"{layer}.v.{r}", n_tok, (d,)),
        "q": _POOL.submit(_normal_rows, s, f"{layer}.q.{r}", n_queries, (H, d)),
    }
    if layer == "csa":
        jobs["ki"] = _POOL.submit(_normal_rows, s, f"{layer}.ki.{r}", n_tok, (w.d_I,))
        jobs["qi"] = _POOL.submit(_normal_rows, s, f"{layer}.qi.{r}", n_queries, (w.H_I, w.d_I))
    out = {k: j.result() for k, j in jobs.items()}
    if layer == "csa":
        out["w"] = rng(s, f"{layer}.w.{r}").random((n_queries, w.H_I), dtype=np.float32)
    return out


def ragged_lengths(w: Workload) -> np.ndarray:
    """Context lengths log-uniform in [L_min, L_max] (rounded)."""
    u = rng(w.seed, "ragged.lengths").random(w.B)
    lo, hi = math.log(w.L_min), math.log(w.L_max)
    return np.round(np.exp(lo + u * (hi - lo))).astype(np.int64)


def page_permutation(w: Workload, name: str, n_pages: int) -> np.ndarray:
    """A seeded shuffle of a pool of physical pages."""
    return rng(w.seed, f"pages.{name}").permutation(n_pages).astype(np.int32)


def rejected_tokens(w: Workload, layer: str, r: int, n: int) -> dict:
    """n draft tokens of request r that speculative decoding rejects: K, V (and
    KI for CSA) rows from streams of their own, different from the request's
    history at the same positions."""
    s, d = w.seed, w.d
    out = {"k": _normal_rows(s, f"{layer}.rej.k.{r}", n, (d,)),
           "v": _normal_rows(s, f"{layer}.rej.v.{r}", n, (d,))}
    if layer == "csa":
        out["ki"] = _normal_rows(s, f"{layer}.rej.ki.{r}", n, (w.d_I,))
    return out
