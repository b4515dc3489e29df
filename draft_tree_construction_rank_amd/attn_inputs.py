"""Seeded synthetic inputs for one tree-attention layer (input synthesis only).

The module draws random numbers, random rooted trees and rounds values to bfloat16.  It
holds none of the attention arithmetic (no scores, softmax or visibility rule); the oracle
under ``oracle/`` and the HIP library consume the same arrays.

Shapes follow the pages' target models (PCTree summary, setup paragraph: the Qwen3 family,
4B/8B/14B, verified in bfloat16): 128-wide heads with grouped keys and values, 32 query
heads over 8 key/value heads (Qwen3-4B and -8B) or 40 over 8 (Qwen3-14B); trees of up to
N = 64 nodes (N = 32 at B = 7).  The pages' prompts (math, code, chat benchmarks) are not
available; context lengths are drawn uniformly from a range instead (default 512..2048).

Value laws: Q, K, V entries N(0, 1) drawn in float32 and rounded once to bfloat16 (round to
nearest even), Q multiplied by ``qscale`` first, so that attention scores at the usual
1/sqrt(D) scale have standard deviation about ``qscale``.  Trees: node i's parent is
uniform over the root (-1) and nodes 0..i-1 ("random"), or parent[i] = i - 1 ("chain"), or
every node a child of the root ("star"); n_nodes per request is Ncap ("full") or uniform
over 0..Ncap ("ragged").  Cache slots past a request's tree hold the same law's values.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = ["AttnInstance", "make_attn_instance", "bf16_bits", "bits_to_f32"]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even; finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the float32 values they hold (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class AttnInstance:
    R: int
    Hq: int
    Hkv: int
    D: int
    Ncap: int
    Cmax: int
    scale: float
    Q: np.ndarray        # uint16 bf16 bits [R][Hq][Ncap+1][D]
    K: np.ndarray        # uint16 bf16 bits [R][Hkv][Cmax][D]
    V: np.ndarray        # uint16 bf16 bits [R][Hkv][Cmax][D]
    ctx_len: np.ndarray  # int32 [R]
    n_nodes: np.ndarray  # int32 [R]
    parent: np.ndarray   # int32 [R][Ncap] (-1 = the root, -2 = no node)

    def f32(self, name: str) -> np.ndarray:
        return bits_to_f32(getattr(self, name))


def _tree(rng: np.random.Generator, n: int, Ncap: int, shape: str) -> np.ndarray:
    par = np.full(Ncap, -2, np.int32)
    for i in range(n):
        if shape == "chain":
            par[i] = i - 1
        elif shape == "star":
            par[i] = -1
        elif shape == "random":
            par[i] = int(rng.integers(-1, i)) if i > 0 else -1
        else:
            raise ValueError(shape)
    return par


def make_attn_instance(*, seed: int, R: int, Hq: int = 32, Hkv: int = 8, D: int = 128,
                       Ncap: int = 64, ctx_lo: int = 512, ctx_hi: int = 2048,
                       Cmax: int | None = None, tree: str = "random", nodes: str = "full",
                       qscale: float = 1.0, threads: int = 8) -> AttnInstance:
    """R requests; request r draws from numpy Generator([seed, 21, r])."""
    if Cmax is None:
        Cmax = ctx_hi + Ncap + 1
    Q = np.empty((R, Hq, Ncap + 1, D), np.uint16)
    K = np.empty((R, Hkv, Cmax, D), np.uint16)
    V = np.empty((R, Hkv, Cmax, D), np.uint16)
    ctx = np.empty(R, np.int32)
    nn = np.empty(R, np.int32)
    par = np.empty((R, Ncap), np.int32)

    def one(r):
        rng = np.random.default_rng([seed, 21, r])
        ctx[r] = int(rng.integers(ctx_lo, ctx_hi + 1))
        nn[r] = Ncap if nodes == "full" else int(rng.integers(0, Ncap + 1))
        par[r] = _tree(rng, int(nn[r]), Ncap, tree)
        Q[r] = bf16_bits(rng.standard_normal((Hq, Ncap + 1, D), dtype=np.float32) *
                         np.float32(qscale))
        K[r] = bf16_bits(rng.standard_normal((Hkv, Cmax, D), dtype=np.float32))
        V[r] = bf16_bits(rng.standard_normal((Hkv, Cmax, D), dtype=np.float32))

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(one, range(R)))
    return AttnInstance(R=R, Hq=Hq, Hkv=Hkv, D=D, Ncap=Ncap, Cmax=Cmax,
                        scale=1.0 / math.sqrt(D), Q=Q, K=K, V=V, ctx_len=ctx, n_nodes=nn,
                        parent=par)
