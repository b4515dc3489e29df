"""Seeded synthetic inputs for draft-tree construction and verification.

This module only draws random numbers and rounds them to the storage dtype.  It holds
none of the method's arithmetic (no Markov bias, no softmax, no ranking, no survival):
the oracle under ``oracle/`` and the HIP library both consume the arrays it returns,
byte for byte.

Workload shapes and value laws (the pages give shapes, not logit statistics):

* PCTree summary (From Chains to Trees, setup paragraph): block sizes B = 7 and 16,
  k = 4 children, budget N = 32 (64 at B = 16); the Qwen3 vocabulary, V = 151936.
* Block logits: N(0, sd=2) per entry, plus planted peaks.  ``tiny``: one uniformly chosen
  token per position gets +6.  The large configs plant 8 distinct tokens per position whose
  vocabulary ranks are drawn from a Zipf(1.1) law (rank -> id through a fixed seeded
  permutation), with boosts spaced linearly from +9 (first draw) down to +4 (eighth).  The
  batched config scales the boosts per request by a strength s ~ U(2, 9): s down to s*4/9.
* Markov head: U, W ~ N(0, sd=r**-0.5), i.e. a bias U[p].W[:, c] of sd r**-0.5.  W is stored
  transposed, as ``Wt[V][r]``, so both tables are row-per-token.  The "strong head"
  companion uses sd r**-0.25 (bias sd 1) so that parent conditioning visibly changes trees.
* Calibration tables: ``linear`` = bin centres (i + 0.5)/16; ``monotone`` = 16 sorted
  U(0.05, 0.95) draws.
* Target rows for verification: row(v) = rho * Lext[d_v] + sqrt(1 - rho^2) * E(v), where
  Lext[d] is the drafter's block-logit row for the position that node v predicts (an extra
  row d = B is drawn for nodes at the last block position) and E(v) is a fresh draw from the
  same block-logit law keyed by (seed, request, the node's token path).  rho = 0 gives
  i.i.d. rows.  A node's row depends only on its path, so the synthetic target is one fixed
  model whatever tree is built.

All draws are made in float64 and rounded once (round-to-nearest-even) to the storage dtype.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Sequence

import numpy as np

__all__ = [
    "Instance",
    "round_bf16",
    "make_instance",
    "target_rows",
    "target_for_tree",
    "make_tie_instance",
    "CONFIGS",
]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float32.

    bfloat16 keeps 8 significant bits.  frexp gives x = m * 2**e with 0.5 <= |m| < 1, so
    m * 256 rounded half-to-even (np.rint) is the 8-bit significand.  Values are rounded
    once from float64 (no float32 intermediate).  The result is exactly representable in
    float32 and in bfloat16.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    y = np.ldexp(np.rint(m * 256.0), e - 8)
    return y.astype(np.float32)


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


@dataclasses.dataclass
class Instance:
    """One round's inputs for R requests (all arrays host numpy, float32-held values)."""

    name: str
    R: int
    B: int
    k: int
    V: int
    r: int
    Ncap: int
    dtype: str  # storage dtype of logits and head: "bf16" | "f32"
    mode: str  # "greedy" | "sample"
    temperature: float
    cal: np.ndarray  # [16] float32
    seed: int
    round: int
    Lext: np.ndarray  # [R][B+1][V] float32 (values representable in dtype)
    U: np.ndarray  # [V][r]
    Wt: np.ndarray  # [V][r]
    root_token: np.ndarray  # [R] int32
    n_budget: np.ndarray  # [R] int32
    tau: np.ndarray  # [R] float32
    rho: float  # target correlation
    peak: str  # "one6" | "zipf8"
    target_peak: str  # peak law of the target's fresh draws E(v)
    strength: np.ndarray  # [R] float64 peak strength per request (boost of rank 1)
    subseed: np.ndarray  # [R] int64: per-request sub-seed used for the block logits
    cond: int = 0  # whose head row biases an expansion: 0 parent, 1 greedy chain, 2 none

    @property
    def L(self) -> np.ndarray:
        """Block logits [R][B][V] (the rows the drafter emitted for this block)."""
        return self.Lext[:, : self.B, :]


def _zipf_planted(rng: np.random.Generator, V: int, n: int, perm: np.ndarray) -> np.ndarray:
    ranks = np.arange(1, V + 1, dtype=np.float64)
    w = ranks ** -1.1
    w /= w.sum()
    pick = rng.choice(V, size=n, replace=False, p=w)  # 0-based ranks, first = rank-1 slot
    return perm[pick]


def _block_rows(rng: np.random.Generator, nrows: int, V: int, peak: str, strength: float,
                perm: np.ndarray | None) -> np.ndarray:
    """float64 [nrows][V]: N(0, 2) plus planted peaks (see module docstring)."""
    x = rng.normal(0.0, 2.0, size=(nrows, V))
    for i in range(nrows):
        if peak == "one6":
            x[i, rng.integers(0, V)] += 6.0
        elif peak == "zipf8":
            ids = _zipf_planted(rng, V, 8, perm)
            boosts = np.linspace(strength, strength * 4.0 / 9.0, 8)
            x[i, ids] += boosts
        elif peak == "none":
            pass
        else:
            raise ValueError(peak)
    return x


# Workload presets.  Names describe the workload; "headline" is B=16, k=4, N=64.
CONFIGS = {
    # V=64, B=4, k=2, N=8, r=8, fp32, linear table, i.i.d. N(0,2) targets, seed 0.
    "tiny": dict(R=1, B=4, k=2, V=64, r=8, Ncap=8, dtype="f32", mode="greedy", temperature=1.0,
                 cal="linear", peak="one6", target_peak="none", rho=0.0, tau=0.0, seed=0),
    # B=7, k=4, N=32, V=151936, r=256, bf16, monotone table, targets at rho=0.8.
    "b7": dict(R=1, B=7, k=4, V=151936, r=256, Ncap=32, dtype="bf16", mode="greedy",
               temperature=1.0, cal="monotone", peak="zipf8", rho=0.8, tau=0.0, seed=1),
    # B=16, N=64 (headline k=4); the k x N sweep overrides k and Ncap.
    "b16": dict(R=1, B=16, k=4, V=151936, r=256, Ncap=64, dtype="bf16", mode="greedy",
                temperature=1.0, cal="monotone", peak="zipf8", rho=0.8, tau=0.0, seed=2),
    # 64 concurrent requests, per-request peak strength U(2, 9), threshold tau.
    "batched": dict(R=64, B=16, k=4, V=151936, r=256, Ncap=64, dtype="bf16", mode="greedy",
                    temperature=1.0, cal="monotone", peak="zipf8", rho=0.8, tau=0.2, seed=3,
                    strength="uniform"),
    # Lossless sampling: 32 requests, B=16, k=4, N=64, targets at rho=0.7.
    "sample": dict(R=32, B=16, k=4, V=151936, r=256, Ncap=64, dtype="bf16", mode="sample",
                   temperature=1.0, cal="monotone", peak="zipf8", rho=0.7, tau=0.0, seed=4),
}


def make_instance(name: str, *, strong_head: bool = False, request_subseeds=None,
                  **overrides) -> Instance:
    """Build a seeded instance from a preset, with optional field overrides.

    ``request_subseeds`` (length R) replaces the per-request sub-seed of the block logits,
    so a single request can be re-drawn without touching the others.
    """
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    R, B, k, V, r = cfg["R"], cfg["B"], cfg["k"], cfg["V"], cfg["r"]
    seed = int(cfg["seed"])
    dtype = cfg["dtype"]

    head_rng = np.random.default_rng([seed, 1])
    sd = r ** -0.25 if strong_head else r ** -0.5
    U = _round(head_rng.normal(0.0, sd, size=(V, r)), dtype)
    Wt = _round(head_rng.normal(0.0, sd, size=(V, r)), dtype)

    cal_kind = cfg["cal"]
    if isinstance(cal_kind, str) and cal_kind == "linear":
        cal = ((np.arange(16) + 0.5) / 16.0).astype(np.float32)
    elif isinstance(cal_kind, str) and cal_kind == "monotone":
        crng = np.random.default_rng([seed, 2])
        cal = np.sort(crng.uniform(0.05, 0.95, size=16)).astype(np.float32)
    elif isinstance(cal_kind, str) and cal_kind.startswith("const:"):
        cal = np.full(16, float(cal_kind[6:]), dtype=np.float32)
    else:
        cal = np.asarray(cal_kind, dtype=np.float32)
        assert cal.shape == (16,)

    perm = np.random.default_rng([seed, 3]).permutation(V) if cfg["peak"] == "zipf8" else None
    srng = np.random.default_rng([seed, 4])
    if cfg.get("strength") == "uniform":
        strength = srng.uniform(2.0, 9.0, size=R)
    else:
        strength = np.full(R, 9.0)
    roots = srng.integers(0, V, size=R).astype(np.int32)

    subseed = np.arange(R, dtype=np.int64) if request_subseeds is None else \
        np.asarray(request_subseeds, dtype=np.int64)
    Lext = np.empty((R, B + 1, V), dtype=np.float32)
    for i in range(R):
        lrng = np.random.default_rng([seed, 5, int(subseed[i])])
        Lext[i] = _round(_block_rows(lrng, B + 1, V, cfg["peak"], float(strength[i]), perm), dtype)

    n_budget = np.full(R, int(cfg["Ncap"]), dtype=np.int32)
    if "n_budget" in cfg:
        n_budget[:] = cfg["n_budget"]
    tau = np.full(R, float(cfg["tau"]), dtype=np.float32)
    return Instance(name=name, R=R, B=B, k=k, V=V, r=r, Ncap=int(cfg["Ncap"]), dtype=dtype,
                    mode=cfg["mode"], temperature=float(cfg["temperature"]), cal=cal,
                    seed=seed, round=int(cfg.get("round", 0)), Lext=Lext, U=U, Wt=Wt,
                    root_token=roots, n_budget=n_budget, tau=tau, rho=float(cfg["rho"]),
                    peak=cfg["peak"], target_peak=cfg.get("target_peak", cfg["peak"]),
                    strength=strength, subseed=subseed)


def target_rows(inst: Instance, req: int, paths: Sequence[Sequence[int]]) -> np.ndarray:
    """Target logit rows for the given token paths of request ``req`` (float32 [n][V]).

    A path is the tuple of draft tokens from the root's child down to the node (the empty
    tuple is the root).  The row for a node at depth d is rho * Lext[req][d] plus
    sqrt(1 - rho^2) times a fresh block-logit draw keyed by (seed, req, path).
    """
    V = inst.V
    out = np.empty((len(paths), V), dtype=np.float32)
    perm = np.random.default_rng([inst.seed, 3]).permutation(V) \
        if inst.target_peak == "zipf8" else None
    a = inst.rho
    b = math.sqrt(max(0.0, 1.0 - a * a))
    for i, path in enumerate(paths):
        d = len(path)
        rng = np.random.default_rng([inst.seed, 6, int(inst.subseed[req]), d,
                                     *[int(t) + 1 for t in path]])
        e = _block_rows(rng, 1, V, inst.target_peak, float(inst.strength[req]), perm)[0]
        row = a * inst.Lext[req, d].astype(np.float64) + b * e
        out[i] = _round(row, inst.dtype)
    return out


def target_for_tree(inst: Instance, token: np.ndarray, parent: np.ndarray,
                    n_nodes: np.ndarray, Ncap: int | None = None) -> np.ndarray:
    """Target logits [R][Ncap+1][V] for emitted trees: row 0 = root, row i+1 = node i.

    ``token``/``parent`` are the emitted tree arrays ([R][Ncap], parent -1 = root).  Rows of
    empty slots are filled with the root's row (they are never read by a verifier).
    """
    Ncap = inst.Ncap if Ncap is None else Ncap
    out = np.empty((inst.R, Ncap + 1, inst.V), dtype=np.float32)

    def one(req):
        n = int(n_nodes[req])
        paths = [()]
        for i in range(n):
            p = int(parent[req, i])
            prefix = () if p < 0 else paths[p + 1]
            paths.append(prefix + (int(token[req, i]),))
        rows = target_rows(inst, req, paths)
        out[req, : n + 1] = rows
        out[req, n + 1:] = rows[0]

    # requests are independent draws (each keyed by its own path seeds): threads only
    # overlap numpy's generator work
    if inst.R > 1:
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1, inst.R)) as ex:
            list(ex.map(one, range(inst.R)))
    else:
        one(0)
    return out


def make_tie_instance(*, seed: int, R: int, B: int, k: int, V: int, r: int, Ncap: int,
                      dtype: str = "bf16", tau: float = 0.0, cal: str = "monotone",
                      grid: float = 0.25) -> Instance:
    """Exact ties at the top-k cutoff.  U = 0 (no Markov bias: the logits a parent sees are
    exactly its block row), Wt ~ N(0, r**-0.5) (multiplied by zero, never influencing z),
    and block logits on a ``grid``-spaced lattice: N(0, 2) rounded to the grid and clipped to
    [-8, 8], then per row two tokens share the value max + 2 and k + 1 further tokens share
    max + 1, so the k-th child is chosen inside a group of equal values.  Distinct values
    differ by at least one grid step; every value is exact in bf16 and float32."""
    head_rng = np.random.default_rng([seed, 1])
    U = np.zeros((V, r), np.float32)
    Wt = _round(head_rng.normal(0.0, r ** -0.5, size=(V, r)), dtype)
    if cal == "monotone":
        cal_v = np.sort(np.random.default_rng([seed, 2]).uniform(0.05, 0.95, 16)).astype(np.float32)
    else:
        cal_v = ((np.arange(16) + 0.5) / 16.0).astype(np.float32)
    srng = np.random.default_rng([seed, 4])
    roots = srng.integers(0, V, size=R).astype(np.int32)
    Lext = np.empty((R, B + 1, V), np.float32)
    for i in range(R):
        lrng = np.random.default_rng([seed, 5, i])
        x = np.clip(np.rint(lrng.normal(0.0, 2.0, size=(B + 1, V)) / grid) * grid, -8.0, 8.0)
        for d in range(B + 1):
            ids = lrng.choice(V, size=min(V, k + 3), replace=False)
            top = x[d].max()
            x[d, ids[:2]] = top + 2.0
            x[d, ids[2:]] = top + 1.0
        Lext[i] = _round(x, dtype)
    return Instance(name="ties", R=R, B=B, k=k, V=V, r=r, Ncap=Ncap, dtype=dtype,
                    mode="greedy", temperature=1.0, cal=cal_v, seed=seed, round=0, Lext=Lext,
                    U=U, Wt=Wt, root_token=roots, n_budget=np.full(R, Ncap, np.int32),
                    tau=np.full(R, tau, np.float32), rho=0.0, peak="ties", target_peak="none",
                    strength=np.zeros(R), subseed=np.arange(R, dtype=np.int64))
