"""A synthetic drafter/target pair for multi-round decoding (seeded; input synthesis only).

The pages measure rounds per sample and accepted tokens per round with real models on
public benchmarks that are not available here.  This module stands in for them with a
"Markov world" of the pages' shapes, keyed so that every round and every tree variant sees
the same models:

* every request i has a base logit row A(i, p) for each absolute position p: N(0, sd 2)
  plus eight planted peaks (ids drawn per (i, p), boosts from `strength` down to
  4/9 of it), like the block-logit law of ``inputs``;
* the drafter's block logits for a round whose root sits at position p0 are
  L[d] = A(i, p0 + 1 + d), d = 0..B-1 (one forward gives the whole block);
* the target's next-token logits after token t at position p - 1 are
  T(i, p, t) = rho * (A(i, p) + U[t] . W) + sqrt(1 - rho^2) * E(i, p, t), E ~ N(0, sd 2):
  the target depends on the last token through the same low-rank head the drafter uses.

``MarkovWorld`` draws with numpy (exact, reproducible; for small vocabularies and the
parity tests); ``TorchMarkovWorld`` draws the same laws on the GPU with a counter-based
hash (different values; for full-vocabulary measurement only).  Neither holds any of the
construction or verification arithmetic: the target's head term is the target model's own
definition, not the drafter's expansion.
"""
from __future__ import annotations

import math

import numpy as np

from . import inputs


class MarkovWorld:
    """numpy Markov world.  U, Wt: the head (float32 arrays holding dtype values)."""

    def __init__(self, *, seed: int, R: int, B: int, V: int, U: np.ndarray, Wt: np.ndarray,
                 dtype: str, rho: float = 0.8, strength: float = 9.0):
        self.seed, self.R, self.B, self.V = int(seed), int(R), int(B), int(V)
        self.U, self.Wt = U, Wt
        self.dtype, self.rho, self.strength = dtype, float(rho), float(strength)
        self._cache = {}

    def base_row(self, i: int, p: int) -> np.ndarray:
        key = (i, p)
        if key not in self._cache:
            rng = np.random.default_rng([self.seed, 11, i, p])
            x = rng.normal(0.0, 2.0, size=self.V)
            ids = rng.choice(self.V, size=min(8, self.V), replace=False)
            x[ids] += np.linspace(self.strength, self.strength * 4.0 / 9.0, len(ids))
            self._cache[key] = x
        return self._cache[key]

    def block_logits(self, pos0: np.ndarray) -> np.ndarray:
        """[R][B][V] float32 block logits of the round for every request."""
        out = np.empty((self.R, self.B, self.V), np.float32)
        for i in range(self.R):
            rows = np.stack([self.base_row(i, int(pos0[i]) + 1 + d) for d in range(self.B)])
            out[i] = inputs._round(rows, self.dtype)
        return out

    def target_row(self, i: int, p: int, t: int) -> np.ndarray:
        rng = np.random.default_rng([self.seed, 12, i, p, int(t)])
        e = rng.normal(0.0, 2.0, size=self.V)
        head = self.Wt.astype(np.float64) @ self.U[int(t)].astype(np.float64)
        b = math.sqrt(max(0.0, 1.0 - self.rho * self.rho))
        return inputs._round(self.rho * (self.base_row(i, p) + head) + b * e, self.dtype)

    def target_rows(self, roots, pos0, token, parent, depth, n_nodes, Ncap: int) -> np.ndarray:
        """[R][Ncap+1][V] target rows of the emitted trees: row 0 for the root (predicting
        position p0 + 1 after the root token), row j + 1 for node j (predicting position
        p0 + depth_j + 1 after its token); empty slots repeat row 0."""
        out = np.empty((self.R, Ncap + 1, self.V), np.float32)
        for i in range(self.R):
            p0 = int(pos0[i])
            out[i, 0] = self.target_row(i, p0 + 1, int(roots[i]))
            n = int(n_nodes[i])
            for j in range(n):
                out[i, j + 1] = self.target_row(i, p0 + int(depth[i, j]) + 1, int(token[i, j]))
            out[i, n + 1:] = out[i, 0]
        return out

    def greedy_sequence(self, i: int, root: int, length: int) -> list:
        """The target's own greedy continuation of request i from `root` at position 0
        (argmax, ties to the lower id): what lossless greedy decoding must emit."""
        seq, t = [], int(root)
        for p in range(1, length + 1):
            t = int(np.argmax(self.target_row(i, p, t)))
            seq.append(t)
        return seq


class TorchMarkovWorld:
    """The same laws drawn on the GPU (counter-based hashing, erfinv normals); U and Wt are
    device tensors.  Values differ from MarkovWorld's; used for full-vocabulary runs."""

    def __init__(self, torch, *, seed: int, R: int, B: int, V: int, U, Wt, rho: float = 0.8,
                 strength: float = 9.0):
        self.t, self.seed, self.R, self.B, self.V = torch, int(seed), int(R), int(B), int(V)
        self.U, self.Wt = U, Wt
        self.rho, self.strength = float(rho), float(strength)

    def _mix(self, z):
        torch = self.t

        def s64(x):
            return x - (1 << 64) if x >= (1 << 63) else x

        def srl(z, k):
            return (z >> k) & ((1 << (64 - k)) - 1)

        z = z + s64(0x9E3779B97F4A7C15)
        z = (z ^ srl(z, 30)) * s64(0xBF58476D1CE4E5B9)
        z = (z ^ srl(z, 27)) * s64(0x94D049BB133111EB)
        return z ^ srl(z, 31)

    def _normal(self, keys, sd):
        torch = self.t
        cols = torch.arange(self.V, device=keys.device, dtype=torch.int64)
        z = self._mix(self._mix(keys.view(-1, 1)) ^ cols.view(1, -1))
        u = (((z >> 40) & ((1 << 24) - 1)).to(torch.float64) + 0.5) / float(1 << 24)
        return (torch.erfinv(2.0 * u - 1.0) * (math.sqrt(2.0) * sd)).to(torch.float32)

    def _base(self, keys):
        torch = self.t
        x = self._normal(keys * 3 + 1, 2.0)
        boosts = torch.linspace(self.strength, self.strength * 4.0 / 9.0, 8, device=x.device)
        for j in range(8):
            ids = self._mix(keys * 17 + 1000 + j) % self.V
            x.scatter_add_(1, ids.view(-1, 1), boosts[j].expand(ids.numel(), 1).contiguous())
        return x

    def _key(self, i, p):
        return (self.seed * 1000003 + i) * 4000037 + p

    def block_logits(self, pos0):
        """[R][B][V] bf16 device tensor."""
        torch = self.t
        i = torch.arange(self.R, device=pos0.device, dtype=torch.int64).view(-1, 1)
        p = pos0.view(-1, 1).to(torch.int64) + 1 + torch.arange(self.B, device=pos0.device).view(1, -1)
        return self._base(self._key(i, p).reshape(-1)).view(self.R, self.B, self.V).to(torch.bfloat16)

    def _target(self, i: int, p, tok):
        """bf16 rows T(i, p, t) for position tensor p and token tensor tok (same length)."""
        torch = self.t
        b = math.sqrt(max(0.0, 1.0 - self.rho * self.rho))
        keys = self._key(i, p)
        head = self.U[tok].float() @ self.Wt.float().t()
        e = self._normal((keys * 4000037 + tok) * 5 + 2, 2.0)
        return (self.rho * (self._base(keys) + head) + b * e).to(torch.bfloat16)

    def target_rows(self, roots, pos0, tree):
        """[R][Ncap+1][V] bf16 device tensor for the emitted trees (row 0: the root)."""
        torch = self.t
        R = self.R
        tok = torch.cat([roots.view(R, 1).to(torch.int64), tree["token"].to(torch.int64)], 1)
        dep = torch.cat([torch.zeros((R, 1), dtype=torch.int64, device=roots.device),
                         tree["depth"].to(torch.int64)], 1)
        tok = torch.where(tok >= 0, tok, tok[:, :1].expand_as(tok))
        out = torch.empty((R, tok.shape[1], self.V), dtype=torch.bfloat16, device=roots.device)
        for i in range(R):
            out[i] = self._target(i, pos0[i].to(torch.int64) + dep[i] + 1, tok[i])
        return out
