"""Tree-attention oracle: one attention layer of the target's verify forward over a round's
draft trees, written out as its plain definition in float64 numpy.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this module; the library under ``draft_tree_construction_rank_amd``
never does.

What is computed (PCTree summary, "From Chains to Trees", introduction: the target checks
every node of the draft tree in one forward; TreeSpark article, introduction: a tree offers
several continuations to one verification pass).  The tree's positions are the root (the
round's last emitted token) and nodes 0..n-1; their keys and values sit in the cache after
the request's ctx_len context entries, root first (slot ctx_len), node i at slot
ctx_len + 1 + i.  The query of tree position j (j = 0: the root; j = i + 1: node i) sees

  * every context slot and the root's slot, and
  * for a node, the slot of itself and of each of its ancestors (its path from the root),

and nothing else: a node is scored exactly as if its own path were the whole continuation.
Scores are scale * q . k, softmax over the visible slots, output = the softmax-weighted sum
of the visible values.  Grouped-query heads: query head hq reads key/value head
hq // (Hq / Hkv).  Output rows for tree positions past n, and every row of a request whose
n is outside [0, Ncap] or whose tree does not fit the cache (ctx_len < 0 or
ctx_len + n + 1 > Cmax), are zeros.

Visibility here is derived by walking parent pointers, not from the 64-bit ancestor masks
the GPU kernel consumes; ``anc_masks`` builds those masks from parents for test inputs.

Parity status: pinned by tests/test_oracle_attention.py (path equivalence against a library
attention routine, a chain tree against causal attention, closed forms, invariances).
"""
from __future__ import annotations

import numpy as np

__all__ = ["path_of", "visible_slots", "anc_masks", "tree_attention", "request_valid"]


def path_of(parent, i: int) -> list:
    """Node i and its ancestors, root side first (parent[i] = -1: a child of the root)."""
    out = []
    while i >= 0:
        out.append(int(i))
        i = int(parent[i])
    return out[::-1]


def visible_slots(ctx: int, parent, j: int) -> np.ndarray:
    """Cache slots seen by tree position j (0 = root, i + 1 = node i), ascending."""
    slots = list(range(ctx + 1))
    if j > 0:
        slots += [ctx + 1 + i for i in path_of(parent, j - 1)]
    return np.array(sorted(slots), dtype=np.int64)


def anc_masks(parent: np.ndarray, n_nodes: np.ndarray, Ncap: int) -> np.ndarray:
    """[R][Ncap] uint64: bit i of row j set iff node i is node j or one of its ancestors."""
    parent = np.asarray(parent)
    R = parent.shape[0]
    out = np.zeros((R, Ncap), dtype=np.uint64)
    for r in range(R):
        for j in range(int(n_nodes[r])):
            m = 0
            for i in path_of(parent[r], j):
                m |= 1 << i
            out[r, j] = np.uint64(m)
    return out


def request_valid(ctx: int, n: int, Ncap: int, Cmax: int) -> bool:
    return 0 <= n <= Ncap and ctx >= 0 and ctx + n + 1 <= Cmax


def tree_attention(Q, K, V, ctx_len, n_nodes, parent, scale: float, reqs=None,
                   heads=None) -> np.ndarray:
    """Q [R][Hq][Ncap+1][D]; K, V [R][Hkv][Cmax][D]; ctx_len, n_nodes [R]; parent
    [R][Ncap] (parent[r][i] < i, -1 = the root).  Returns float64 [R][Hq][Ncap+1][D].
    ``reqs`` / ``heads`` (optional index lists) restrict the work to those requests and
    query heads; the other rows are left zero."""
    R, Hq, Nq, D = Q.shape
    Hkv, Cmax = K.shape[1], K.shape[2]
    G = Hq // Hkv
    Ncap = Nq - 1
    O = np.zeros((R, Hq, Nq, D), np.float64)
    for r in (range(R) if reqs is None else reqs):
        ctx, n = int(ctx_len[r]), int(n_nodes[r])
        if not request_valid(ctx, n, Ncap, Cmax):
            continue
        vis = [visible_slots(ctx, parent[r], j) for j in range(n + 1)]
        for hq in (range(Hq) if heads is None else heads):
            h = hq // G
            Kr = np.asarray(K[r, h, :ctx + n + 1], np.float64)
            Vr = np.asarray(V[r, h, :ctx + n + 1], np.float64)
            for j in range(n + 1):
                s = float(scale) * (Kr[vis[j]] @ np.asarray(Q[r, hq, j], np.float64))
                p = np.exp(s - s.max())
                p /= p.sum()
                O[r, hq, j] = p @ Vr[vis[j]]
    return O
