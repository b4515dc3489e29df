"""Pins for the tree-attention oracle (no GPU).

Each test checks ``oracle.attention`` against something other than itself:

* path equivalence: every tree position's output equals ordinary attention (torch's
  scaled_dot_product_attention in float64, no mask) of its query over the keys of its own
  sequence (context, root, then its path), with the path found here by a depth-first walk
  from the root rather than by the oracle's parent walk;
* a chain tree equals causal attention over context + chain (bottom-right causal mask);
* K = 0 gives the plain mean of the visible values, whose count is ctx + 1 + depth;
* outputs do not depend on the keys/values of nodes off the query's path, and do depend
  on those on it;
* grouped heads equal ungrouped heads over repeated keys/values;
* ancestor masks built from parents equal the C oracle's emitted masks for a real tree;
* rows past n and whole invalid requests are zero.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import attention as oa
from draft_tree_construction_rank_amd import attn_inputs, inputs


def _small(seed, **kw):
    d = dict(seed=seed, R=3, Hq=4, Hkv=2, D=16, Ncap=12, ctx_lo=0, ctx_hi=20, threads=1)
    d.update(kw)
    return attn_inputs.make_attn_instance(**d)


def _dfs_paths(parent, n):
    """Path (root side first, node last) of every node, by depth-first search from the root."""
    kids = {-1: []}
    for i in range(n):
        kids.setdefault(int(parent[i]), []).append(i)
        kids.setdefault(i, [])
    paths = {}
    stack = [(-1, [])]
    while stack:
        v, path = stack.pop()
        for c in kids[v]:
            paths[c] = path + [c]
            stack.append((c, path + [c]))
    return paths


def _sdpa(q, k, v, scale, mask=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float64))
    out = F.scaled_dot_product_attention(t(q)[None, None], t(k)[None, None], t(v)[None, None],
                                         attn_mask=None if mask is None else torch.from_numpy(mask)[None, None],
                                         scale=scale)
    return out[0, 0].numpy()


@pytest.mark.parametrize("seed,tree,qscale", [(0, "random", 1.0), (1, "random", 4.0),
                                              (2, "star", 1.0), (3, "chain", 2.0)])
def test_path_equivalence(seed, tree, qscale):
    inst = _small(seed, tree=tree, qscale=qscale, nodes="ragged")
    Q, K, V = inst.f32("Q"), inst.f32("K"), inst.f32("V")
    O = oa.tree_attention(Q, K, V, inst.ctx_len, inst.n_nodes, inst.parent, inst.scale)
    G = inst.Hq // inst.Hkv
    for r in range(inst.R):
        ctx, n = int(inst.ctx_len[r]), int(inst.n_nodes[r])
        paths = _dfs_paths(inst.parent[r], n)
        for hq in range(inst.Hq):
            h = hq // G
            for j in range(n + 1):
                slots = list(range(ctx + 1)) + ([ctx + 1 + i for i in paths[j - 1]] if j else [])
                want = _sdpa(Q[r, hq, j:j + 1], K[r, h, slots], V[r, h, slots], inst.scale)[0]
                np.testing.assert_allclose(O[r, hq, j], want, rtol=1e-12, atol=1e-12)


def test_chain_is_causal():
    inst = _small(4, tree="chain", nodes="full", ctx_lo=5, ctx_hi=9)
    Q, K, V = inst.f32("Q"), inst.f32("K"), inst.f32("V")
    O = oa.tree_attention(Q, K, V, inst.ctx_len, inst.n_nodes, inst.parent, inst.scale)
    G = inst.Hq // inst.Hkv
    for r in range(inst.R):
        ctx, n = int(inst.ctx_len[r]), int(inst.n_nodes[r])
        L = ctx + n + 1
        mask = np.tril(np.ones((n + 1, L), bool), k=ctx)
        for hq in range(inst.Hq):
            want = _sdpa(Q[r, hq, :n + 1], K[r, hq // G, :L], V[r, hq // G, :L], inst.scale, mask)
            np.testing.assert_allclose(O[r, hq, :n + 1], want, rtol=1e-12, atol=1e-12)


def test_zero_keys_average_visible_values():
    inst = _small(5, nodes="ragged")
    Q, V = inst.f32("Q"), inst.f32("V")
    K = np.zeros(inst.K.shape, np.float32)
    O = oa.tree_attention(Q, K, V, inst.ctx_len, inst.n_nodes, inst.parent, inst.scale)
    G = inst.Hq // inst.Hkv
    for r in range(inst.R):
        ctx, n = int(inst.ctx_len[r]), int(inst.n_nodes[r])
        paths = _dfs_paths(inst.parent[r], n)
        for j in range(n + 1):
            depth = len(paths[j - 1]) if j else 0
            slots = list(range(ctx + 1)) + ([ctx + 1 + i for i in paths[j - 1]] if j else [])
            assert len(slots) == ctx + 1 + depth
            for hq in range(inst.Hq):
                want = V[r, hq // G, slots].astype(np.float64).sum(0) / (ctx + 1 + depth)
                np.testing.assert_allclose(O[r, hq, j], want, rtol=1e-12, atol=1e-12)


def test_off_path_nodes_do_not_matter():
    inst = _small(6, R=1, nodes="full", tree="random")
    Q, K, V = inst.f32("Q"), inst.f32("K"), inst.f32("V")
    base = oa.tree_attention(Q, K, V, inst.ctx_len, inst.n_nodes, inst.parent, inst.scale)
    ctx, n = int(inst.ctx_len[0]), int(inst.n_nodes[0])
    paths = _dfs_paths(inst.parent[0], n)
    rng = np.random.default_rng(7)
    for victim in range(n):
        K2, V2 = K.copy(), V.copy()
        K2[0, :, ctx + 1 + victim] += rng.normal(0, 3, K2.shape[-1]).astype(np.float32)
        V2[0, :, ctx + 1 + victim] += rng.normal(0, 3, V2.shape[-1]).astype(np.float32)
        O2 = oa.tree_attention(Q, K2, V2, inst.ctx_len, inst.n_nodes, inst.parent, inst.scale)
        for j in range(n + 1):
            on_path = j > 0 and victim in paths[j - 1]
            same = np.array_equal(O2[0, :, j], base[0, :, j])
            assert same != on_path, (victim, j)


def test_grouped_heads_equal_repeated_kv():
    inst = _small(8, Hq=8, Hkv=2, nodes="ragged")
    Q, K, V = inst.f32("Q"), inst.f32("K"), inst.f32("V")
    O = oa.tree_attention(Q, K, V, inst.ctx_len, inst.n_nodes, inst.parent, inst.scale)
    Kr, Vr = np.repeat(K, 4, axis=1), np.repeat(V, 4, axis=1)
    O1 = oa.tree_attention(Q, Kr, Vr, inst.ctx_len, inst.n_nodes, inst.parent, inst.scale)
    np.testing.assert_array_equal(O, O1)
    # and a different grouping is a different result (the head map matters)
    O2 = oa.tree_attention(Q, np.tile(K, (1, 4, 1, 1)), np.tile(V, (1, 4, 1, 1)),
                           inst.ctx_len, inst.n_nodes, inst.parent, inst.scale)
    assert not np.allclose(O, O2)


def test_masks_match_emitted_tree():
    inst = inputs.make_instance("tiny")
    t = oracle.build_tree(inst, tau=0.0)
    n = t["n_nodes"]
    assert int(n[0]) > 3
    m = oa.anc_masks(t["parent"], n, inst.Ncap)
    np.testing.assert_array_equal(m, t["mask"].astype(np.uint64))


def test_zero_rows_and_invalid_requests():
    inst = _small(9, R=4, nodes="ragged", ctx_lo=3, ctx_hi=6)
    inst.n_nodes[1] = inst.Ncap + 1   # n out of range
    inst.ctx_len[2] = -1              # negative context
    inst.ctx_len[3] = inst.Cmax - int(inst.n_nodes[3])  # tree does not fit
    Q, K, V = inst.f32("Q"), inst.f32("K"), inst.f32("V")
    O = oa.tree_attention(Q, K, V, inst.ctx_len, inst.n_nodes, inst.parent, inst.scale)
    n0 = int(inst.n_nodes[0])
    assert O[0, :, :n0 + 1].any(axis=-1).all()
    assert not O[0, :, n0 + 1:].any()
    assert not O[1:].any()


def test_large_scores_stay_finite():
    inst = _small(10, qscale=60.0)
    Q, K, V = inst.f32("Q"), inst.f32("K"), inst.f32("V")
    O = oa.tree_attention(Q, K, V, inst.ctx_len, inst.n_nodes, inst.parent, inst.scale)
    assert np.isfinite(O).all()
    # at this temperature each row is close to the value of its best visible key
    r, hq, j = 0, 1, 0
    ctx = int(inst.ctx_len[r])
    s = K[r, hq // 2, :ctx + 1].astype(np.float64) @ Q[r, hq, j]
    assert math.isclose(O[r, hq, j, 0], float(V[r, hq // 2, int(np.argmax(s)), 0]), abs_tol=0.05)
