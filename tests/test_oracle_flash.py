"""Pins for the oracle's two-stage M-ary tree (TreeFlash explainer, technical summary,
methodology: two-stage inference construction, on this library's Markov head).  No GPU.

* brute force: an independent numpy enumeration of the whole lattice (every depth's M
  tokens from the unconditioned rows, each node's q from a direct float64 softmax of the
  parent-conditioned row), survival products in float32, the global order, top-N;
* M = 1: the chain of the per-row argmax tokens of the unconditioned block rows;
* M = V: the lattice holds every token, so the tree equals the parent-conditioned tree with
  k = V (the library's main build, a different code path);
* U = 0: every state's law is the unconditioned row, so the tree equals the marginal
  (no-bias) tree with k = M;
* nesting in N; every depth's tokens lie in that depth's stage-1 set.
"""
import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from oracle_helpers import cal_bin, check_structure, small_instance, tree_paths


def _flash(inst, **kw):
    return oracle.build_tree(inst, method=oracle.BUILD_FLASH, **kw)


def _stage1(inst, req, M):
    """Per block row, the M largest logits (ties: lower id), in that order."""
    sets = []
    for j in range(inst.B):
        row = inst.L[req, j].astype(np.float64)
        order = sorted(range(inst.V), key=lambda c: (-row[c], c))
        sets.append(order[:M])
    return sets


def _flash_brute(inst, req, N, tau):
    M = inst.k
    sets = _stage1(inst, req, M)
    U, Wt = inst.U.astype(np.float64), inst.Wt.astype(np.float64)
    root = int(inst.root_token[req])

    def children(j, t):
        z = inst.L[req, j].astype(np.float64) + Wt @ U[t]
        lse = logsumexp(z)
        ranked = sorted(sets[j], key=lambda c: (-z[c], c))
        return [(c, z[c] - lse) for c in ranked]

    nodes, frontier = [], [dict(token=root, depth=0, s=np.float32(1.0), ranks=())]
    while frontier:
        nxt = []
        for nd in frontier:
            if nd["depth"] >= inst.B:
                continue
            for i, (c, lq) in enumerate(children(nd["depth"], nd["token"])):
                a = inst.cal[cal_bin(np.exp(lq))]
                ch = dict(token=c, depth=nd["depth"] + 1, s=np.float32(nd["s"] * np.float32(a)),
                          ranks=nd["ranks"] + (i,), logq=np.float32(lq))
                nodes.append(ch)
                nxt.append(ch)
        frontier = nxt
    keep = [n for n in nodes if not (n["s"] < np.float32(tau))]
    keep.sort(key=lambda n: (-float(n["s"]), n["depth"], n["ranks"]))
    keep = keep[:N]
    keep.sort(key=lambda n: (n["depth"], n["ranks"]))
    return keep, sets


CASES = [dict(seed=s, V=v, r=r, B=b, k=m, Ncap=n, tau=t)
         for s, (v, r, b, m, n, t) in enumerate([
             (24, 4, 3, 2, 6, 0.0), (20, 4, 3, 3, 12, 0.0), (16, 4, 4, 2, 10, 0.0),
             (30, 8, 3, 4, 20, 0.0), (12, 2, 3, 3, 30, 0.02), (24, 4, 3, 2, 6, 0.3),
             (10, 4, 2, 5, 40, 0.0)])]
PLATEAU = [0.25] * 4 + [0.5] * 4 + [0.75] * 4 + [1.0] * 4


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
@pytest.mark.parametrize("table", ["monotone", "plateau"])
def test_flash_matches_brute_force(case, table):
    c = dict(case)
    tau = c.pop("tau")
    inst = small_instance(c.pop("seed") + 40, cal="monotone", tau=tau, **c)
    if table == "plateau":
        inst.cal = np.array(PLATEAU, np.float32)
    t = _flash(inst, tau=tau)
    keep, sets = _flash_brute(inst, 0, inst.Ncap, tau)
    n = int(t["n_nodes"][0])
    assert n == len(keep)
    check_structure(inst, t, 0)
    paths = tree_paths(t, 0)
    for i, nd in enumerate(keep):
        assert int(t["depth"][0, i]) == nd["depth"]
        assert int(t["token"][0, i]) == nd["token"]
        assert t["surv"][0, i] == nd["s"]
        assert abs(float(t["logq"][0, i]) - float(nd["logq"])) <= 1e-6 * max(1.0, abs(float(nd["logq"])))
        assert paths[i][-1] in sets[nd["depth"] - 1]


def test_flash_m1_is_the_marginal_argmax_chain():
    inst = small_instance(5, V=40, r=8, B=5, k=1, Ncap=5)
    t = _flash(inst, tau=0.0)
    want = [int(np.argmax(inst.L[0, j])) for j in range(inst.B)]
    assert int(t["n_nodes"][0]) == inst.B
    assert [int(x) for x in t["token"][0, :inst.B]] == want
    assert [int(x) for x in t["parent"][0, :inst.B]] == [-1, 0, 1, 2, 3]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_flash_full_lattice_equals_parent_conditioned_tree(seed):
    """M = V: the stage-1 sets hold every token, so each node's children are all tokens
    ranked by the conditional logit, which is the parent-conditioned tree with k = V."""
    inst = small_instance(60 + seed, V=6, r=4, B=3, k=6, Ncap=20, cal="monotone")
    tf = _flash(inst, tau=0.0)
    tp = oracle.build_tree(inst, tau=0.0)
    for f in ("token", "parent", "depth", "mask", "surv", "logq", "n_nodes", "cand"):
        np.testing.assert_array_equal(tf[f], tp[f], err_msg=f)


@pytest.mark.parametrize("seed", [0, 1])
def test_flash_without_head_equals_marginal_tree(seed):
    inst = small_instance(70 + seed, V=30, r=4, B=4, k=3, Ncap=16, cal="monotone")
    inst.U = np.zeros_like(inst.U)
    tf = _flash(inst, tau=0.0)
    inst.cond = oracle.COND_NONE
    tm = oracle.build_tree(inst, tau=0.0)
    for f in ("token", "parent", "depth", "mask", "surv", "logq", "n_nodes", "cand"):
        np.testing.assert_array_equal(tf[f], tm[f], err_msg=f)


def test_flash_nesting_in_budget():
    inst = small_instance(80, V=24, r=4, B=4, k=3, Ncap=24, cal="monotone")
    full = tree_paths(_flash(inst, tau=0.0), 0)
    for n in (1, 3, 7, 15):
        part = tree_paths(_flash(inst, tau=0.0, n_budget=n), 0)
        assert set(part) <= set(full) and len(part) == n
