"""Pins for the oracle's verifiers (no GPU).

Greedy: closed forms (target = draft rows; an off-tree target argmax).  Sample: exact
enumeration of the emitted law over every ordered draw of siblings (it must equal the
target law, TreeSpark lossless section); the single-draft acceptance rate sum(min(p, q))
(Leviathan et al. 2023, recalled on the same page); p = q forces every first-ranked sibling
to be accepted; Gumbel-top-k order frequencies against Plackett-Luce; chi-square tests of
the emitted tokens over 10^6 rounds at T in {0.6, 1.0, 1.5}; negative controls planted in the
oracle must be caught.
"""
import itertools

import numpy as np
import pytest
from scipy import stats
from scipy.special import logsumexp, softmax

import oracle
from oracle_helpers import (chisq_binned, exact_emitted_law, node_dist, plackett_luce, small_instance,
                            tree_paths)


# ------------------------------------------------------------------ greedy ---------------
def _target_from_rows(inst, tree, rowfn):
    n = int(tree["n_nodes"][0])
    t = np.zeros((1, inst.Ncap + 1, inst.V), np.float32)
    t[0, 0] = rowfn(0, int(inst.root_token[0]))
    for i in range(n):
        t[0, i + 1] = rowfn(int(tree["depth"][0, i]), int(tree["token"][0, i]))
    t[0, n + 1:] = t[0, 0]
    return t


@pytest.mark.parametrize("seed", range(8))
def test_greedy_target_equal_to_draft_accepts_chain_prefix(seed):
    """U = 0 and target row(v) = L[d_v] (rho = 1): the target's argmax chain is the drafter's
    rank-0 chain, so accept_len = the longest prefix of that chain present in the tree."""
    inst = small_instance(seed, V=20, r=4, B=4, k=2, Ncap=3 + seed, cal="monotone")
    inst.U[:] = 0.0
    tree = oracle.build_tree(inst)
    tgt = _target_from_rows(inst, tree, lambda d, t: inst.Lext[0, d])
    res = oracle.verify_greedy(inst, tree, tgt)
    chain = [int(np.argmax(inst.Lext[0, d])) for d in range(inst.B + 1)]
    paths = set(tree_paths(tree))
    m = 0
    while m < inst.B and tuple(chain[: m + 1]) in paths:
        m += 1
    assert res["accept_len"][0] == m
    assert list(res["out_tokens"][0, : m + 1]) == chain[: m + 1]
    assert res["n_out"][0] == m + 1


def test_greedy_off_tree_argmax_rejects_at_root():
    inst = small_instance(1, V=20, r=4, B=3, k=2, Ncap=6)
    tree = oracle.build_tree(inst)
    kids = set(int(x) for x in tree["cand"][0, 0])
    off = min(c for c in range(inst.V) if c not in kids)
    tgt = np.zeros((1, inst.Ncap + 1, inst.V), np.float32)
    tgt[0, 0, off] = 5.0
    res = oracle.verify_greedy(inst, tree, tgt)
    assert res["accept_len"][0] == 0 and res["out_tokens"][0, 0] == off
    assert res["n_out"][0] == 1 and (res["path"][0] == -1).all()


def test_greedy_ties_take_lower_id():
    inst = small_instance(2, V=20, r=4, B=3, k=2, Ncap=6)
    tree = oracle.build_tree(inst)
    tgt = np.zeros((1, inst.Ncap + 1, inst.V), np.float32)
    res = oracle.verify_greedy(inst, tree, tgt)  # all-equal rows: argmax = token 0
    assert res["out_tokens"][0, 0] == 0


# ------------------------------------------------------------------ exact law ------------
def _rand_pq(rng, V, sharp=1.0):
    p = softmax(rng.normal(0, sharp, V))
    q = softmax(rng.normal(0, sharp, V))
    return p, q


@pytest.mark.parametrize("V,k", [(2, 1), (3, 1), (3, 2), (4, 2), (5, 3), (6, 3), (6, 2), (4, 3)])
def test_exact_law_equals_target(V, k):
    rng = np.random.default_rng(V * 10 + k)
    for trial in range(20):
        p, q = _rand_pq(rng, V, sharp=0.5 + trial * 0.2)
        law = exact_emitted_law(p, q, k)
        assert np.abs(law - p).max() < 1e-11


def test_exact_law_depth_two_joint():
    """Joint law of the first two tokens at depth <= 2: first ~ p_root, and given an
    accepted first token x the chain at x has law p_x, so P(x, y) = p_root(x) p_x(y)."""
    rng = np.random.default_rng(7)
    V, k = 5, 2
    p0, q0 = _rand_pq(rng, V)
    pc = [softmax(rng.normal(0, 1, V)) for _ in range(V)]
    qc = [softmax(rng.normal(0, 1, V)) for _ in range(V)]
    first = exact_emitted_law(p0, q0, k)
    joint = np.array([[first[x] * exact_emitted_law(pc[x], qc[x], k)[y] for y in range(V)]
                      for x in range(V)])
    want = np.outer(p0, np.ones(V)) * np.array(pc)
    assert np.abs(joint - want).max() < 1e-11


@pytest.mark.parametrize("fault", [1, 2])
def test_exact_law_negative_controls_fail(fault):
    rng = np.random.default_rng(3)
    oracle.set_fault(fault)
    try:
        worst = 0.0
        for _ in range(10):
            p, q = _rand_pq(rng, 5, sharp=1.5)
            worst = max(worst, np.abs(exact_emitted_law(p, q, 3) - p).max())
    finally:
        oracle.set_fault(0)
    assert worst > 1e-3


# ------------------------------------------------------------------ statistics -----------
def _lossless_instance(T, seed=11, k=3):
    inst = small_instance(seed, V=16, r=4, B=2, k=k, Ncap=5, mode="sample", temperature=T,
                          cal="linear")
    rng = np.random.default_rng(100 + seed)
    tab = rng.normal(0, 1.5, size=(inst.B + 1, inst.V, inst.V)).astype(np.float32)
    return inst, tab


def _lossless_pvalue(inst, tab, T, n):
    first, second = oracle.sample_rounds(inst, tab, n, temperature=T)
    root = int(inst.root_token[0])
    p0 = softmax(tab[0, root].astype(np.float64) / T)
    s1, d1 = chisq_binned(np.bincount(first, minlength=inst.V).astype(float), p0)
    stat, dof = s1, d1
    for x in range(inst.V):
        sel = second[(first == x) & (second >= 0)]
        if len(sel) < 200:
            continue
        px = softmax(tab[1, x].astype(np.float64) / T)
        s, d = chisq_binned(np.bincount(sel, minlength=inst.V).astype(float), px)
        stat += s
        dof += d
    return stats.chi2.sf(stat, dof), (second >= 0).mean()


@pytest.mark.parametrize("T", [0.6, 1.0, 1.5])
def test_chisq_lossless_1e6_rounds(T):
    inst, tab = _lossless_instance(T)
    pval, frac2 = _lossless_pvalue(inst, tab, T, 1_000_000)
    assert frac2 > 0.05  # the second-token test has real data
    assert pval > 1e-4, pval


def test_chisq_negative_control_rejected():
    T = 1.0
    inst, tab = _lossless_instance(T)
    oracle.set_fault(1)
    try:
        pval, _ = _lossless_pvalue(inst, tab, T, 1_000_000)
    finally:
        oracle.set_fault(0)
    assert pval < 1e-9, pval


def _depth_b_instance(T, seed=21, k=3):
    """B = 1 with every drawn sibling kept: a round that accepts a sibling descends to a
    depth-B node, so its second token is that node's terminal draw from p."""
    inst = small_instance(seed, V=16, r=4, B=1, k=k, Ncap=k, mode="sample", temperature=T,
                          cal="linear", peak="none")
    rng = np.random.default_rng(300 + seed)
    tab = rng.normal(0, 1.5, size=(inst.B + 1, inst.V, inst.V)).astype(np.float32)
    # the root's target row follows the draft row, so most rounds accept a sibling
    root = int(inst.root_token[0])
    tab[0, root] = (node_dist(inst, 0, 0, root, 1.0) + rng.normal(0, 0.3, inst.V)).astype(np.float32)
    return inst, tab


def _depth_b_pvalue(inst, tab, T, n):
    """Chi-square of the second token given the first against p of the depth-B node
    (softmax of its own target row at temperature T)."""
    first, second = oracle.sample_rounds(inst, tab, n, temperature=T)
    stat, dof = 0.0, 0
    for x in range(inst.V):
        sel = second[(first == x) & (second >= 0)]
        if len(sel) < 200:
            continue
        px = softmax(tab[1, x].astype(np.float64) / T)
        s, d = chisq_binned(np.bincount(sel, minlength=inst.V).astype(float), px)
        stat += s
        dof += d
    return stats.chi2.sf(stat, dof), (second >= 0).mean(), dof


@pytest.mark.parametrize("T", [0.6, 1.0, 1.5])
def test_chisq_depth_b_terminal_draw(T):
    """TreeSpark lossless section: at the last block position there is no draft row, so the
    round ends with a draw from the target law p of that node."""
    inst, tab = _depth_b_instance(T)
    pval, frac2, dof = _depth_b_pvalue(inst, tab, T, 600_000)
    assert frac2 > 0.2 and dof >= 60  # many depth-B draws under test
    assert pval > 1e-4, pval


def test_chisq_depth_b_negative_control_rejected():
    """A depth-B draw taken from the parent's target row must fail the same test."""
    T = 1.0
    inst, tab = _depth_b_instance(T)
    oracle.set_fault(3)
    try:
        pval, _, _ = _depth_b_pvalue(inst, tab, T, 600_000)
    finally:
        oracle.set_fault(0)
    assert pval < 1e-9, pval


def test_single_draft_acceptance_rate():
    """k = 1: the root's draft is accepted with probability sum_x min(p(x), q(x)); an
    accepted draft is in the tree (N >= 1, tau = 0), so the round then emits a second token."""
    T = 1.0
    inst, tab = _lossless_instance(T, seed=5, k=1)
    n = 400_000
    first, second = oracle.sample_rounds(inst, tab, n, temperature=T)
    root = int(inst.root_token[0])
    p0 = softmax(tab[0, root].astype(np.float64) / T)
    q0 = softmax(node_dist(inst, 0, 0, root, T))
    a = np.minimum(p0, q0).sum()
    got = (second >= 0).sum()
    z = (got - n * a) / np.sqrt(n * a * (1 - a))
    assert abs(z) < 4.5, (got / n, a)


def test_p_equals_q_accepts_first_ranked_sibling():
    """U = 0 and a target equal to the block logits: p = q at every node, so u * q(x) < p(x)
    always holds for the first drawn sibling; with the whole candidate tree kept, every round
    accepts the Gumbel-argmax child of the root and then of that child."""
    T = 0.8
    inst = small_instance(4, V=12, r=4, B=2, k=2, Ncap=6, mode="sample", temperature=T)
    inst.U[:] = 0.0
    tab = np.zeros((inst.B + 1, inst.V, inst.V), np.float32)
    for d in range(inst.B + 1):
        tab[d, :, :] = inst.Lext[0, d]
    n = 3000
    first, second = oracle.sample_rounds(inst, tab, n, temperature=T)
    assert (second >= 0).all()
    root = int(inst.root_token[0])
    y0 = inst.Lext[0, 0].astype(np.float64) / T
    for rnd in range(50):
        h = oracle.root_hash(rnd, 0, root)
        g = [-np.log(-np.log(oracle.uniform(inst.seed, h, oracle.STREAM_GUMBEL, c)))
             for c in range(inst.V)]
        x1 = int(np.argmax(y0 + np.array(g)))
        assert first[rnd] == x1


def test_gumbel_topk_matches_plackett_luce():
    """Gumbel-top-k ranked children are an ordered draw without replacement from q."""
    T = 1.0
    inst = small_instance(8, V=6, r=4, B=2, k=2, mode="sample", temperature=T)
    root = int(inst.root_token[0])
    y = node_dist(inst, 0, 0, root, T)
    q = np.exp(y - logsumexp(y))
    pairs = list(itertools.permutations(range(inst.V), 2))
    idx = {p: i for i, p in enumerate(pairs)}
    counts = np.zeros(len(pairs))
    n = 60_000
    for i in range(n):
        e = oracle.expand(inst, 0, 0, root, oracle.mix64(i))
        counts[idx[tuple(int(x) for x in e["child_tok"])]] += 1
    probs = np.array([plackett_luce(q, p) for p in pairs])
    assert abs(probs.sum() - 1) < 1e-12
    stat, dof = chisq_binned(counts, probs)
    assert stats.chi2.sf(stat, dof) > 1e-4
