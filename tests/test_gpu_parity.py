"""GPU parity: the HIP path (through the C ABI) against the oracle, element by element.

Discrete outputs (topology, tokens, masks, candidate lists, survival bits, accepted paths)
must match exactly on margin-certified inputs; logq within 1e-5 * max(1, |ref|).  Sizes
span several 64-row tiles, ragged vocabulary tails and the full V = 151936 workloads.
"""
import numpy as np
import pytest

import oracle
from draft_tree_construction_rank_amd import inputs
from oracle_helpers import check_structure, tree_paths
from parity_helpers import (STRESS_MARGIN, case_instance, certified, compare_trees,
                            compare_verify, deep_path_targets, instance, tie_targets,
                            tree_targets)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    import torch
    from draft_tree_construction_rank_amd import runner
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return runner


def _gpu_round(rt, inst, **pkw):
    rnd = rt.Round(inst, **pkw)
    d = rt.to_device(inst)
    rnd.build(d)
    import torch
    torch.cuda.synchronize()
    return rnd, d, rt.tree_to_numpy(rnd.tree)


def _greedy_case(rt, inst, rows=None, margin=None, key=None):
    """Certify, build on the GPU, compare `rows` (default: every request) with the oracle,
    check every request's structure, then greedy-verify against targets keyed by the
    oracle trees' token paths and compare the walks.  `key` names a full-vocabulary case
    (its instance and stored sub-seeds) instead of `inst`."""
    if key is not None:
        inst = case_instance(key)
    print("case", key or inst.name, "R=%d B=%d k=%d V=%d N=%d" % (
        inst.R, inst.B, inst.k, inst.V, inst.Ncap), flush=True)
    rows = list(range(inst.R)) if rows is None else rows
    inst, ref = certified(inst, rows, margin=margin, key=key)
    rnd, d, got = _gpu_round(rt, inst)
    compare_trees(ref, got, rows)
    for i in range(inst.R):
        check_structure(inst, got, i)
    sub = tree_targets(inst, ref, rows)
    vres = oracle.verify_greedy(inst, ref, sub)
    if rows == list(range(inst.R)):
        tgt = sub
    else:
        tgt = np.zeros((inst.R, inst.Ncap + 1, inst.V), np.float32)
        tgt[rows] = sub
    del sub
    out = rnd.verify_greedy(rt.target_to_device(inst, tgt))
    import torch
    torch.cuda.synchronize()
    gv = {k: v.cpu().numpy() for k, v in out.items()}
    compare_verify(vres, gv, rows)
    print("  compared %d requests: mean nodes %.1f, mean accept_len %.2f" % (
        len(rows), float(ref["n_nodes"].mean()), float(vres["accept_len"].mean())), flush=True)
    return inst, ref, got, gv


def _check_expansions(inst, got, rows):
    """Expansion counts: per request equal to the oracle's level-synchronous build (the same
    schedule: every frontier node kept at a level is expanded at the next), and the per-level
    row counts add up to them and are zero past the last level reached."""
    lref = oracle.build_tree(inst, requests=rows, method=1)
    assert np.array_equal(lref["n_expand"], got["n_expand"][rows]), (lref["n_expand"], got["n_expand"][rows])
    lr = got["level_rows"]
    assert int(lr.sum()) == int(got["n_expand"].sum())
    used = np.nonzero(lr)[0]
    if len(used):
        last = int(used.max())
        assert (lr[:last + 1] > 0).all() and (lr[last + 1:] == 0).all(), lr


# ------------------------------------------------------------------ small, several tiles ----
SMALL = [
    dict(seed=1, V=1000, r=8, B=4, k=2, Ncap=8, R=3, dtype="f32"),
    dict(seed=2, V=3001, r=16, B=5, k=3, Ncap=20, R=5, dtype="bf16"),
    dict(seed=3, V=777, r=24, B=6, k=4, Ncap=40, R=4, dtype="bf16", tau=0.01),
    dict(seed=4, V=4096, r=64, B=3, k=8, Ncap=64, R=3, dtype="f32"),
    dict(seed=5, V=257, r=8, B=8, k=1, Ncap=6, R=2, dtype="bf16"),
    dict(seed=6, V=130, r=32, B=4, k=5, Ncap=33, R=6, dtype="bf16", tau=0.02),
    dict(seed=7, V=2048, r=256, B=3, k=4, Ncap=64, R=2, dtype="bf16"),
    # group mode (a level of more than 64 rows, bf16, V a multiple of 8) with a ragged last
    # 32-column block: the copy clamps of the staging ring
    dict(seed=8, V=1000, r=64, B=4, k=4, Ncap=32, R=8, dtype="bf16"),
    dict(seed=9, V=1736, r=256, B=3, k=3, Ncap=40, R=12, dtype="bf16", tau=0.01),
    # a wide batch: several 256-row groups per level (the last one ragged) and many merges
    # and selects per workgroup
    dict(seed=10, V=2048, r=32, B=3, k=4, Ncap=32, R=200, dtype="bf16"),
    # the largest block count (B = 32): a 32-level chain, a wide tree of N = 64, and a level
    # of more than 64 rows (group mode) at that B
    dict(seed=11, V=700, r=16, B=32, k=1, Ncap=32, R=2, dtype="f32"),
    dict(seed=12, V=1000, r=32, B=32, k=2, Ncap=64, R=3, dtype="bf16"),
    dict(seed=13, V=1000, r=32, B=32, k=2, Ncap=64, R=40, dtype="bf16"),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: "seed%d" % c["seed"])
def test_small_instances(rt, cfg):
    c = dict(cfg)
    tau = c.pop("tau", 0.0)
    inst = instance("tiny", strong=True, cal="monotone", rho=0.5, **c)
    inst.tau = np.full(inst.R, tau, np.float32)
    inst, ref, got, _ = _greedy_case(rt, inst, margin=STRESS_MARGIN)
    _check_expansions(inst, got, list(range(inst.R)))


def test_tiny_config(rt):
    _greedy_case(rt, instance("tiny"))


@pytest.mark.parametrize("strong", [0, 1])
def test_b7_config(rt, strong):
    _greedy_case(rt, None, key="b7|strong=%d" % strong)


@pytest.mark.parametrize("strong", [0, 1])
def test_b16_headline(rt, strong):
    inst, ref, got, _ = _greedy_case(rt, None, key="b16|strong=%d" % strong)
    _check_expansions(inst, got, [0])


def test_b16_sharp_peaks(rt):
    """Planted boosts large enough that child probabilities spread over the calibration bins,
    so survival ordering (not only breadth-first order) decides the tree at full V."""
    _greedy_case(rt, None, key="b16|sharp")


@pytest.mark.parametrize("k", [1, 2, 4, 8])
@pytest.mark.parametrize("N", [16, 32, 64])
def test_b16_sweep(rt, k, N):
    inst, ref, got, _ = _greedy_case(rt, None, key="b16|k=%d|N=%d" % (k, N))
    if k == 1:
        # k = 1: the argmax chain of the parent-conditioned logits (PCTree: k = 1 = chain)
        t = int(inst.root_token[0])
        Wt = inst.Wt.astype(np.float64)
        for dd in range(min(inst.B, N)):
            z = inst.L[0, dd].astype(np.float64) + Wt @ inst.U[t].astype(np.float64)
            t = int(np.argmax(z))
            assert got["token"][0, dd] == t


@pytest.mark.parametrize("tau", [0.05, 0.2, 0.5, 0.0])
def test_batched_config(rt, tau):
    """The batched workload (64 requests, per-request peak strength): every request is
    compared with the oracle; tau = 0 keeps full 64-node trees (65 expansions each)."""
    inst, ref, got, _ = _greedy_case(rt, None, key="batched|tau=%g|strong=0" % tau)
    _check_expansions(inst, got, list(range(inst.R)) if tau > 0 else list(range(8)))


@pytest.mark.parametrize("tau", [0.05, 0.0])
def test_batched_strong_head(rt, tau):
    """Strong-head companion of the batched workload (U, W sd r^-1/4, bias sd 1), so that a
    wrong parent row in the group-mode expansion changes the trees."""
    inst, ref, got, _ = _greedy_case(rt, None, key="batched|tau=%g|strong=1" % tau)
    _check_expansions(inst, got, list(range(inst.R)) if tau > 0 else list(range(8)))


# ------------------------------------------------------------------ head variants ----------
@pytest.mark.parametrize("key", ["b16|strong=1|cond=1", "b16|strong=1|cond=2",
                                 "batched|tau=0.05|strong=1|cond=1",
                                 "batched|tau=0.05|strong=1|cond=2"])
def test_head_variants_full_vocab(rt, key):
    """Shared-Markov (chain head) and marginal (no head) trees at V = 151936, through the
    W-resident kernel (one request) and the streaming kernel (64 requests)."""
    _greedy_case(rt, None, key=key)


VARIANT_SMALL = [
    dict(seed=1, V=1000, r=8, B=4, k=2, Ncap=8, R=3, dtype="f32"),
    dict(seed=7, V=2048, r=256, B=3, k=4, Ncap=64, R=2, dtype="bf16"),
    dict(seed=10, V=2048, r=32, B=3, k=4, Ncap=32, R=200, dtype="bf16"),
]


@pytest.mark.parametrize("cond", [1, 2])
@pytest.mark.parametrize("cfg", VARIANT_SMALL, ids=lambda c: "seed%d" % c["seed"])
def test_head_variants_small(rt, cfg, cond):
    """Tile mode (float32 and bf16 heads) and group mode (levels of more than 64 rows)."""
    inst = instance("tiny", strong=True, cal="monotone", rho=0.5, cond=cond, **cfg)
    _greedy_case(rt, inst, margin=STRESS_MARGIN)


# ------------------------------------------------------------------ exact ties -------------
TIES = [
    # tile mode, full vocabulary, one request
    dict(seed=31, R=1, B=16, k=4, V=151936, r=256, Ncap=64),
    # group mode (levels of more than 64 rows), several requests
    dict(seed=42, R=8, B=4, k=4, V=2048, r=64, Ncap=32),
    dict(seed=58, R=6, B=5, k=3, V=4096, r=32, Ncap=48),
    # k = 1: the argmax of two equal maxima is the lower id
    dict(seed=34, R=2, B=8, k=1, V=1000, r=16, Ncap=8),
]


@pytest.mark.parametrize("cfg", TIES, ids=lambda c: "seed%d" % c["seed"])
def test_exact_ties_lower_token_id(rt, cfg):
    """Exact ties (U = 0, logits on a 0.25 grid with equal values planted across the top-k
    cutoff): children and verify argmaxes must take the lower token id, bit for bit with the
    oracle.  Only the calibration-bin margin is certified: ranking gaps are 0 or >= 0.25."""
    import torch
    inst = inputs.make_tie_instance(**cfg)
    print("case ties", cfg, flush=True)
    ref = oracle.build_tree(inst)
    assert (ref["margins"]["q_edge"] >= 1e-3).all(), ref["margins"]["q_edge"]
    assert (ref["margins"]["key_gap"] == 0).any()  # ties are really decided
    rnd, d, got = _gpu_round(rt, inst)
    rows = list(range(inst.R))
    compare_trees(ref, got, rows)
    for i in rows:
        check_structure(inst, got, i)
    tgt = tie_targets(inst, ref, cfg["seed"])
    vres = oracle.verify_greedy(inst, ref, tgt)
    assert (vres["margins"]["argmax_gap"] == 0).all()
    out = rnd.verify_greedy(rt.target_to_device(inst, tgt))
    torch.cuda.synchronize()
    gv = {k: v.cpu().numpy() for k, v in out.items()}
    compare_verify(vres, gv, rows)


# ------------------------------------------------------------------ edge cases -------------
def test_edge_bad_root_budget_and_empty(rt):
    inst = instance("tiny", strong=True, V=500, r=8, B=3, k=2, Ncap=5, R=5, dtype="bf16")
    inst.root_token = inst.root_token.copy()
    inst.root_token[1] = inst.V      # bad root
    inst.root_token[3] = -4          # bad root
    inst.n_budget = np.array([0, 3, 9, 5, -2], np.int32)  # 9 and -2 are clamped
    rows = list(range(inst.R))
    ref = oracle.build_tree(inst, requests=rows)
    rnd, d, got = _gpu_round(rt, inst)
    compare_trees(ref, got, rows)
    assert got["status"][1] & 1 and got["status"][3] & 1
    assert got["status"][2] & 2 and got["status"][4] & 2
    assert got["n_nodes"][0] == 0 and (got["cand"][0, 0] >= 0).all()


def test_edge_single_level_and_k_equals_v(rt):
    inst = instance("tiny", strong=True, V=6, r=8, B=1, k=6, Ncap=6, R=2, dtype="f32")
    _greedy_case(rt, inst, margin=STRESS_MARGIN)


@pytest.mark.parametrize("cfg", [dict(seed=11, V=700, r=16, B=32, k=1, Ncap=32, R=2, dtype="f32"),
                                 dict(seed=12, V=1000, r=32, B=32, k=2, Ncap=64, R=3,
                                      dtype="bf16")], ids=["chain", "tree"])
def test_edge_deepest_path_accepted(rt, cfg):
    """Targets planted to choose the drafted child along each tree's deepest path (B = 32):
    the greedy walk accepts the whole path (all 32 blocks on the chain) and emits the leaf's
    own target choice, as the oracle does."""
    import torch
    inst = instance("tiny", strong=True, cal="monotone", rho=0.5, **cfg)
    print("case deepest path", cfg, flush=True)
    inst, ref = certified(inst, margin=STRESS_MARGIN)
    rnd, d, got = _gpu_round(rt, inst)
    rows = list(range(inst.R))
    compare_trees(ref, got, rows)
    tgt = tree_targets(inst, ref, rows)
    depth = deep_path_targets(inst, ref, tgt)
    vres = oracle.verify_greedy(inst, ref, tgt)
    assert np.array_equal(vres["accept_len"], depth), (vres["accept_len"], depth)
    out = rnd.verify_greedy(rt.target_to_device(inst, tgt))
    torch.cuda.synchronize()
    gv = {k: v.cpu().numpy() for k, v in out.items()}
    compare_verify(vres, gv, rows)
    if inst.k == 1:
        assert (gv["accept_len"] == inst.B).all() and (gv["n_out"] == inst.B + 1).all()


def test_deterministic_repeat(rt):
    inst = case_instance("b7|strong=1")
    rnd, d, a = _gpu_round(rt, inst)
    rnd.build(d)
    import torch
    torch.cuda.synchronize()
    b = rt.tree_to_numpy(rnd.tree)
    for f in a:
        assert np.array_equal(a[f], b[f]), f


def test_wait_give_up_reports_timeout(rt, monkeypatch):
    """Forced from the host: DT_WAIT_LIMIT=1 makes the construction kernel's internal waits give
    up after two polls (every kernel still exits normally).  Requests of a round that gave up
    report DT_REQ_SYNC_TIMEOUT with an empty tree and the verifier emits nothing for them;
    the next round, with the default bound, is complete again."""
    import torch
    inst = instance("tiny", strong=True, V=2048, r=32, B=4, k=4, Ncap=32, R=8, dtype="bf16")
    monkeypatch.setenv("DT_WAIT_LIMIT", "1")
    rnd, d, got = _gpu_round(rt, inst)
    monkeypatch.delenv("DT_WAIT_LIMIT")
    timed_out = (got["status"] & 4) != 0
    assert timed_out.any(), got["status"]
    assert (got["n_nodes"][timed_out] == 0).all()
    assert (got["token"][timed_out] == -1).all()
    tgt = np.zeros((inst.R, inst.Ncap + 1, inst.V), np.float32)
    out = rnd.verify_greedy(rt.target_to_device(inst, tgt))
    torch.cuda.synchronize()
    assert (out["n_out"].cpu().numpy()[timed_out] == 0).all()
    assert (out["accept_len"].cpu().numpy()[timed_out] == 0).all()
    rnd.build(d)
    torch.cuda.synchronize()
    again = rt.tree_to_numpy(rnd.tree)
    assert (again["status"] & 4 == 0).all() and (again["n_nodes"] == inst.Ncap).all()
    for i in range(inst.R):
        check_structure(inst, again, i)
