"""The multi-round driver on the GPU (through the C ABI) with the load policy: every request
emits exactly the target's own greedy continuation at every load level, the per-round
threshold and budget are the policy's, and the rounds-per-sample bookkeeping adds up."""
import numpy as np
import pytest

from driver_helpers import LENGTH, LOADS, TAU_MAX, policy, world_and_base

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("load", LOADS)
def test_driver_emits_the_target_greedy_sequence(load):
    import torch
    from draft_tree_construction_rank_amd import driver, runner
    assert torch.cuda.is_available()
    world, base = world_and_base()
    print("driver load %g R=%d B=%d k=%d V=%d N=%d" % (load, base.R, base.B, base.k, base.V,
                                                         base.Ncap), flush=True)
    p = runner.params_for(base)
    U = torch.from_numpy(base.U).cuda().to(torch.bfloat16)
    Wt = torch.from_numpy(base.Wt).cuda().to(torch.bfloat16)

    def block_logits(pos0):
        return torch.from_numpy(world.block_logits(pos0)).cuda().to(torch.bfloat16)

    def target_rows(roots, pos0, tree):
        t = {f: tree[f].cpu().numpy() for f in ("token", "parent", "depth", "n_nodes")}
        rows = world.target_rows(roots, pos0, t["token"], t["parent"], t["depth"], t["n_nodes"],
                                 base.Ncap)
        return torch.from_numpy(rows).cuda().to(torch.bfloat16)

    capacity = base.R * base.Ncap
    res = driver.run(p, U=U, Wt=Wt, roots=base.root_token, length=LENGTH,
                     load_of_round=lambda t: load, tau_max=TAU_MAX, capacity=capacity,
                     block_logits=block_logits, target_rows=target_rows)
    for i in range(base.R):
        assert res.tokens[i] == world.greedy_sequence(i, int(base.root_token[i]), LENGTH), i
    tau, n = policy(load, base.R, base.Ncap, capacity)
    assert (res.tau == tau).all() and (res.n_budget == n).all()
    assert (res.n_nodes <= n).all() and (res.accept_len <= base.B).all()
    assert (res.n_out == res.accept_len + 1).all()
    cum = np.cumsum(res.n_out, 0)
    for i in range(base.R):
        assert cum[res.rounds_to_length[i] - 1, i] >= LENGTH
        assert res.rounds_to_length[i] == 1 or cum[res.rounds_to_length[i] - 2, i] < LENGTH


def test_driver_edge_collection_counts_accepted_nodes():
    """Every accepted draft node is one accepted edge at a visited node, and the final
    (target) token of a round is never a child in the tree, so the accepted edges number
    exactly the accepted nodes; q is a probability."""
    import torch
    from draft_tree_construction_rank_amd import driver, runner
    world, base = world_and_base()
    p = runner.params_for(base)
    U = torch.from_numpy(base.U).cuda().to(torch.bfloat16)
    Wt = torch.from_numpy(base.Wt).cuda().to(torch.bfloat16)
    res = driver.run(p, U=U, Wt=Wt, roots=base.root_token, length=LENGTH,
                     load_of_round=lambda t: 0.0, tau_max=TAU_MAX, capacity=base.R * base.Ncap,
                     block_logits=lambda pos0: torch.from_numpy(world.block_logits(pos0)).cuda().to(torch.bfloat16),
                     target_rows=lambda roots, pos0, tree: torch.from_numpy(world.target_rows(
                         roots, pos0, *[tree[f].cpu().numpy() for f in ("token", "parent", "depth", "n_nodes")],
                         base.Ncap)).cuda().to(torch.bfloat16),
                     collect_edges=True)
    assert res.edge_q.size > 0 and ((res.edge_q > 0) & (res.edge_q <= 1)).all()
    assert int(res.edge_acc.sum()) == int(res.accept_len.sum())
    cal = driver.fit_calibration(res.edge_q, res.edge_acc, prior=base.cal)
    assert (np.diff(cal) >= 0).all() and (cal >= 0).all() and (cal <= 1).all()
