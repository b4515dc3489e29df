"""Multi-round decoding with the load policy, on the oracle (no GPU): greedy speculative
decoding is lossless, so whatever trees the load policy allows, every request must emit
exactly the target's own greedy continuation (PCTree summary: greedy verification)."""
import numpy as np
import pytest

from driver_helpers import LENGTH, LOADS, oracle_loop, world_and_base


@pytest.mark.parametrize("load", LOADS)
def test_oracle_loop_emits_the_target_greedy_sequence(load):
    world, base = world_and_base()
    toks, accept = oracle_loop(world, base, load)
    for i in range(base.R):
        assert toks[i] == world.greedy_sequence(i, int(base.root_token[i]), LENGTH)
    assert accept.min() >= 0 and accept.max() <= base.B


def test_heavier_load_accepts_less_per_round():
    """The policy shrinks the trees as load rises (smaller budgets, higher thresholds), so
    fewer draft tokens are accepted per round."""
    world, base = world_and_base()
    means = [oracle_loop(world, base, ld)[1].mean() for ld in (0.0, 0.9)]
    assert means[0] > means[1], means


def test_fit_calibration_recovers_monotone_rates():
    """Edges drawn with a known non-decreasing acceptance rate per bin: the fitted table
    recovers the rates; an out-of-order pair of bins is pooled to their weighted mean; empty
    bins take the bin below; the table stays in [0, 1] and non-decreasing."""
    from draft_tree_construction_rank_amd.driver import fit_calibration
    rng = np.random.default_rng(5)
    true = np.linspace(0.02, 0.9, 16)
    q = rng.uniform(0, 1, 400_000)
    b = np.minimum(15, np.floor(16 * q).astype(int))
    acc = (rng.uniform(0, 1, q.size) < true[b]).astype(float)
    cal = fit_calibration(q, acc)
    assert np.abs(cal - true).max() < 0.02
    assert (np.diff(cal) >= 0).all()
    # two bins out of order -> pooled (weighted mean of the two rates)
    q2 = np.array([0.10] * 100 + [0.15] * 300)          # bins 1 and 2
    a2 = np.array([1.0] * 60 + [0.0] * 40 + [1.0] * 60 + [0.0] * 240)
    cal2 = fit_calibration(q2, a2)
    assert cal2[0] == 0.0 and abs(cal2[1] - 0.3) < 1e-6 and abs(cal2[2] - 0.3) < 1e-6
    assert (cal2[3:] == cal2[2]).all()
