"""Pins for the oracle's counter-based randomness (no GPU).

Philox4x32-10 is pinned to the published known-answer vectors; the SplitMix64 output mix
to the reference generator's first outputs; the uniform map to its closed form and to a
Kolmogorov-Smirnov test; the Gumbel transform to the Gumbel law.
"""
import os

import numpy as np
import pytest
from scipy import stats

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLD, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_philox_known_answers():
    rows = _rows("philox4x32_10_kat.txt")
    assert len(rows) == 3
    for r in rows:
        v = [int(x, 16) for x in r]
        out = oracle.philox(v[0:4], v[4:6])
        assert [int(x) for x in out] == v[6:10]


def test_splitmix64_sequence():
    want = [int(r[0], 16) for r in _rows("splitmix64_seq.txt")]
    gamma = 0x9E3779B97F4A7C15
    got = [oracle.mix64((i * gamma) & (2**64 - 1)) for i in range(len(want))]
    assert got == want


def test_uniform_closed_form():
    # u = ((word >> 8) + 0.5) * 2^-24 with word = philox(ctr=(i/4, stream, lo h, hi h), key=seed)
    seed, h = 0x1234_5678_9ABC_DEF0, 0x0FED_CBA9_8765_4321
    for i in range(12):
        w = oracle.philox([i >> 2, 2, h & 0xFFFFFFFF, h >> 32],
                          [seed & 0xFFFFFFFF, seed >> 32])[i & 3]
        assert oracle.uniform(seed, h, 2, i) == ((int(w) >> 8) + 0.5) / 2.0**24


def test_uniform_law():
    u = np.array([oracle.uniform(7, oracle.mix64(j), 1, i) for j in range(50) for i in range(400)])
    assert u.min() > 0.0 and u.max() < 1.0
    assert stats.kstest(u, "uniform").pvalue > 1e-3


def test_gumbel_law():
    u = np.array([oracle.uniform(11, oracle.mix64(j), 3, i) for j in range(40) for i in range(500)])
    g = -np.log(-np.log(u))
    assert stats.kstest(g, "gumbel_r").pvalue > 1e-3


def test_hash_depends_on_path_not_slot():
    h0 = oracle.root_hash(3, 5, 17)
    assert oracle.root_hash(3, 5, 17) == h0
    assert oracle.root_hash(4, 5, 17) != h0
    assert oracle.root_hash(3, 6, 17) != h0
    assert oracle.root_hash(3, 5, 18) != h0
    a = oracle.child_hash(oracle.child_hash(h0, 1), 2)
    b = oracle.child_hash(oracle.child_hash(h0, 2), 1)
    assert a != b
