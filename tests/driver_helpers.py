"""Shared set-up of the multi-round driver tests: a small Markov world and an oracle-driven
decoding loop (test infrastructure; the GPU loop is draft_tree_construction_rank_amd.driver)."""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
from draft_tree_construction_rank_amd import inputs, synth

SHAPE = dict(seed=51, R=4, B=5, k=3, V=600, r=16, Ncap=12, dtype="bf16")
LOADS = (0.0, 0.5, 0.9)
TAU_MAX, LENGTH = 0.5, 24


def world_and_base():
    base = inputs.make_instance("tiny", strong_head=True, cal="monotone", **SHAPE)
    w = synth.MarkovWorld(seed=SHAPE["seed"], R=base.R, B=base.B, V=base.V, U=base.U,
                          Wt=base.Wt, dtype=base.dtype, rho=0.8)
    return w, base


def policy(load, R, Ncap, capacity):
    """The closed form of the load policy (pinned against the library on the CPU)."""
    n = int(np.clip(np.floor((1.0 - np.float64(np.float32(load))) * capacity / R), 1, Ncap))
    return np.float32(TAU_MAX) * np.float32(load), n


def oracle_loop(world, base, load, length=LENGTH):
    """The decoding loop on the oracle: per round the policy's (tau, N), the world's block
    logits, oracle build, the world's target rows, oracle greedy verify."""
    R = base.R
    capacity = R * base.Ncap
    roots = base.root_token.astype(np.int64).copy()
    pos0 = np.zeros(R, np.int64)
    produced = [[] for _ in range(R)]
    accept = []
    for t in range(4 * length + 8):
        if all(len(p) >= length for p in produced):
            break
        tau, n = policy(load, R, base.Ncap, capacity)
        L = world.block_logits(pos0)
        Lext = np.concatenate([L, L[:, -1:]], 1)
        inst = dataclasses.replace(base, Lext=Lext, root_token=roots.astype(np.int32),
                                   n_budget=np.full(R, n, np.int32), tau=np.full(R, tau, np.float32))
        tree = oracle.build_tree(inst)
        tgt = world.target_rows(roots, pos0, tree["token"], tree["parent"], tree["depth"],
                                tree["n_nodes"], base.Ncap)
        v = oracle.verify_greedy(inst, tree, tgt)
        accept.append(v["accept_len"].copy())
        for i in range(R):
            k = int(v["n_out"][i])
            toks = [int(x) for x in v["out_tokens"][i, :k]]
            produced[i].extend(toks)
            roots[i] = toks[-1]
            pos0[i] += k
    return [p[:length] for p in produced], np.array(accept)
