"""Multi-round decoding driver with the load-adaptive tree policy (argument marshalling and
orchestration only: every tree is built and verified by libdtree's kernels).

One round for R requests: the policy (dt_load_policy) turns the current load into each
request's stopping threshold tau and node budget N; the drafter's block logits for the
round come from the world; tree_build builds the trees; the world gives the target's rows
for the emitted trees; tree_verify_greedy walks them.  Each request appends its emitted
tokens (accepted draft tokens and the target's own next token), whose last becomes the
next round's root.  The driver records per round accepted lengths, tree sizes and kernel
times, and per request the number of rounds it took to emit `length` tokens ("rounds per
sample").  TreeSpark article, core idea: the load-adaptive serving policy; PCTree summary,
analysis paragraph: rounds per sample.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, List, Optional

import numpy as np
import torch

from . import binding as B


@dataclasses.dataclass
class DriverResult:
    tokens: List[List[int]]   # per request, the first `length` emitted tokens
    rounds_to_length: np.ndarray  # [R] rounds each request needed to emit `length` tokens
    accept_len: np.ndarray    # [rounds][R]
    n_nodes: np.ndarray       # [rounds][R]
    n_out: np.ndarray         # [rounds][R]
    tau: np.ndarray           # [rounds] threshold of the round
    n_budget: np.ndarray      # [rounds] node budget of the round
    build_us: np.ndarray      # [rounds] tree_build time (HIP events; 0 without timing)
    verify_us: np.ndarray     # [rounds] tree_verify_greedy time
    edge_q: Optional[np.ndarray] = None    # drafted edges at visited nodes: q of the child
    edge_acc: Optional[np.ndarray] = None  # and whether the target took that child (0/1)

    def summary(self) -> dict:
        acc = self.accept_len.astype(np.float64)
        return {"rounds_per_sample": float(self.rounds_to_length.mean()),
                "mean_accept_len": float(acc.mean()),
                "tokens_per_round": float(self.n_out.mean()),
                "mean_nodes": float(self.n_nodes.mean()),
                "build_us_mean": float(self.build_us.mean()),
                "verify_us_mean": float(self.verify_us.mean())}


def fit_calibration(q: np.ndarray, acc: np.ndarray, prior: Optional[np.ndarray] = None) -> np.ndarray:
    """Calibration table from observed edges (TreeSpark article, core idea: the
    parent-conditioned probability is calibrated to an edge-acceptance estimate).  Reading:
    the lookup's own 16 equal-width bins on q, the acceptance rate per bin, made
    non-decreasing by pool-adjacent-violators weighted by the bin counts; a bin without
    edges takes the value of the nearest bin below it (the prior's entry if none)."""
    q = np.asarray(q, np.float64)
    acc = np.asarray(acc, np.float64)
    b = np.minimum(15, np.floor(16.0 * q).astype(np.int64))
    cnt = np.bincount(b, minlength=16).astype(np.float64)
    hit = np.bincount(b, weights=acc, minlength=16)
    # pool-adjacent-violators over the non-empty bins, in bin order
    blocks = []  # [value, weight, first bin, last bin]
    for i in range(16):
        if cnt[i] == 0:
            continue
        blocks.append([hit[i] / cnt[i], cnt[i], i, i])
        while len(blocks) > 1 and blocks[-2][0] > blocks[-1][0]:
            v2, w2, _, e2 = blocks.pop()
            v1, w1, s1, _ = blocks.pop()
            blocks.append([(v1 * w1 + v2 * w2) / (w1 + w2), w1 + w2, s1, e2])
    out = np.full(16, np.nan)
    for v, _, s0, e0 in blocks:
        out[s0:e0 + 1] = v
    last = None
    for i in range(16):
        if np.isnan(out[i]):
            out[i] = last if last is not None else (float(prior[i]) if prior is not None else 0.0)
        last = out[i]
    out = np.maximum.accumulate(np.clip(out, 0.0, 1.0))
    return out.astype(np.float32)


def run(params: B.dt_params, *, U: torch.Tensor, Wt: torch.Tensor, roots: np.ndarray,
        length: int, load_of_round: Callable[[int], float], tau_max: float, capacity: int,
        block_logits: Callable[[np.ndarray], torch.Tensor],
        target_rows: Callable[[np.ndarray, np.ndarray, dict], torch.Tensor],
        max_rounds: Optional[int] = None, timed: bool = True,
        collect_edges: bool = False) -> DriverResult:
    """Decode until every request has emitted `length` tokens (greedy verification).

    params: round parameters (R, B, k, V, r, Ncap, dtypes, cond; greedy mode).
    block_logits(pos0) -> [R][B][V] device tensor; target_rows(roots, pos0, tree) ->
    [R][Ncap+1][V] device tensor (row 0 = root).  pos0[i] is the absolute position of
    request i's root (the last emitted token), 0 at the start."""
    if params.mode != B.DT_GREEDY:
        raise ValueError("the driver verifies greedily")
    R = params.R
    dev = U.device
    ws = B.alloc_workspace(params, dev)
    tree = B.alloc_tree(params, dev)
    vout = B.alloc_verify(params, dev)
    roots = np.asarray(roots, np.int64).copy()
    pos0 = np.zeros(R, np.int64)
    produced: List[List[int]] = [[] for _ in range(R)]
    done = np.full(R, -1, np.int64)
    acc_l, nn_l, no_l, tau_l, nb_l, bus, vus = [], [], [], [], [], [], []
    eq, ea = [], []
    limit = max_rounds if max_rounds is not None else 4 * length + 8
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for t in range(limit):
        if (done >= 0).all():
            break
        tau, nb = B.load_policy(float(load_of_round(t)), R, tau_max=tau_max, capacity=capacity,
                                Ncap=params.Ncap)
        L = block_logits(pos0)
        root_d = torch.from_numpy(roots.astype(np.int32)).to(dev)
        nb_d = torch.from_numpy(nb).to(dev)
        tau_d = torch.from_numpy(tau).to(dev)
        if timed:
            ev[0].record()
        B.tree_build(params, L, U, Wt, root_d, nb_d, tau_d, tree, ws)
        if timed:
            ev[1].record()
        tgt = target_rows(roots, pos0, tree)
        if timed:
            ev[2].record()
        B.tree_verify_greedy(params, tree, tgt, vout, ws)
        end = torch.cuda.Event(enable_timing=True) if timed else None
        if timed:
            end.record()
        torch.cuda.synchronize()
        if timed:
            bus.append(ev[0].elapsed_time(ev[1]) * 1e3)
            vus.append(ev[2].elapsed_time(end) * 1e3)
        else:
            bus.append(0.0)
            vus.append(0.0)
        n_out = vout["n_out"].cpu().numpy()
        out_tok = vout["out_tokens"].cpu().numpy()
        acc_l.append(vout["accept_len"].cpu().numpy())
        nn_l.append(tree["n_nodes"].cpu().numpy())
        no_l.append(n_out)
        tau_l.append(float(tau[0]))
        nb_l.append(int(nb[0]))
        if collect_edges:
            # the children in the tree of every node the walk visited (the root first), and
            # whether each is the token the target emitted there
            tok = tree["token"].cpu().numpy()
            par = tree["parent"].cpu().numpy()
            lq = tree["logq"].cpu().numpy()
            path = vout["path"].cpu().numpy()
            for i in range(R):
                nacc = int(acc_l[-1][i])
                visited = [-1] + [int(x) for x in path[i, :nacc]]
                for j, v in enumerate(visited):
                    kids = np.nonzero(par[i, :int(nn_l[-1][i])] == v)[0]
                    eq.extend(np.exp(lq[i, kids].astype(np.float64)))
                    ea.extend((tok[i, kids] == out_tok[i, j]).astype(np.float64))
        for i in range(R):
            k = int(n_out[i])
            if k <= 0:
                raise RuntimeError("request %d emitted nothing (status %d)" % (
                    i, int(tree["status"][i].item())))
            toks = [int(x) for x in out_tok[i, :k]]
            produced[i].extend(toks)
            roots[i] = toks[-1]
            pos0[i] += k
            if done[i] < 0 and len(produced[i]) >= length:
                done[i] = t + 1
        del tgt, L
    if (done < 0).any():
        raise RuntimeError("round limit reached before every request emitted %d tokens" % length)
    return DriverResult(tokens=[p[:length] for p in produced], rounds_to_length=done,
                        accept_len=np.array(acc_l), n_nodes=np.array(nn_l),
                        n_out=np.array(no_l), tau=np.array(tau_l), n_budget=np.array(nb_l),
                        build_us=np.array(bus), verify_us=np.array(vus),
                        edge_q=np.array(eq) if collect_edges else None,
                        edge_acc=np.array(ea) if collect_edges else None)
