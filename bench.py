#!/usr/bin/env python3
"""Benchmark: one step = one round of the whole hot path on one MI355X -- tree_build (all
levels: Markov bias, softmax, top-k, calibration, survival, select, emit) followed by
tree_verify_greedy -- for the batched draft-tree workload: R = 64 requests, B = 16, k = 4,
N = 64, V = 151936, r = 256, bf16, per-request planted-peak strength U(2, 9), stopping
threshold tau (default 0.05), greedy verification against rho = 0.8 targets.

Prints one JSON line: draft trees/s (whole job), ms per step, the roofline of the dominant
kernel (the fused expansion kernel, timed live with HIP events on the launch stream), and the
CPU oracle's rate on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--tau T] [--no-cpu-baseline] [--no-extras]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft trees/sec & µs/round (B=16,k=4,N=64,V=151936); % HBM peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
KERNEL_SOURCES = ("draft_tree_construction_rank_amd/csrc/build_kernels.hip",
                  "draft_tree_construction_rank_amd/csrc/dt_build_common.h",
                  "draft_tree_construction_rank_amd/csrc/dt_internal.h",
                  "draft_tree_construction_rank_amd/csrc/dt_mma.h",
                  "draft_tree_construction_rank_amd/csrc/dt_device.h")
COUNTERS = os.path.join(ROOT, "profiles", "k_build_counters.json")


def kernel_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def gpu_targets(inst, tree, rho, gen_seed, torch):
    """Target rows [R][Ncap+1][V] on the GPU: rho * L[depth] + sqrt(1-rho^2) * E, where E is a
    fresh draw of the block-logit law (N(0, 2) plus eight planted peaks with Zipf(1.1)
    ranks and the request's strength).  Keyed by slot (timing only, no parity use)."""
    import numpy as np
    R, N1, V = inst.R, inst.Ncap + 1, inst.V
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(gen_seed)
    E = torch.randn((R, N1, V), generator=g, device=dev, dtype=torch.float32) * 2.0
    rng = np.random.default_rng([inst.seed, 99])
    perm = np.random.default_rng([inst.seed, 3]).permutation(V)
    w = np.arange(1, V + 1, dtype=np.float64) ** -1.1
    w /= w.sum()
    cdf = np.cumsum(w)
    picks = np.searchsorted(cdf, rng.random((R, N1, 16)))  # ranks; duplicates dropped below
    idx, val = [], []
    for r in range(R):
        boosts = np.linspace(inst.strength[r], inst.strength[r] * 4.0 / 9.0, 8)
        for i in range(N1):
            seen = []
            for pk in picks[r, i]:
                if pk not in seen:
                    seen.append(pk)
                if len(seen) == 8:
                    break
            for j, pk in enumerate(seen):
                idx.append((r * N1 + i) * V + int(perm[pk]))
                val.append(boosts[j])
    flat = E.view(-1)
    flat.index_add_(0, torch.tensor(idx, device=dev, dtype=torch.int64),
                    torch.tensor(val, device=dev, dtype=torch.float32))
    depth = tree["depth"].to(torch.int64)  # [R][Ncap], 0 for empty slots
    rows_depth = torch.cat([torch.zeros((R, 1), dtype=torch.int64, device=dev), depth], 1)
    Lext = torch.from_numpy(inst.Lext).to(dev)  # [R][B+1][V]
    Lsel = torch.gather(Lext, 1, rows_depth.unsqueeze(-1).expand(R, N1, V))
    b = math.sqrt(max(0.0, 1.0 - rho * rho))
    return (rho * Lsel + b * E).to(torch.bfloat16).contiguous()


def algorithmic_bytes(inst, level_rows_per_req, n_expand) -> float:
    """Bytes the method must move in one round (algorithmic, per unit of work): the L rows
    used (one V-row per request per level at which it expands) + W once + the U rows."""
    V, r = inst.V, inst.r
    l_bytes = sum(level_rows_per_req) * V * 2
    return l_bytes + r * V * 2 + sum(n_expand) * r * 2


def run_workload(inst, tau, steps, warmup, torch, rt, B, timing=True):
    d = rt.to_device(inst, "cuda", tau=tau)
    rnd = rt.Round(inst)
    rnd.build(d)
    torch.cuda.synchronize()
    tgt = gpu_targets(inst, rnd.tree, inst.rho, 1234, torch)
    rnd.verify_greedy(tgt)
    torch.cuda.synchronize()
    tree_np = rt.tree_to_numpy(rnd.tree)
    # per request: number of levels at which it expanded = distinct depths of expanded nodes
    levels_used = []
    for i in range(inst.R):
        n = int(tree_np["n_nodes"][i])
        ds = set(int(x) for x in tree_np["depth"][i, :n] if int(x) < inst.B)
        levels_used.append(1 + len(ds))  # the root's level plus one per expanded depth
    # best-first expansion count: the root plus every tree node above the last block position
    n_expand = [1 + int((tree_np["depth"][i, :int(tree_np["n_nodes"][i])] < inst.B).sum())
                for i in range(inst.R)]
    for _ in range(warmup):
        rnd.build(d)
        rnd.verify_greedy(tgt)
    torch.cuda.synchronize()
    if timing:
        B.timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        rnd.build(d)
        rnd.verify_greedy(tgt)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kms, launches = B.timing_read() if timing else (0.0, 0)
    if timing:
        B.timing_enable(False)
    vout = {k: v.cpu().numpy() for k, v in rnd.vout.items()}
    return dict(ms_per_step=(t1 - t0) * 1e3 / steps, expand_ms=kms, expand_launches=launches,
                levels_used=levels_used, n_expand=n_expand, tree=tree_np, verify=vout,
                target=tgt, level_rows=tree_np["level_rows"].tolist())


def _events(torch, n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


def _stats(us):
    import numpy as np
    a = np.asarray(us, dtype=np.float64)
    return {"median": round(float(np.median(a)), 2), "p90": round(float(np.percentile(a, 90)), 2),
            "mean": round(float(a.mean()), 2), "n": int(a.size)}


class Flusher:
    """Streams a 512 MiB buffer (read + write) to push earlier data out of the 256 MB
    Infinity Cache (MALL) before a cold-timed round."""

    def __init__(self, torch):
        self.buf = torch.zeros((512 << 20) // 4, dtype=torch.int32, device="cuda")

    def __call__(self):
        self.buf.add_(1)


def time_calls(torch, calls, n, flusher=None):
    """Per-call event timing (µs) of each callable in `calls`, run in order n times on the
    current stream; with a flusher the MALL is flushed before every repetition."""
    evs = [_events(torch, n) for _ in calls]
    for i in range(n):
        if flusher is not None:
            flusher()
        for c, fn in enumerate(calls):
            evs[c][i][0].record()
            fn()
            evs[c][i][1].record()
    torch.cuda.synchronize()
    return [[a.elapsed_time(b) * 1e3 for a, b in ev] for ev in evs]


def build_profile(inst, torch, rt, flusher, steps=30, warmup=5, **pkw):
    """tree_build alone on one workload: warm and cold µs per call (median/p90)."""
    d = rt.to_device(inst, "cuda")
    rnd = rt.Round(inst, **pkw)
    for _ in range(warmup):
        rnd.build(d)
    torch.cuda.synchronize()
    warm = time_calls(torch, [lambda: rnd.build(d)], steps)[0]
    cold = time_calls(torch, [lambda: rnd.build(d)], max(10, steps // 3), flusher)[0]
    return {"build_us_warm": _stats(warm), "build_us_cold": _stats(cold),
            "trees_per_s": round(inst.R / (_stats(warm)["median"] * 1e-6), 1)}, rnd, d


def greedy_round_profile(inst, tau, torch, rt, flusher, steps=30, warmup=5):
    """tree_build + tree_verify_greedy per round: warm and cold medians, trees/s."""
    d = rt.to_device(inst, "cuda", tau=tau)
    rnd = rt.Round(inst)
    rnd.build(d)
    torch.cuda.synchronize()
    tgt = gpu_targets(inst, rnd.tree, inst.rho, 1234, torch)
    for _ in range(warmup):
        rnd.build(d)
        rnd.verify_greedy(tgt)
    torch.cuda.synchronize()
    bw, vw = time_calls(torch, [lambda: rnd.build(d), lambda: rnd.verify_greedy(tgt)], steps)
    bc, vc = time_calls(torch, [lambda: rnd.build(d), lambda: rnd.verify_greedy(tgt)],
                        max(10, steps // 3), flusher)
    rw = [a + b for a, b in zip(bw, vw)]
    rc = [a + b for a, b in zip(bc, vc)]
    tn = rt.tree_to_numpy(rnd.tree)
    return {"round_us_warm": _stats(rw), "round_us_cold": _stats(rc),
            "build_us_warm": _stats(bw), "verify_us_warm": _stats(vw),
            "trees_per_s": round(inst.R / (_stats(rw)["median"] * 1e-6), 1),
            "mean_nodes": round(float(tn["n_nodes"].mean()), 2),
            "mean_expansions": round(float(tn["n_expand"].mean()), 2),
            "mean_accept_len": round(float(rnd.vout["accept_len"].float().mean()), 3),
            "level_rows": tn["level_rows"].tolist()}


def sample_round_us(torch, rt, inputs, temperature, flusher, steps=20, warmup=3):
    """Lossless-sampling round on the sample workload (R=32, B=16, k=4, N=64, V=151936):
    tree_build in sample mode (Gumbel-top-k siblings) followed by tree_verify_sample
    (recursive rejection) against rho=0.7 targets; also the two parts."""
    inst = inputs.make_instance("sample", temperature=temperature)
    d = rt.to_device(inst, "cuda")
    rnd = rt.Round(inst)
    rnd.build(d)
    torch.cuda.synchronize()
    tgt = gpu_targets(inst, rnd.tree, inst.rho, 4321, torch)
    for _ in range(warmup):
        rnd.build(d)
        rnd.verify_sample(d, tgt)
    torch.cuda.synchronize()
    bw, vw = time_calls(torch, [lambda: rnd.build(d), lambda: rnd.verify_sample(d, tgt)], steps)
    bc, vc = time_calls(torch, [lambda: rnd.build(d), lambda: rnd.verify_sample(d, tgt)],
                        max(10, steps // 2), flusher)
    acc = float(rnd.vout["accept_len"].float().mean())
    return {"round_us_warm": _stats([a + b for a, b in zip(bw, vw)]),
            "round_us_cold": _stats([a + b for a, b in zip(bc, vc)]),
            "build_us_warm": _stats(bw), "verify_us_warm": _stats(vw),
            "trees_per_s": round(inst.R / (_stats([a + b for a, b in zip(bw, vw)])["median"] * 1e-6), 1),
            "mean_accept_len": round(acc, 3)}


def _hashed_normal(torch, keys, V, sd):
    """N(0, sd) rows keyed by int64 `keys` (one row per key): SplitMix64-style mixing of
    (key, column) to a uniform, then the inverse normal CDF.  Bench input synthesis only."""
    M = (1 << 64) - 1
    c1, c2, g = 0xBF58476D1CE4E5B9, 0x94D049BB133111EB, 0x9E3779B97F4A7C15

    def s64(x):  # as signed int64
        return x - (1 << 64) if x >= (1 << 63) else x

    def srl(z, k):  # logical right shift of int64
        return (z >> k) & ((1 << (64 - k)) - 1)

    def mix(z):
        z = z + s64(g)
        z = (z ^ srl(z, 30)) * s64(c1)
        z = (z ^ srl(z, 27)) * s64(c2)
        return z ^ srl(z, 31)

    cols = torch.arange(V, device=keys.device, dtype=torch.int64)
    z = mix(mix(keys.view(-1, 1)) ^ cols.view(1, -1))
    u = (srl(z, 40).to(torch.float64) + 0.5) / float(1 << 24)
    return (torch.erfinv(2.0 * u - 1.0) * (math.sqrt(2.0) * sd)).to(torch.float32)


def markov_target(torch, inst, d, tree, rho):
    """Target rows [R][N+1][V] of a Markov target model: row(v) = rho * (L[d_v] + U[t_v].W)
    + sqrt(1 - rho^2) * E(request, d_v, t_v), a function of the node's depth and token only,
    so every tree variant is verified against the same model."""
    R, N1, V = inst.R, tree["token"].shape[1] + 1, inst.V
    dev = d.L.device
    tok = torch.cat([d.root_token.view(R, 1).to(torch.int64), tree["token"].to(torch.int64)], 1)
    dep = torch.cat([torch.zeros((R, 1), dtype=torch.int64, device=dev),
                     tree["depth"].to(torch.int64)], 1)
    tok = torch.where(tok >= 0, tok, tok[:, :1].expand_as(tok))  # empty slots: the root
    out = torch.empty((R, N1, V), dtype=torch.bfloat16, device=dev)
    b = math.sqrt(max(0.0, 1.0 - rho * rho))
    Wt = d.Wt.float()
    for r in range(R):
        bias = d.U[tok[r]].float() @ Wt.t()                                  # [N1][V]
        Lrow = d.L[r].float()[dep[r].clamp(max=inst.B - 1)]                  # [N1][V]
        keys = (r * 1000003 + dep[r]) * 4000037 + tok[r]
        out[r] = (rho * (Lrow + bias) + b * _hashed_normal(torch, keys, V, 2.0)).to(torch.bfloat16)
    return out


def mechanism_isolation(torch, rt, inputs, rho=0.8):
    """Chain (k = 1), Shared-Markov (chain head), parent-conditioned and marginal (no head)
    trees of the batched workload with a strong head (R = 64, B = 16, N = 64, k = 4,
    tau = 0), greedily verified against one Markov target: mean accepted draft nodes."""
    import numpy as np
    from draft_tree_construction_rank_amd import binding as Bd
    inst = inputs.make_instance("batched", strong_head=True, tau=0.0)
    d = rt.to_device(inst, "cuda", tau=0.0)
    out = {}
    variants = [("chain_k1", dict(k=1, Ncap=inst.B, cond=Bd.DT_COND_PARENT)),
                ("shared_markov", dict(cond=Bd.DT_COND_CHAIN)),
                ("pctree", dict(cond=Bd.DT_COND_PARENT)),
                ("marginal", dict(cond=Bd.DT_COND_NONE))]
    for name, kw in variants:
        rnd = rt.Round(inst, **kw)
        nb = torch.full((inst.R,), rnd.p.Ncap, dtype=torch.int32, device="cuda")
        dd = rt.DeviceInputs(L=d.L, U=d.U, Wt=d.Wt, root_token=d.root_token, n_budget=nb, tau=d.tau)
        rnd.build(dd)
        torch.cuda.synchronize()
        tgt = markov_target(torch, inst, d, rnd.tree, rho)
        rnd.verify_greedy(tgt)
        torch.cuda.synchronize()
        acc = rnd.vout["accept_len"].float().cpu().numpy()
        us = time_calls(torch, [lambda: rnd.build(dd)], 10)[0]
        out[name] = {"mean_accept_len": round(float(acc.mean()), 3),
                     "sem": round(float(acc.std(ddof=1) / np.sqrt(len(acc))), 3),
                     "tree_build_us_median": _stats(us)["median"]}
        del tgt
    # the two-stage M-ary tree (M = k = 4) on the same inputs and target
    rnd = rt.Round(inst)
    nb = torch.full((inst.R,), rnd.p.Ncap, dtype=torch.int32, device="cuda")
    fws = torch.empty(Bd.dt_flash_workspace_bytes(rnd.p), dtype=torch.uint8, device="cuda")
    fcall = lambda: Bd.tree_build_flash(rnd.p, d.L, d.U, d.Wt, d.root_token, nb, d.tau, rnd.tree, fws)
    fcall()
    torch.cuda.synchronize()
    tgt = markov_target(torch, inst, d, rnd.tree, rho)
    rnd.verify_greedy(tgt)
    torch.cuda.synchronize()
    acc = rnd.vout["accept_len"].float().cpu().numpy()
    us = time_calls(torch, [fcall], 10)[0]
    out["treeflash_m4"] = {"mean_accept_len": round(float(acc.mean()), 3),
                           "sem": round(float(acc.std(ddof=1) / np.sqrt(len(acc))), 3),
                           "tree_build_us_median": _stats(us)["median"]}
    return out


def flash_profile(torch, rt, inputs, flusher, steps=30):
    """tree_build_flash (M = 4, tau = 0) on the b7, b16 and batched workloads: warm and cold
    µs per call; per call the MFMA flops of the state pass (R * (1 + M (B - 1)) states of
    2 r V each) and its algorithmic bytes (every block row once, W once, the states' U rows)."""
    from draft_tree_construction_rank_amd import binding as Bd
    out = {}
    for name in ("b7", "b16", "batched"):
        inst = inputs.make_instance(name, tau=0.0)
        d = rt.to_device(inst, "cuda", tau=0.0)
        p = rt.params_for(inst)
        tree = Bd.alloc_tree(p, "cuda")
        ws = torch.empty(Bd.dt_flash_workspace_bytes(p), dtype=torch.uint8, device="cuda")
        call = lambda: Bd.tree_build_flash(p, d.L, d.U, d.Wt, d.root_token, d.n_budget, d.tau, tree, ws)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        warm = _stats(time_calls(torch, [call], steps)[0])
        cold = _stats(time_calls(torch, [call], max(10, steps // 3), flusher)[0])
        ns = inst.R * (1 + inst.k * (inst.B - 1))
        flops = 2.0 * ns * inst.r * inst.V
        byts = float(inst.R * inst.B * inst.V * 2 + inst.r * inst.V * 2 + ns * inst.r * 2)
        t = warm["median"] * 1e-6
        out[name] = {"R": inst.R, "B": inst.B, "M": inst.k, "N": inst.Ncap, "states": ns,
                     "build_us_warm": warm, "build_us_cold": cold,
                     "trees_per_s": round(inst.R / t, 1),
                     "mean_nodes": float(tree["n_nodes"].float().mean().item()),
                     "mfma_tflops": round(flops / t / 1e12, 1),
                     "mfma_frac": round(flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "alg_gbs": round(byts / t / 1e9, 1),
                     "hbm_frac": round(byts / t / 1e9 / HBM_PEAK_GBS, 4)}
        del d, tree, ws
    return out


def load_sweep(torch, rt, inputs, loads=(0.0, 0.5, 0.8, 0.95), length=64):
    """Multi-round decoding of the batched workload's shape (R = 64, B = 16, k = 4, N = 64,
    V = 151936, strong head) on the synthetic Markov world.  The calibration table is first
    fitted to the world (acceptance rate of drafted edges per q bin, from rounds at no
    load); then per load level the policy's threshold and budget, rounds per sample (rounds
    to emit `length` tokens), accepted tokens per round, nodes per tree and the build +
    verify time per round; a chain (k = 1) at no load for reference."""
    from draft_tree_construction_rank_amd import driver, synth
    inst = inputs.make_instance("batched", strong_head=True, tau=0.0)
    U = torch.from_numpy(inst.U).cuda().to(torch.bfloat16)
    Wt = torch.from_numpy(inst.Wt).cuda().to(torch.bfloat16)
    world = synth.TorchMarkovWorld(torch, seed=7, R=inst.R, B=inst.B, V=inst.V, U=U, Wt=Wt,
                                   rho=0.8)

    def bl(pos0):
        return world.block_logits(torch.from_numpy(pos0).cuda())

    def tr(roots, pos0, tree):
        return world.target_rows(torch.from_numpy(roots).cuda(), torch.from_numpy(pos0).cuda(), tree)

    out = {}
    # calibration: edges drafted at visited nodes in rounds at no load, binned by q
    p0 = rt.params_for(inst)
    cal_run = driver.run(p0, U=U, Wt=Wt, roots=inst.root_token, length=24,
                         load_of_round=lambda t: 0.0, tau_max=0.5, capacity=inst.R * p0.Ncap,
                         block_logits=bl, target_rows=tr, collect_edges=True)
    cal = driver.fit_calibration(cal_run.edge_q, cal_run.edge_acc, prior=inst.cal)
    out["calibration"] = {"edges": int(cal_run.edge_q.size),
                          "table": [round(float(x), 4) for x in cal]}
    runs = [("load%g" % ld, ld, {}) for ld in loads] + [("chain_k1_load0", 0.0, dict(k=1, Ncap=inst.B))]
    for name, ld, kw in runs:
        p = rt.params_for(inst, **kw)
        for i in range(16):
            p.cal[i] = float(cal[i])
        res = driver.run(p, U=U, Wt=Wt, roots=inst.root_token, length=length,
                         load_of_round=lambda t, ld=ld: ld, tau_max=0.5,
                         capacity=inst.R * p.Ncap, block_logits=bl, target_rows=tr)
        sm = res.summary()
        sm.update({"tau": float(res.tau[0]), "n_budget": int(res.n_budget[0]),
                   "tokens_per_s_build_verify": round(
                       float(res.n_out.sum()) / ((res.build_us.sum() + res.verify_us.sum()) * 1e-6), 1)})
        out[name] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in sm.items()}
    return out


def kbuild_fractions(inst, res, B):
    """HBM and MFMA fractions of k_build for a measured workload (alg bytes and flops per
    launch over the event-timed average launch)."""
    steps_launch = max(1, res["expand_launches"])
    avg_us = res["expand_ms"] * 1e3 / steps_launch
    alg = algorithmic_bytes(inst, res["levels_used"], res["n_expand"])
    flops = sum(res["n_expand"]) * 2.0 * inst.r * inst.V
    return {"k_build_avg_us": round(avg_us, 2), "alg_bytes_per_launch": int(alg),
            "hbm_gbs": round(alg / (avg_us * 1e-6) / 1e9, 1),
            "hbm_frac": round(alg / (avg_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_flops_per_launch": int(flops),
            "mfma_tflops": round(flops / (avg_us * 1e-6) / 1e12, 2),
            "mfma_frac": round(flops / (avg_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def host_model():
    try:
        return [ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo")
                if ln.startswith("model name")][0]
    except Exception:
        return platform.processor()


class pinned_single_thread:
    """Runs the oracle single-threaded on one core: the calling thread's affinity is set to
    one CPU (the first one this process may use) and oracle calls run without a pool."""

    def __enter__(self):
        self.old_aff = os.sched_getaffinity(0)
        self.core = min(self.old_aff)
        os.sched_setaffinity(0, {self.core})
        self.old_env = os.environ.get("DT_ORACLE_THREADS")
        os.environ["DT_ORACLE_THREADS"] = "1"
        return self

    def __exit__(self, *a):
        os.sched_setaffinity(0, self.old_aff)
        if self.old_env is None:
            os.environ.pop("DT_ORACLE_THREADS", None)
        else:
            os.environ["DT_ORACLE_THREADS"] = self.old_env


def cpu_baseline(inst, tau, res, budget_s=15.0):
    """The oracle, as it stands, on a bounded sample: build + greedy verify of the first
    requests of the same workload until ~budget_s of CPU time, single thread on one core."""
    import oracle
    oracle.build(force=False)
    tgt = res["target"]
    with pinned_single_thread() as pin:
        done, t0 = 0, time.perf_counter()
        while done < inst.R and time.perf_counter() - t0 < budget_s:
            row = tgt[done:done + 1].float().cpu().numpy()
            tr = oracle.build_tree(inst, requests=[done], tau=tau)
            oracle.verify_greedy(inst, tr, row)
            done += 1
        dt = time.perf_counter() - t0
    return {"value": round(done / dt, 3), "unit": "trees/s", "cores": 1, "kind": "oracle",
            "sample": "first %d of %d requests of the same workload (build + greedy verify), "
                      "%.1f s, one thread pinned to CPU %d; host %s, nproc %d" % (
                          done, inst.R, dt, pin.core, host_model(), len(os.sched_getaffinity(0)))}


def oracle_per_config(inputs, rounds=3):
    """The oracle's µs per round (build, one thread, one core; median of `rounds`) on the
    single-request workloads."""
    import numpy as np
    import oracle
    out = {}
    with pinned_single_thread():
        for name in ("tiny", "b7", "b16"):
            inst = inputs.make_instance(name)
            ts = []
            for _ in range(rounds):
                t0 = time.perf_counter()
                oracle.build_tree(inst)
                ts.append((time.perf_counter() - t0) * 1e6)
            med = float(np.median(ts))
            out[name] = {"build_us_median": round(med, 1), "trees_per_s": round(1e6 / med, 3)}
    return out


# ---------------------------------------------------------------- tree attention ----------
ATTN_WORKLOADS = {
    # name: (R, Hq, Hkv, Ncap, ctx_lo, ctx_hi)
    "batched_R64_N64": (64, 32, 8, 64, 512, 2048),
    "R1_N64_ctx2048": (1, 32, 8, 64, 2048, 2048),
    "R1_N32_ctx1024": (1, 32, 8, 32, 1024, 1024),
    "batched_R64_N64_14b": (64, 40, 8, 64, 512, 2048),
}


def _attn_inputs(torch, R, Hq, Hkv, Ncap, ctx_lo, ctx_hi, seed=7):
    """Device inputs drawn directly on the GPU (N(0,1) bf16), random full trees of Ncap
    nodes (parent uniform over the root and earlier nodes), ancestor masks and depths built
    here on the host."""
    import numpy as np
    rng = np.random.default_rng(seed)
    ctx = rng.integers(ctx_lo, ctx_hi + 1, size=R).astype(np.int32)
    Cmax = ctx_hi + Ncap + 1
    par = np.full((R, Ncap), -1, np.int64)
    depth = np.zeros((R, Ncap), np.int64)
    masks = np.zeros((R, Ncap), np.uint64)
    for r in range(R):
        m = [0] * Ncap
        for i in range(Ncap):
            p = int(rng.integers(-1, i)) if i else -1
            par[r, i] = p
            depth[r, i] = 1 + (depth[r, p] if p >= 0 else 0)
            m[i] = (m[p] if p >= 0 else 0) | (1 << i)
        masks[r] = np.array(m, dtype=np.uint64)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    D = 128
    Q = torch.randn((R, Hq, Ncap + 1, D), generator=g, device="cuda").to(torch.bfloat16)
    K = torch.randn((R, Hkv, Cmax, D), generator=g, device="cuda").to(torch.bfloat16)
    V = torch.randn((R, Hkv, Cmax, D), generator=g, device="cuda").to(torch.bfloat16)
    return dict(Q=Q, K=K, V=V, O=torch.empty_like(Q), Cmax=Cmax, ctx=ctx, depth=depth,
                ctx_d=torch.from_numpy(ctx).cuda(),
                n_d=torch.full((R,), Ncap, dtype=torch.int32, device="cuda"),
                anc_d=torch.from_numpy(masks.view(np.int64)).cuda())


def attention_profile(torch, B, flusher, steps=30):
    """tree_attention alone: warm and cold µs per call, algorithmic HBM bytes (K and V of
    every used slot once, Q and O) and MFMA flops (4 * D per visible (query, key) pair) per
    call, and the fractions of the HBM and bf16 MFMA peaks."""
    out = {}
    for name, (R, Hq, Hkv, Ncap, lo, hi) in ATTN_WORKLOADS.items():
        d = _attn_inputs(torch, R, Hq, Hkv, Ncap, lo, hi)
        p = B.make_attn_params(R=R, Hq=Hq, Hkv=Hkv, D=128, Ncap=Ncap, Cmax=d["Cmax"],
                               scale=1.0 / math.sqrt(128))
        ws = B.alloc_attn_workspace(p, "cuda")
        call = lambda: B.tree_attention(p, d["Q"], d["K"], d["V"], d["ctx_d"], d["n_d"],
                                        d["anc_d"], d["O"], ws)
        for _ in range(5):
            call()
        torch.cuda.synchronize()
        warm = _stats(time_calls(torch, [call], steps)[0])
        cold = _stats(time_calls(torch, [call], max(10, steps // 3), flusher)[0])
        keys = d["ctx"].astype("int64") + Ncap + 1
        byts = float(Hkv * keys.sum() * 128 * 2 * 2 + 2 * R * Hq * (Ncap + 1) * 128 * 2)
        # visible keys: the root query sees ctx + 1 slots, node i sees ctx + 1 + depth_i
        vis = float((d["ctx"].astype("int64") + 1).sum() * (Ncap + 1) + d["depth"].sum())
        flops = 4.0 * 128 * Hq * vis
        t = warm["median"] * 1e-6
        out[name] = {"R": R, "Hq": Hq, "Hkv": Hkv, "N": Ncap, "ctx": [lo, hi],
                     "us_warm": warm, "us_cold": cold,
                     "workspace_bytes": B.dt_attn_workspace_bytes(p),
                     "alg_bytes": int(byts), "alg_flops": int(flops),
                     "hbm_gbs": round(byts / t / 1e9, 1),
                     "hbm_frac": round(byts / t / 1e9 / HBM_PEAK_GBS, 4),
                     "mfma_tflops": round(flops / t / 1e12, 1),
                     "mfma_frac": round(flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        del d, ws
        torch.cuda.empty_cache()
    return out


def attention_oracle_rate():
    """The float64 oracle on the host for one request of the batched workload (all 32 query
    heads, 65 tree positions, context 1280): requests per second on one core."""
    import numpy as np
    import oracle.attention as oa
    from draft_tree_construction_rank_amd import attn_inputs
    inst = attn_inputs.make_attn_instance(seed=5, R=1, Hq=32, Hkv=8, D=128, Ncap=64,
                                          ctx_lo=1280, ctx_hi=1280, threads=1)
    Q, K, V = inst.f32("Q"), inst.f32("K"), inst.f32("V")
    t0 = time.perf_counter()
    oa.tree_attention(Q, K, V, inst.ctx_len, inst.n_nodes, inst.parent, inst.scale)
    dt = time.perf_counter() - t0
    return {"requests_per_s": round(1.0 / dt, 3), "cores": 1,
            "sample": "one request, 32 query heads x 65 tree positions, context 1280"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--tau", type=float, default=0.05)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter scaling)")
    ap.add_argument("--attention-only", nargs="*", metavar="WORKLOAD", default=None,
                    help="time only tree_attention on the named workloads (all if none given) "
                         "and print their JSON; for profiling")
    ap.add_argument("--flash-only", action="store_true",
                    help="time only tree_build_flash on the b7, b16 and batched workloads and "
                         "print their JSON; for profiling")
    ap.add_argument("--sample-only", type=float, nargs="*", metavar="T", default=None,
                    help="time only the lossless-sampling round (tree_build in sample mode + "
                         "tree_verify_sample) at the given temperatures (1.0 if none given) "
                         "and print their JSON; for profiling")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (requests shard "
              "across GPUs without communication). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from draft_tree_construction_rank_amd import binding as B
    from draft_tree_construction_rank_amd import inputs
    from draft_tree_construction_rank_amd import runner as rt

    B.lib()  # fail loudly if the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.copy_calibration:
        x = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        del x, y

    if args.attention_only is not None:
        global ATTN_WORKLOADS
        names = args.attention_only or list(ATTN_WORKLOADS)
        ATTN_WORKLOADS = {k: v for k, v in ATTN_WORKLOADS.items() if k in names}
        print(json.dumps(attention_profile(torch, B, Flusher(torch))), flush=True)
        return
    if args.flash_only:
        print(json.dumps({"tree_build_flash": flash_profile(torch, rt, inputs, Flusher(torch),
                                                            steps=args.steps)}), flush=True)
        return
    if args.sample_only is not None:
        fl = Flusher(torch)
        for T in args.sample_only or [1.0]:
            r = sample_round_us(torch, rt, inputs, T, fl, steps=args.steps, warmup=args.warmup)
            print(json.dumps({"sample_round": {"temperature": T, **r}}), flush=True)
        return

    inst = inputs.make_instance("batched", tau=args.tau)
    res = run_workload(inst, args.tau, args.steps, args.warmup, torch, rt, B)
    ms = res["ms_per_step"]
    value = inst.R / (ms * 1e-3)
    # roofline of the dominant kernel: the persistent construction kernel k_build (one
    # launch per round), timed with HIP events on the launch stream
    launches_per_step = res["expand_launches"] / args.steps
    avg_us = res["expand_ms"] * 1e3 / max(1, res["expand_launches"])
    round_bytes = algorithmic_bytes(inst, res["levels_used"], res["n_expand"])
    per_launch_bytes = round_bytes / launches_per_step
    achieved = per_launch_bytes / (avg_us * 1e-6) / 1e9
    traffic = None
    if os.path.exists(COUNTERS):
        c = json.load(open(COUNTERS))
        if c.get("kernel_sha") == kernel_sha() and c.get("tau") == args.tau:
            traffic = c.get("hbm_bytes_per_launch")
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "k_build (persistent level loop: MFMA Markov bias + online softmax + "
                      "top-k per vocabulary split, merge, calibration, survival, select, emit)",
            "avg_launch_us": round(avg_us, 3), "launches_per_step": launches_per_step,
            "alg_bytes_per_launch": int(per_launch_bytes)}
    line = {"metric": METRIC, "value": round(value, 1), "unit": "trees/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "batched draft-tree round: tree_build + tree_verify_greedy, "
                                   "R=64, B=16, k=4, N=64, V=151936, r=256, tau=%g" % args.tau,
                       "R": inst.R, "B": inst.B, "k": inst.k, "N": inst.Ncap, "V": inst.V,
                       "r": inst.r, "tau": args.tau},
            "us_per_round": round(ms * 1e3, 2),
            "roofline": roof,
            "tree_stats": {"mean_nodes": float(res["tree"]["n_nodes"].mean()),
                           "mean_expansions": float(sum(res["n_expand"]) / inst.R),
                           "mean_accept_len": float(res["verify"]["accept_len"].mean()),
                           "level_rows": res["level_rows"]}}
    if not args.no_extras:
        flusher = Flusher(torch)
        extras = {}
        # the headline workload per round: warm and cold (MALL flushed), median and p90
        extras["headline_per_round"] = greedy_round_profile(inst, args.tau, torch, rt, flusher)
        # full trees: tau = 0 keeps 64 nodes per request (65 expansions each), the regime
        # where the expansion's MFMA work binds
        full = run_workload(inst, 0.0, 20, 3, torch, rt, B)
        fx = kbuild_fractions(inst, full, B)
        fx.update(greedy_round_profile(inst, 0.0, torch, rt, flusher))
        extras["batched_tau0_full_trees"] = fx
        for t in (0.2, 0.5):
            if t != args.tau:
                r2 = run_workload(inst, t, 20, 3, torch, rt, B)
                e = kbuild_fractions(inst, r2, B)
                e["trees_per_s"] = round(inst.R / (r2["ms_per_step"] * 1e-3), 1)
                e["us_per_round"] = round(r2["ms_per_step"] * 1e3, 2)
                extras["batched_tau%g" % t] = e
        # single-request workloads: tree_build latency, warm and cold
        per = {}
        for name in ("tiny", "b7"):
            per[name] = build_profile(inputs.make_instance(name), torch, rt, flusher)[0]
        h = inputs.make_instance("b16")
        sweep = {}
        for k in (1, 2, 4, 8):
            for n in (16, 32, 64):
                hk = inputs.make_instance("b16", k=k, Ncap=n) if (k, n) != (4, 64) else h
                sweep["k%d_N%d" % (k, n)] = build_profile(hk, torch, rt, flusher)[0]
        per["b16_sweep"] = sweep
        extras["per_config"] = per
        extras["tree_build_us_R1_B16_k4_N64"] = sweep["k4_N64"]["build_us_warm"]["median"]
        extras["sample"] = {"T%g" % T: sample_round_us(torch, rt, inputs, T, flusher)
                            for T in (0.6, 1.0, 1.5)}
        extras["mechanism_isolation_markov_target"] = mechanism_isolation(torch, rt, inputs)
        extras["multi_round_load_sweep"] = load_sweep(torch, rt, inputs)
        extras["tree_attention"] = attention_profile(torch, B, flusher)
        extras["tree_build_flash"] = flash_profile(torch, rt, inputs, flusher)
        if not args.no_cpu_baseline:
            extras["tree_attention"]["oracle"] = attention_oracle_rate()
        extras["targets"] = {
            "tree_build_us_R1_B16_k4_N64": {"measured_median": extras["tree_build_us_R1_B16_k4_N64"],
                                            "target": 100.0,
                                            "met": extras["tree_build_us_R1_B16_k4_N64"] < 100.0},
            "batched_hbm_frac_target": 0.6,
            "batched_hbm_frac": {("tau%g" % t): (roof["frac"] if t == args.tau else
                                                 extras.get("batched_tau%g" % t, {}).get("hbm_frac"))
                                 for t in (0.05, 0.2, 0.5)},
            "batched_full_trees": {"hbm_frac": fx["hbm_frac"], "mfma_frac": fx["mfma_frac"]}}
        if not args.no_cpu_baseline:
            extras["oracle_per_config"] = oracle_per_config(inputs)
        line["extras"] = extras
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inst, args.tau, res)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
