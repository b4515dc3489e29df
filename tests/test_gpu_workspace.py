"""A workspace's contents on entry do not matter (the calling conventions of include/dtree.h).

Every call here starts on a workspace filled with 0xFF bytes (NaN floats, all-ones
counters, tags and indices) and on outputs filled with 0xAB bytes; then a second round of
other shapes (another dtype, vocabulary, k, N or R) runs on the same workspace with the
first round's contents still in it.  Both rounds are compared with the oracle element by
element, as in the parity tests.
"""
import numpy as np
import pytest

import oracle
from oracle_helpers import check_structure
from parity_helpers import (STRESS_MARGIN, certified, compare_trees, compare_verify, instance,
                            sample_verify_margins, tree_targets)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    import torch
    from draft_tree_construction_rank_amd import runner
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return runner


def _dirty(nbytes):
    import torch
    return torch.full((max(int(nbytes), 256),), 0xFF, dtype=torch.uint8, device="cuda")


def _smear(outs):
    import torch
    for v in outs.values():
        v.view(-1).view(torch.uint8).fill_(0xAB)


def _build(rt, inst, ws):
    import torch
    rnd = rt.Round(inst)
    assert ws.numel() >= rnd.ws.numel()
    rnd.ws = ws
    _smear(rnd.tree)
    _smear(rnd.vout)
    d = rt.to_device(inst)
    rnd.build(d)
    torch.cuda.synchronize()
    got = rt.tree_to_numpy(rnd.tree)
    for i in range(inst.R):
        check_structure(inst, got, i)
    return rnd, d, got


GREEDY = [
    # group mode (levels of more than 64 rows), then tile mode with a float32 head
    dict(seed=8, V=1000, r=64, B=4, k=4, Ncap=32, R=8, dtype="bf16"),
    dict(seed=1, V=1000, r=8, B=4, k=2, Ncap=8, R=3, dtype="f32"),
]


def test_build_and_greedy_verify(rt):
    import torch
    from draft_tree_construction_rank_amd import binding
    insts = [instance("tiny", strong=True, cal="monotone", rho=0.5, **c) for c in GREEDY]
    ws = _dirty(max(binding.dt_build_workspace_bytes(rt.params_for(i)) for i in insts))
    for c, inst in zip(GREEDY, insts):
        print("case", c, flush=True)
        inst, ref = certified(inst, margin=STRESS_MARGIN)
        rnd, d, got = _build(rt, inst, ws)
        rows = list(range(inst.R))
        compare_trees(ref, got, rows)
        tgt = tree_targets(inst, ref, rows)
        vres = oracle.verify_greedy(inst, ref, tgt)
        out = rnd.verify_greedy(rt.target_to_device(inst, tgt))
        torch.cuda.synchronize()
        compare_verify(vres, {k: v.cpu().numpy() for k, v in out.items()}, rows)


SAMPLE = [
    dict(seed=12, V=1000, r=16, B=4, k=3, Ncap=12, R=4, dtype="bf16", temperature=0.6),
    dict(seed=11, V=300, r=8, B=3, k=2, Ncap=6, R=3, dtype="f32", temperature=1.0),
]


def test_sample_build_and_verify(rt):
    import torch
    from draft_tree_construction_rank_amd import binding
    insts = [instance("tiny", strong=True, cal="monotone", rho=0.7, mode="sample", **c)
             for c in SAMPLE]
    ws = _dirty(max(binding.dt_build_workspace_bytes(rt.params_for(i)) for i in insts))
    for c, inst in zip(SAMPLE, insts):
        print("case", c, flush=True)
        inst, ref = certified(inst, verify_target=sample_verify_margins, margin=STRESS_MARGIN)
        rnd, d, got = _build(rt, inst, ws)
        rows = list(range(inst.R))
        compare_trees(ref, got, rows)
        tgt = tree_targets(inst, ref, rows)
        vref = oracle.verify_sample(inst, ref, tgt)
        out = rnd.verify_sample(d, rt.target_to_device(inst, tgt))
        torch.cuda.synchronize()
        compare_verify(vref, {k: v.cpu().numpy() for k, v in out.items()}, rows)


FLASH = [
    dict(seed=21, V=130, r=16, B=8, k=4, Ncap=24, R=5, dtype="bf16"),
    dict(seed=2, V=96, r=8, B=5, k=3, Ncap=20, tau=0.0),
]


def test_flash_build(rt):
    import torch
    from draft_tree_construction_rank_amd import binding
    insts = [instance("tiny", strong=True, **dict(dict(tau=0.0), **c)) for c in FLASH]
    ws = _dirty(max(binding.dt_flash_workspace_bytes(rt.params_for(i)) for i in insts))
    for c, inst in zip(FLASH, insts):
        print("case", c, flush=True)
        inst, ref = certified(inst, margin=STRESS_MARGIN, method=oracle.BUILD_FLASH)
        p = rt.params_for(inst)
        d = rt.to_device(inst)
        tree = binding.alloc_tree(p, "cuda")
        _smear(tree)
        binding.tree_build_flash(p, d.L, d.U, d.Wt, d.root_token, d.n_budget, d.tau, tree, ws)
        torch.cuda.synchronize()
        got = rt.tree_to_numpy(tree)
        compare_trees(ref, got, list(range(inst.R)))
        np.testing.assert_array_equal(ref["n_expand"], got["n_expand"])
        for i in range(inst.R):
            check_structure(inst, got, i)


ATTN = [
    # both split their key ranges (partials in the workspace, then the combine kernel)
    dict(seed=7, R=1, Hq=8, Hkv=2, Ncap=64, ctx_lo=900, ctx_hi=1300),
    dict(seed=2, R=2, Hq=8, Hkv=2, Ncap=12, ctx_lo=300, ctx_hi=700, nodes="ragged"),
]


def test_tree_attention(rt):
    import torch
    from draft_tree_construction_rank_amd import attn_inputs, binding
    from test_gpu_attention import _compare, _dev
    insts = [attn_inputs.make_attn_instance(D=128, threads=4, **c) for c in ATTN]
    params = [binding.make_attn_params(R=i.R, Hq=i.Hq, Hkv=i.Hkv, D=i.D, Ncap=i.Ncap,
                                       Cmax=i.Cmax, scale=i.scale) for i in insts]
    need = [binding.dt_attn_workspace_bytes(p) for p in params]
    assert min(need) > 0
    ws = _dirty(max(need))
    for c, inst, p in zip(ATTN, insts, params):
        print("case", c, flush=True)
        d = _dev(inst)
        O = torch.full(tuple(d["Q"].shape), float("nan"), dtype=torch.bfloat16, device="cuda")
        binding.tree_attention(p, d["Q"], d["K"], d["V"], d["ctx"], d["n"], d["anc"], O, ws)
        torch.cuda.synchronize()
        _compare(inst, O.float().cpu().numpy())
