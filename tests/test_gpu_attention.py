"""GPU parity for tree attention: the HIP kernel (through the C ABI) against the float64
oracle, element by element.

Tolerance, from the kernel's arithmetic: Q, K, V are bf16 on both sides (the oracle reads
the same values); scores and sums accumulate in fp32 (relative error ~1e-4 at these
lengths); the probabilities are rounded to bf16 for the value product (unit roundoff
u = 2^-8), which moves an output by at most u * sum(p |v|) / sum(p) = u * M, where M is
the oracle's output over |V|; the output is rounded to bf16 (u * |O|).  The test allows
|O_gpu - O_ref| <= 2u * M + u * |O_ref| + 1e-6.  Rows past n and rows of invalid requests
must be exactly zero.

Cases cover every launch shape (4 to 9 wavefronts, 32- and 64-key blocks, one to four
query groups, single and split key ranges with the combine kernel), ragged context lengths
and trees, chain/star/random trees, empty trees, zero context, peaked scores, invalid
requests, and the full workload (64 requests, 32 query heads over 8 key/value heads,
N = 64, contexts of 512..2048) in the launch configuration the benchmark times.
"""
import numpy as np
import pytest

from draft_tree_construction_rank_amd import attn_inputs
from oracle import attention as oa

pytestmark = pytest.mark.gpu

U = 2.0 ** -8


@pytest.fixture(scope="module")
def B():
    import torch
    from draft_tree_construction_rank_amd import binding
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()
    return binding


def _dev(inst):
    import torch
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    masks = oa.anc_masks(inst.parent, np.clip(inst.n_nodes, 0, inst.Ncap), inst.Ncap)
    return dict(Q=bf(inst.Q), K=bf(inst.K), V=bf(inst.V),
                ctx=torch.from_numpy(inst.ctx_len.astype(np.int32)).cuda(),
                n=torch.from_numpy(inst.n_nodes.astype(np.int32)).cuda(),
                anc=torch.from_numpy(masks.view(np.int64)).cuda())


def _run(B, inst, d=None):
    import torch
    d = d or _dev(inst)
    p = B.make_attn_params(R=inst.R, Hq=inst.Hq, Hkv=inst.Hkv, D=inst.D, Ncap=inst.Ncap,
                           Cmax=inst.Cmax, scale=inst.scale)
    ws = B.alloc_attn_workspace(p, "cuda")
    # garbage in the output, so that every row the kernel must write is checked
    O = torch.full(tuple(d["Q"].shape), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.tree_attention(p, d["Q"], d["K"], d["V"], d["ctx"], d["n"], d["anc"], O, ws)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), B.dt_attn_workspace_bytes(p)


def _compare(inst, got, reqs=None, heads=None):
    Q, K, V = inst.f32("Q"), inst.f32("K"), inst.f32("V")
    ref = oa.tree_attention(Q, K, V, inst.ctx_len, inst.n_nodes, inst.parent, inst.scale,
                            reqs=reqs, heads=heads)
    mag = oa.tree_attention(Q, K, np.abs(V), inst.ctx_len, inst.n_nodes, inst.parent,
                            inst.scale, reqs=reqs, heads=heads)
    reqs = range(inst.R) if reqs is None else reqs
    heads = range(inst.Hq) if heads is None else heads
    worst = 0.0
    for r in reqs:
        ctx, n = int(inst.ctx_len[r]), int(inst.n_nodes[r])
        ok = oa.request_valid(ctx, n, inst.Ncap, inst.Cmax)
        live = n + 1 if ok else 0
        for hq in heads:
            g, rf, mg = got[r, hq], ref[r, hq], mag[r, hq]
            assert np.isfinite(g[:live]).all(), (r, hq)
            assert (g[live:] == 0).all(), ("rows past the tree must be zero", r, hq)
            tol = 2 * U * mg[:live] + U * np.abs(rf[:live]) + 1e-6
            err = np.abs(g[:live] - rf[:live])
            bad = np.argwhere(err > tol)
            assert bad.size == 0, ("request", r, "head", hq, "row/col", bad[:4].tolist(),
                                   g[:live][tuple(bad[0])], rf[:live][tuple(bad[0])])
            if live:
                worst = max(worst, float((err / tol).max()))
    return worst


SMALL = [
    dict(name="g4_n12", seed=1, R=3, Hq=8, Hkv=2, Ncap=12, ctx_lo=0, ctx_hi=90, nodes="ragged"),
    dict(name="g4_n12_split", seed=2, R=2, Hq=8, Hkv=2, Ncap=12, ctx_lo=300, ctx_hi=700,
         nodes="ragged"),
    dict(name="g4_n32", seed=3, R=3, Hq=8, Hkv=2, Ncap=32, ctx_lo=10, ctx_hi=500),
    dict(name="g4_n55", seed=4, R=2, Hq=8, Hkv=2, Ncap=55, ctx_lo=33, ctx_hi=333),
    dict(name="g4_n63", seed=5, R=2, Hq=8, Hkv=2, Ncap=63, ctx_lo=64, ctx_hi=640),
    dict(name="g4_n64", seed=6, R=2, Hq=8, Hkv=2, Ncap=64, ctx_lo=100, ctx_hi=400),
    dict(name="g4_n64_split", seed=7, R=1, Hq=8, Hkv=2, Ncap=64, ctx_lo=900, ctx_hi=1300),
    dict(name="g5_n64_ragged", seed=8, R=3, Hq=10, Hkv=2, Ncap=64, ctx_lo=0, ctx_hi=300,
         nodes="ragged"),
    dict(name="g1_n64", seed=9, R=2, Hq=2, Hkv=2, Ncap=64, ctx_lo=1, ctx_hi=200),
    dict(name="g16_n64", seed=10, R=1, Hq=16, Hkv=1, Ncap=64, ctx_lo=0, ctx_hi=200),
    dict(name="g8_n32_peaky", seed=11, R=3, Hq=16, Hkv=2, Ncap=32, ctx_lo=5, ctx_hi=300,
         qscale=4.0),
    dict(name="chain", seed=12, R=2, Hq=8, Hkv=2, Ncap=64, ctx_lo=0, ctx_hi=150, tree="chain"),
    dict(name="star", seed=13, R=2, Hq=8, Hkv=2, Ncap=64, ctx_lo=0, ctx_hi=150, tree="star"),
    dict(name="ctx0", seed=14, R=3, Hq=8, Hkv=2, Ncap=20, ctx_lo=0, ctx_hi=0, nodes="ragged"),
    dict(name="ncap1", seed=15, R=4, Hq=4, Hkv=4, Ncap=1, ctx_lo=0, ctx_hi=70, nodes="ragged"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c["name"] for c in SMALL])
def test_small(B, case):
    kw = {k: v for k, v in case.items() if k != "name"}
    inst = attn_inputs.make_attn_instance(D=128, threads=4, **kw)
    print("case", case["name"], flush=True)
    got, ws = _run(B, inst)
    w = _compare(inst, got)
    print("  worst err/tol %.3f, workspace %d" % (w, ws))


def test_split_path_taken(B):
    """The split case above really goes through the workspace and the combine kernel."""
    p = B.make_attn_params(R=1, Hq=8, Hkv=2, D=128, Ncap=64, Cmax=1300 + 65, scale=0.1)
    assert B.dt_attn_workspace_bytes(p) > 0
    p = B.make_attn_params(R=2, Hq=8, Hkv=2, D=128, Ncap=64, Cmax=400 + 65, scale=0.1)
    assert B.dt_attn_workspace_bytes(p) > 0


def test_invalid_requests_are_zero(B):
    inst = attn_inputs.make_attn_instance(seed=16, R=6, Hq=8, Hkv=2, D=128, Ncap=16, ctx_lo=10,
                                          ctx_hi=200, nodes="ragged", threads=4)
    inst.n_nodes[1] = inst.Ncap + 3
    inst.n_nodes[2] = -1
    inst.ctx_len[3] = -5
    inst.ctx_len[4] = inst.Cmax - int(inst.n_nodes[4])  # one slot short
    got, _ = _run(B, inst)
    for r in (1, 2, 3, 4):
        assert (got[r] == 0).all(), r
    _compare(inst, got)


def test_full_workload_batched(B):
    """64 requests, Qwen3-8B attention shape, N = 64 full random trees, contexts 512..2048:
    every request, two query heads each (all key/value heads covered across requests)."""
    inst = attn_inputs.make_attn_instance(seed=100, R=64, Hq=32, Hkv=8, D=128, Ncap=64,
                                          ctx_lo=512, ctx_hi=2048)
    got, ws = _run(B, inst)
    assert ws == 0  # single key split at this size
    for r in range(inst.R):
        _compare(inst, got, reqs=[r], heads=[r % 32, (r + 13) % 32])


def test_full_workload_ragged(B):
    inst = attn_inputs.make_attn_instance(seed=101, R=64, Hq=32, Hkv=8, D=128, Ncap=64,
                                          ctx_lo=512, ctx_hi=2048, nodes="ragged")
    got, _ = _run(B, inst)
    for r in range(0, inst.R, 3):
        _compare(inst, got, reqs=[r], heads=[(5 * r) % 32])


def test_full_workload_single_request(B):
    """One request (the split path at full shape): every query head."""
    inst = attn_inputs.make_attn_instance(seed=102, R=1, Hq=32, Hkv=8, D=128, Ncap=64,
                                          ctx_lo=2048, ctx_hi=2048)
    got, ws = _run(B, inst)
    assert ws > 0
    _compare(inst, got)


def test_gqa_14b_shape(B):
    """Qwen3-14B grouping (40 query heads over 8 key/value heads): two query groups."""
    inst = attn_inputs.make_attn_instance(seed=103, R=4, Hq=40, Hkv=8, D=128, Ncap=64,
                                          ctx_lo=100, ctx_hi=900)
    got, _ = _run(B, inst)
    _compare(inst, got, heads=[0, 4, 9, 17, 22, 31, 38, 39])
