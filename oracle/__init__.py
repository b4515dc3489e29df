"""Python wrapper around the plain C oracle (``dtree_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package; the library under ``draft_tree_construction_rank_amd``
never does.  Arguments are marshalled to float32/int32 numpy arrays; the arithmetic is all in
C (float64, single thread).

Parity status: every exported function is pinned by CPU tests (see tests/test_oracle_*.py).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dtree_oracle.c")
_LIB = os.path.join(_HERE, "libdtree_oracle.so")

GREEDY, SAMPLE = 0, 1
STREAM_GUMBEL, STREAM_ACCEPT, STREAM_RESID = 1, 2, 3
STATUS_BAD_ROOT, STATUS_BUDGET_CLAMPED = 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (single thread, no FMA contraction, float64)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
                               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Params(C.Structure):
    _fields_ = [("R", C.c_int32), ("B", C.c_int32), ("k", C.c_int32), ("V", C.c_int32),
                ("r", C.c_int32), ("Ncap", C.c_int32), ("mode", C.c_int32),
                ("temperature", C.c_double), ("cal", C.c_float * 16), ("seed", C.c_uint64),
                ("round", C.c_uint32)]


class _Tree(C.Structure):
    _fields_ = [("token", C.c_void_p), ("parent", C.c_void_p), ("depth", C.c_void_p),
                ("mask", C.c_void_p), ("surv", C.c_void_p), ("logq", C.c_void_p),
                ("n_nodes", C.c_void_p), ("cand", C.c_void_p), ("status", C.c_void_p),
                ("n_expand", C.c_void_p)]


class _Verify(C.Structure):
    _fields_ = [("accept_len", C.c_void_p), ("path", C.c_void_p), ("out_tokens", C.c_void_p),
                ("n_out", C.c_void_p)]


MARGIN_DTYPE = np.dtype([("key_gap", np.float64), ("q_edge", np.float64),
                         ("accept", np.float64), ("draw_gap", np.float64),
                         ("argmax_gap", np.float64)])

_lib: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = C.CDLL(_LIB)
        vp = C.c_void_p
        L.or_philox4x32_10.argtypes = [vp, vp, vp]
        L.or_mix64.restype = C.c_uint64
        L.or_mix64.argtypes = [C.c_uint64]
        L.or_root_hash.restype = C.c_uint64
        L.or_root_hash.argtypes = [C.c_uint32, C.c_int32, C.c_int32]
        L.or_child_hash.restype = C.c_uint64
        L.or_child_hash.argtypes = [C.c_uint64, C.c_int32]
        L.or_uniform.restype = C.c_double
        L.or_uniform.argtypes = [C.c_uint64, C.c_uint64, C.c_uint32, C.c_uint32]
        L.or_expand.restype = C.c_double
        L.or_expand.argtypes = [C.POINTER(Params), vp, vp, vp, C.c_int32, C.c_int32, C.c_uint64,
                                vp, vp, vp, vp]
        L.or_build.argtypes = [C.POINTER(Params), vp, vp, vp, vp, vp, vp, C.c_int32,
                               C.POINTER(_Tree), vp]
        L.or_verify_greedy.argtypes = [C.POINTER(Params), C.POINTER(_Tree), vp,
                                       C.POINTER(_Verify), vp]
        L.or_verify_sample.argtypes = [C.POINTER(Params), C.POINTER(_Tree), vp, vp, vp, vp, vp,
                                       C.POINTER(_Verify), vp]
        L.or_chain_probs.argtypes = [vp, vp, C.c_int32, vp, C.c_int32, vp, vp]
        L.or_sample_rounds.argtypes = [C.POINTER(Params), vp, vp, vp, C.c_int32, C.c_int32,
                                       C.c_float, vp, C.c_int64, vp, vp]
        L.or_set_fault.argtypes = [C.c_int32]
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def make_params(inst, *, R=None, mode=None, temperature=None, round_=None) -> Params:
    P = Params()
    P.R = inst.R if R is None else R
    P.B, P.k, P.V, P.r, P.Ncap = inst.B, inst.k, inst.V, inst.r, inst.Ncap
    m = inst.mode if mode is None else mode
    P.mode = SAMPLE if m in ("sample", SAMPLE) else GREEDY
    P.temperature = inst.temperature if temperature is None else float(temperature)
    for i in range(16):
        P.cal[i] = float(inst.cal[i])
    P.seed = inst.seed
    P.round = inst.round if round_ is None else int(round_)
    return P


def _c32(a, dt=np.float32):
    return np.ascontiguousarray(a, dtype=dt)


def philox(ctr, key) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().or_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def mix64(x: int) -> int:
    return int(lib().or_mix64(x & (2**64 - 1)))


def root_hash(round_: int, request: int, root_token: int) -> int:
    return int(lib().or_root_hash(round_, request, root_token))


def child_hash(h: int, token: int) -> int:
    return int(lib().or_child_hash(h, token))


def uniform(seed: int, h: int, stream: int, index: int) -> float:
    return float(lib().or_uniform(seed, h, stream, index))


def expand(inst, req: int, depth: int, token: int, h: int = 0, *, mode=None,
           temperature=None):
    """One expansion: returns dict(y[V], lse, child_tok[k], child_y[k], gap)."""
    P = make_params(inst, mode=mode, temperature=temperature)
    L = _c32(inst.L[req])
    U = _c32(inst.U)
    Wt = _c32(inst.Wt)
    y = np.zeros(inst.V, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    ct = np.zeros(inst.k, dtype=np.int32)
    cy = np.zeros(inst.k, dtype=np.float64)
    gap = lib().or_expand(C.byref(P), _p(L), _p(U), _p(Wt), depth, token, h, _p(y), _p(lse),
                          _p(ct), _p(cy))
    return dict(y=y, lse=float(lse[0]), child_tok=ct, child_y=cy, gap=float(gap))


def new_tree(R: int, Ncap: int, k: int) -> dict:
    return dict(token=np.zeros((R, Ncap), np.int32), parent=np.zeros((R, Ncap), np.int16),
                depth=np.zeros((R, Ncap), np.uint8), mask=np.zeros((R, Ncap), np.uint64),
                surv=np.zeros((R, Ncap), np.float32), logq=np.zeros((R, Ncap), np.float32),
                n_nodes=np.zeros(R, np.int32), cand=np.zeros((R, Ncap + 1, k), np.int32),
                status=np.zeros(R, np.int32), n_expand=np.zeros(R, np.int32))


def _tree_struct(t: dict) -> _Tree:
    s = _Tree()
    for f, _ in _Tree._fields_:
        setattr(s, f, _p(t[f]))
    return s


def new_margins(R: int) -> np.ndarray:
    m = np.zeros(R, dtype=MARGIN_DTYPE)
    for f in MARGIN_DTYPE.names:
        m[f] = np.inf
    return m


def build_tree(inst, *, requests=None, method: int = 0, n_budget=None, tau=None,
               margins: Optional[np.ndarray] = None, mode=None, temperature=None,
               round_=None) -> dict:
    """Build trees for the listed requests (default all).  ``method`` 0 = best-first
    priority queue, 1 = level-synchronous.  Returns the tree dict (arrays over the listed
    requests, in that order)."""
    reqs = list(range(inst.R)) if requests is None else list(requests)
    R = len(reqs)
    P = make_params(inst, R=R, mode=mode, temperature=temperature, round_=round_)
    L = _c32(inst.L[reqs])
    roots = _c32(inst.root_token[reqs], np.int32)
    nb = _c32((inst.n_budget if n_budget is None else np.broadcast_to(n_budget, inst.R))[reqs],
              np.int32)
    ta = _c32((inst.tau if tau is None else np.broadcast_to(np.float32(tau), inst.R))[reqs])
    t = new_tree(R, inst.Ncap, inst.k)
    ts = _tree_struct(t)
    mg = margins if margins is not None else new_margins(R)
    # request ids enter the random keys: pass the true id through a per-request call when
    # the subset is not 0..R-1
    if reqs == list(range(R)):
        rc = lib().or_build(C.byref(P), _p(L), _p(_c32(inst.U)), _p(_c32(inst.Wt)), _p(roots),
                            _p(nb), _p(ta), method, C.byref(ts), _p(mg))
        assert rc == 0
    else:
        for i, rq in enumerate(reqs):
            one = _build_one(inst, rq, method, int(nb[i]), float(ta[i]), mode, temperature,
                             round_)
            for f in t:
                t[f][i] = one[0][f][rq]
            mg[i] = one[1][rq]
    t["margins"] = mg
    t["requests"] = reqs
    return t


def _build_one(inst, rq, method, nb, tau, mode, temperature, round_):
    """Build request rq alone but with its true request id (id enters the random keys)."""
    R = rq + 1
    P = make_params(inst, R=R, mode=mode, temperature=temperature, round_=round_)
    L = np.zeros((R, inst.B, inst.V), np.float32)
    L[rq] = inst.L[rq]
    roots = np.full(R, -1, np.int32)
    roots[rq] = inst.root_token[rq]
    nbs = np.zeros(R, np.int32)
    nbs[rq] = nb
    taus = np.zeros(R, np.float32)
    taus[rq] = tau
    t = new_tree(R, inst.Ncap, inst.k)
    ts = _tree_struct(t)
    mg = new_margins(R)
    rc = lib().or_build(C.byref(P), _p(L), _p(_c32(inst.U)), _p(_c32(inst.Wt)), _p(roots),
                        _p(nbs), _p(taus), method, C.byref(ts), _p(mg))
    assert rc == 0
    return t, mg


def _verify_struct(R: int, B: int):
    o = dict(accept_len=np.zeros(R, np.int32), path=np.zeros((R, B), np.int32),
             out_tokens=np.zeros((R, B + 1), np.int32), n_out=np.zeros(R, np.int32))
    s = _Verify()
    for f, _ in _Verify._fields_:
        setattr(s, f, _p(o[f]))
    return o, s


def _subset_tree(tree: dict, reqs_needed: int, ids) -> dict:
    """Place a tree over listed requests into arrays indexed by true request id."""
    out = {}
    for f, v in tree.items():
        if f in ("margins", "requests"):
            continue
        a = np.zeros((reqs_needed,) + v.shape[1:], dtype=v.dtype)
        if f == "status":
            a[:] = STATUS_BAD_ROOT  # requests not listed are skipped by the verifiers
        for i, rq in enumerate(ids):
            a[rq] = v[i]
        out[f] = a
    return out


def verify_greedy(inst, tree: dict, target: np.ndarray, margins=None) -> dict:
    """Greedy accept-walk for the requests in ``tree['requests']``; target [len][Ncap+1][V]."""
    ids = tree["requests"]
    R = max(ids) + 1
    full = _subset_tree(tree, R, ids)
    tg = np.zeros((R, inst.Ncap + 1, inst.V), np.float32)
    tg[ids] = target
    P = make_params(inst, R=R)
    ts = _tree_struct(full)
    o, os_ = _verify_struct(R, inst.B)
    mg = new_margins(R)
    lib().or_verify_greedy(C.byref(P), C.byref(ts), _p(tg), C.byref(os_), _p(mg))
    res = {f: v[ids] for f, v in o.items()}
    res["margins"] = mg[ids]
    return res


def verify_sample(inst, tree: dict, target: np.ndarray, *, temperature=None,
                  round_=None) -> dict:
    """Lossless sample verify for the requests in ``tree['requests']``."""
    ids = tree["requests"]
    R = max(ids) + 1
    full = _subset_tree(tree, R, ids)
    tg = np.zeros((R, inst.Ncap + 1, inst.V), np.float32)
    tg[ids] = target
    L = np.zeros((R, inst.B, inst.V), np.float32)
    L[ids] = inst.L[ids]
    roots = np.zeros(R, np.int32)
    roots[ids] = inst.root_token[ids]
    P = make_params(inst, R=R, mode=SAMPLE, temperature=temperature, round_=round_)
    ts = _tree_struct(full)
    o, os_ = _verify_struct(R, inst.B)
    mg = new_margins(R)
    lib().or_verify_sample(C.byref(P), C.byref(ts), _p(L), _p(_c32(inst.U)), _p(_c32(inst.Wt)),
                           _p(roots), _p(tg), C.byref(os_), _p(mg))
    res = {f: v[ids] for f, v in o.items()}
    res["margins"] = mg[ids]
    return res


def chain_probs(p: np.ndarray, q: np.ndarray, x) -> tuple:
    p = np.ascontiguousarray(p, np.float64)
    q = np.ascontiguousarray(q, np.float64)
    xs = np.ascontiguousarray(x, np.int32)
    acc = np.zeros(len(xs), np.float64)
    res = np.zeros(len(p), np.float64)
    lib().or_chain_probs(_p(p), _p(q), len(p), _p(xs), len(xs), _p(acc), _p(res))
    return acc, res


def sample_rounds(inst, target_tab: np.ndarray, n_rounds: int, *, temperature=None,
                  n_budget=None, tau=0.0) -> tuple:
    """Run n_rounds full sample rounds of request 0 with a (depth, token) target table."""
    P = make_params(inst, R=1, mode=SAMPLE, temperature=temperature)
    tab = _c32(target_tab)
    assert tab.shape == (inst.B + 1, inst.V, inst.V)
    first = np.zeros(n_rounds, np.int32)
    second = np.zeros(n_rounds, np.int32)
    nb = inst.Ncap if n_budget is None else n_budget
    lib().or_sample_rounds(C.byref(P), _p(_c32(inst.L[:1])), _p(_c32(inst.U)),
                           _p(_c32(inst.Wt)), int(inst.root_token[0]), int(nb), float(tau),
                           _p(tab), n_rounds, _p(first), _p(second))
    return first, second


def set_fault(mode: int) -> None:
    lib().or_set_fault(mode)
