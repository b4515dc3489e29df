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
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dtree_oracle.c")
_LIB = os.path.join(_HERE, "libdtree_oracle.so")

GREEDY, SAMPLE = 0, 1
BUILD_HEAP, BUILD_LEVELSYNC, BUILD_FLASH = 0, 1, 2
COND_PARENT, COND_CHAIN, COND_NONE = 0, 1, 2
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
                ("round", C.c_uint32), ("req_base", C.c_int32), ("cond", C.c_int32)]


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
        L.or_build_flash.argtypes = [C.POINTER(Params), vp, vp, vp, vp, vp, vp,
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


def make_params(inst, *, R=None, mode=None, temperature=None, round_=None,
                req_base=0) -> Params:
    P = Params()
    P.req_base = int(req_base)
    P.cond = int(getattr(inst, "cond", 0))
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


def workers() -> int:
    """Threads for per-request oracle calls (each call is single-threaded C; ctypes releases
    the GIL).  DT_ORACLE_THREADS overrides; at most 16."""
    env = os.environ.get("DT_ORACLE_THREADS")
    n = int(env) if env else min(16, os.cpu_count() or 1)
    return max(1, min(16, n))


def _map(fn, items):
    items = list(items)
    if len(items) <= 1 or workers() == 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(max_workers=min(workers(), len(items))) as ex:
        return list(ex.map(fn, items))


def build_tree(inst, *, requests=None, method: int = 0, n_budget=None, tau=None,
               margins: Optional[np.ndarray] = None, mode=None, temperature=None,
               round_=None) -> dict:
    """Build trees for the listed requests (default all).  ``method`` 0 = best-first
    priority queue, 1 = level-synchronous, 2 = the two-stage M-ary tree (M = inst.k,
    greedy; or_build_flash).  Returns the tree dict (arrays over the listed requests, in
    that order).  Each request is built by its own single-request call, keyed by its true
    request id; the calls run on a thread pool."""
    reqs = list(range(inst.R)) if requests is None else list(requests)
    R = len(reqs)
    nb = np.asarray(inst.n_budget if n_budget is None else np.broadcast_to(n_budget, inst.R),
                    np.int64)
    ta = np.asarray(inst.tau if tau is None else np.broadcast_to(np.float32(tau), inst.R),
                    np.float32)
    U, Wt = _c32(inst.U), _c32(inst.Wt)

    def one(rq):
        P = make_params(inst, R=1, mode=mode, temperature=temperature, round_=round_,
                        req_base=rq)
        # every array handed to C is held in a local for the whole call (an address taken
        # from a temporary would point at freed memory)
        L = _c32(inst.L[rq:rq + 1])
        root = _c32(inst.root_token[rq:rq + 1], np.int32)
        budget = _c32(nb[rq:rq + 1], np.int32)
        thr = _c32(ta[rq:rq + 1])
        t = new_tree(1, inst.Ncap, inst.k)
        ts = _tree_struct(t)
        mg = new_margins(1)
        if method == 2:
            rc = lib().or_build_flash(C.byref(P), _p(L), _p(U), _p(Wt), _p(root), _p(budget),
                                      _p(thr), C.byref(ts), _p(mg))
        else:
            rc = lib().or_build(C.byref(P), _p(L), _p(U), _p(Wt), _p(root), _p(budget),
                                _p(thr), method, C.byref(ts), _p(mg))
        assert rc == 0
        return t, mg

    res = _map(one, reqs)
    t = new_tree(R, inst.Ncap, inst.k)
    mg = margins if margins is not None else new_margins(R)
    for i, (one_t, one_m) in enumerate(res):
        for f in t:
            t[f][i] = one_t[f][0]
        mg[i] = one_m[0]
    t["margins"] = mg
    t["requests"] = reqs
    return t


def _verify_struct(R: int, B: int):
    o = dict(accept_len=np.zeros(R, np.int32), path=np.zeros((R, B), np.int32),
             out_tokens=np.zeros((R, B + 1), np.int32), n_out=np.zeros(R, np.int32))
    s = _Verify()
    for f, _ in _Verify._fields_:
        setattr(s, f, _p(o[f]))
    return o, s


def _tree_row(tree: dict, i: int) -> dict:
    """Request i of a tree dict as a single-request tree (contiguous copies)."""
    return {f: np.ascontiguousarray(v[i:i + 1]) for f, v in tree.items()
            if f not in ("margins", "requests")}


def _collect(outs, B):
    R = len(outs)
    o = dict(accept_len=np.zeros(R, np.int32), path=np.zeros((R, B), np.int32),
             out_tokens=np.zeros((R, B + 1), np.int32), n_out=np.zeros(R, np.int32))
    mg = new_margins(R)
    for i, (oi, mi) in enumerate(outs):
        for f in o:
            o[f][i] = oi[f][0]
        mg[i] = mi[0]
    o["margins"] = mg
    return o


def verify_greedy(inst, tree: dict, target: np.ndarray, margins=None) -> dict:
    """Greedy accept-walk for the requests in ``tree['requests']``; target [len][Ncap+1][V]."""
    ids = tree["requests"]

    def one(i):
        P = make_params(inst, R=1, req_base=ids[i])
        t1 = _tree_row(tree, i)
        ts = _tree_struct(t1)
        o, os_ = _verify_struct(1, inst.B)
        mg = new_margins(1)
        tg = _c32(target[i:i + 1])
        lib().or_verify_greedy(C.byref(P), C.byref(ts), _p(tg), C.byref(os_), _p(mg))
        return o, mg

    return _collect(_map(one, range(len(ids))), inst.B)


def verify_sample(inst, tree: dict, target: np.ndarray, *, temperature=None,
                  round_=None) -> dict:
    """Lossless sample verify for the requests in ``tree['requests']``."""
    ids = tree["requests"]
    U, Wt = _c32(inst.U), _c32(inst.Wt)

    def one(i):
        rq = ids[i]
        P = make_params(inst, R=1, mode=SAMPLE, temperature=temperature, round_=round_,
                        req_base=rq)
        t1 = _tree_row(tree, i)
        ts = _tree_struct(t1)
        o, os_ = _verify_struct(1, inst.B)
        mg = new_margins(1)
        L = _c32(inst.L[rq:rq + 1])
        roots = _c32(inst.root_token[rq:rq + 1], np.int32)
        tg = _c32(target[i:i + 1])
        lib().or_verify_sample(C.byref(P), C.byref(ts), _p(L), _p(U), _p(Wt), _p(roots),
                               _p(tg), C.byref(os_), _p(mg))
        return o, mg

    return _collect(_map(one, range(len(ids))), inst.B)


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
    L, U, Wt = _c32(inst.L[:1]), _c32(inst.U), _c32(inst.Wt)  # alive for the whole call
    lib().or_sample_rounds(C.byref(P), _p(L), _p(U), _p(Wt), int(inst.root_token[0]), int(nb),
                           float(tau),
                           _p(tab), n_rounds, _p(first), _p(second))
    return first, second


def set_fault(mode: int) -> None:
    lib().or_set_fault(mode)
