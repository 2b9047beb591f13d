"""CPU oracle for the conditional draft-tree builder -- TEST INFRASTRUCTURE.

A thin ctypes wrapper over ``dtree_oracle.c`` (plain single-threaded C, double
precision).  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product
path (``conditional_draft_tree_amd``) never does.

Every function here only marshals numpy arrays into the C routines; the
arithmetic is in ``dtree_oracle.c``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dtree_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off", "-o", tmp, _SRC, "-lm"],
            check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = C.CDLL(_LIB)
            vp, i32p, f64p = C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_double)
            lib.oracle_topm_row.argtypes = [vp, C.c_int, C.c_int, C.c_int, i32p, f64p]
            lib.oracle_gru.argtypes = [vp, C.c_int64, C.c_int, f64p, vp, vp, vp, vp, C.c_int,
                                       C.c_int, f64p]
            lib.oracle_dist.argtypes = [i32p, f64p, C.c_int, vp, C.c_int, C.c_int, f64p,
                                        C.c_double, C.c_double, i32p, f64p]
            lib.oracle_tail_lse.argtypes = [vp, C.c_int, C.c_int, C.c_int, C.c_double, i32p, f64p]
            lib.oracle_build_request.argtypes = (
                [C.c_int] * 6 + [C.c_double, C.c_int, C.c_double] + [vp] * 8 +
                [i32p, i32p, i32p, f64p, C.POINTER(C.c_uint8), i32p, C.POINTER(C.c_uint32),
                 f64p, i32p, f64p, C.c_int, f64p, i32p])
            lib.oracle_score_paths.argtypes = (
                [C.c_int] * 5 + [C.c_double, C.c_int] + [vp] * 8 + [C.c_int, i32p, i32p, f64p, C.c_int])
            lib.oracle_accept_greedy.argtypes = [C.c_int, C.c_int, i32p, i32p, i32p, i32p, i32p,
                                                 i32p]
            for f in (lib.oracle_topm_row, lib.oracle_gru, lib.oracle_dist, lib.oracle_tail_lse,
                      lib.oracle_build_request, lib.oracle_score_paths, lib.oracle_accept_greedy):
                f.restype = C.c_int
            _lib = lib
    return _lib


def _ptr(a, ctype=None):
    if a is None:
        return None
    if ctype is None:
        return C.c_void_p(a.ctypes.data)
    return a.ctypes.data_as(C.POINTER(ctype))


def _dt(a) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle inputs are float32 or bf16 bit patterns (uint16), got {a.dtype}")


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def topm_row(row: np.ndarray, M: int):
    """Top-M of one row of base logits: (idx int32 [M], val float64 [M])."""
    row = np.ascontiguousarray(row)
    idx = np.empty(M, np.int32)
    val = np.empty(M, np.float64)
    _check(_load().oracle_topm_row(_ptr(row), _dt(row), row.shape[0], M, _ptr(idx, C.c_int32),
                                   _ptr(val, C.c_double)), "oracle_topm_row")
    return idx, val


def gru(xmat: np.ndarray, xrow: int, h: np.ndarray, w_ih, w_hh, b_ih=None, b_hh=None):
    """One GRU step: x = xmat[xrow], h float64 [H] -> h' float64 [H]."""
    dt = _dt(xmat)
    H, E = w_hh.shape[1], w_ih.shape[1]
    h = np.ascontiguousarray(h, np.float64)
    out = np.empty(H, np.float64)
    _check(_load().oracle_gru(_ptr(xmat), int(xrow), dt, _ptr(h, C.c_double), _ptr(w_ih), _ptr(w_hh),
                              _ptr(b_ih), _ptr(b_hh), E, H, _ptr(out, C.c_double)), "oracle_gru")
    return out


def tail_lse(row: np.ndarray, M: int, T: float = 0.0) -> float:
    """log sum of exp(x / T) (T = 1 when T = 0) over the row's logits outside its
    top M (the full-vocabulary mode's tail); -inf when M = V."""
    row = np.ascontiguousarray(row)
    idx, _ = topm_row(row, M)
    out = np.zeros(1, np.float64)
    _check(_load().oracle_tail_lse(_ptr(row), _dt(row), row.shape[0], M, float(T), _ptr(idx, C.c_int32),
                                   _ptr(out, C.c_double)), "oracle_tail_lse")
    return float(out[0])


def dist(idx: np.ndarray, val: np.ndarray, Cmat: np.ndarray, h: np.ndarray, T: float = 0.0,
         tail: float = -np.inf):
    """Sorted children (tok int32 [M], logp float64 [M]) of a node with state h;
    ``tail`` (the row's tail_lse) adds the rest of the vocabulary to the
    normalizer (-inf: normalized over the M-slice)."""
    idx = np.ascontiguousarray(idx, np.int32)
    val = np.ascontiguousarray(val, np.float64)
    h = np.ascontiguousarray(h, np.float64)
    M, H = idx.shape[0], Cmat.shape[1]
    tok = np.empty(M, np.int32)
    lp = np.empty(M, np.float64)
    _check(_load().oracle_dist(_ptr(idx, C.c_int32), _ptr(val, C.c_double), M, _ptr(Cmat), _dt(Cmat),
                               H, _ptr(h, C.c_double), float(T), float(tail), _ptr(tok, C.c_int32),
                               _ptr(lp, C.c_double)), "oracle_dist")
    return tok, lp


def build_request(inp: dict, b: int, M: int, n: int, T: float = 0.0, eps: float = 1e-5,
                  full_vocab: bool = False) -> dict:
    """Tree of request b.  ``inp`` holds numpy arrays: base [B,L,V], emb [V,E],
    w_ih [3H,E], w_hh [3H,H], b_ih/b_hh [3H] (or None), C [V,H], h0 [B,H] float32
    (or None).  ``full_vocab``: normalize children over the whole vocabulary
    (corrected top-M plus the uncorrected tail; ``tail`` [L] is returned)."""
    base = np.ascontiguousarray(inp["base"][b])
    L, V = base.shape
    E, H = inp["w_ih"].shape[1], inp["w_hh"].shape[1]
    S = n + 1
    out = dict(tokens=np.empty(S, np.int32), parents=np.empty(S, np.int32),
               depths=np.empty(S, np.int32), scores=np.empty(S, np.float64),
               mask=np.empty((S, S), np.uint8), count=np.zeros(1, np.int32),
               flags=np.zeros(1, np.uint32), min_gap=np.zeros(1, np.float64),
               topm_idx=np.empty((L, M), np.int32), topm_val=np.empty((L, M), np.float64),
               tail=np.empty(L, np.float64), first_flag=np.zeros(1, np.int32))
    h0 = inp.get("h0")
    h0b = None if h0 is None else np.ascontiguousarray(h0[b], np.float32)
    rc = _load().oracle_build_request(
        V, L, E, H, M, n, float(T), _dt(base), float(eps), _ptr(base), _ptr(inp["emb"]),
        _ptr(inp["w_ih"]), _ptr(inp["w_hh"]), _ptr(inp.get("b_ih")), _ptr(inp.get("b_hh")),
        _ptr(inp["C"]), _ptr(h0b),
        _ptr(out["tokens"], C.c_int32), _ptr(out["parents"], C.c_int32),
        _ptr(out["depths"], C.c_int32), _ptr(out["scores"], C.c_double),
        _ptr(out["mask"], C.c_uint8), _ptr(out["count"], C.c_int32),
        _ptr(out["flags"], C.c_uint32), _ptr(out["min_gap"], C.c_double),
        _ptr(out["topm_idx"], C.c_int32), _ptr(out["topm_val"], C.c_double), int(bool(full_vocab)),
        _ptr(out["tail"], C.c_double), _ptr(out["first_flag"], C.c_int32))
    _check(rc, "oracle_build_request")
    out["count"] = int(out["count"][0])
    out["flags"] = int(out["flags"][0])
    out["min_gap"] = float(out["min_gap"][0])
    # slot of the first pop decided by a margin below eps (0: none); slots
    # before it were decided by margins of at least eps
    out["first_flag"] = int(out["first_flag"][0])
    return out


def build_batch(inp: dict, M: int, n: int, T: float = 0.0, eps: float = 1e-5,
                requests=None, threads: int = 1, full_vocab: bool = False) -> list:
    """Trees of several requests; each request is one single-threaded oracle
    call, spread over ``threads`` worker threads (the C call drops the GIL)."""
    B = inp["base"].shape[0]
    reqs = list(range(B)) if requests is None else list(requests)
    _load()
    if threads <= 1:
        return [build_request(inp, b, M, n, T, eps, full_vocab) for b in reqs]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(lambda b: build_request(inp, b, M, n, T, eps, full_vocab), reqs))


def score_paths(inp: dict, b: int, M: int, paths, T: float = 0.0, full_vocab: bool = False) -> np.ndarray:
    """Conditional score of each token path (list of token lists) of request b."""
    base = np.ascontiguousarray(inp["base"][b])
    L, V = base.shape
    E, H = inp["w_ih"].shape[1], inp["w_hh"].shape[1]
    P = len(paths)
    arr = np.full((max(P, 1), L), -1, np.int32)
    lens = np.zeros(max(P, 1), np.int32)
    for i, p in enumerate(paths):
        arr[i, :len(p)] = p
        lens[i] = len(p)
    out = np.empty(max(P, 1), np.float64)
    h0 = inp.get("h0")
    h0b = None if h0 is None else np.ascontiguousarray(h0[b], np.float32)
    rc = _load().oracle_score_paths(
        V, L, E, H, M, float(T), _dt(base), _ptr(base), _ptr(inp["emb"]), _ptr(inp["w_ih"]),
        _ptr(inp["w_hh"]), _ptr(inp.get("b_ih")), _ptr(inp.get("b_hh")), _ptr(inp["C"]),
        _ptr(h0b), P, _ptr(arr, C.c_int32), _ptr(lens, C.c_int32), _ptr(out, C.c_double),
        int(bool(full_vocab)))
    _check(rc, "oracle_score_paths")
    return out[:P]


def accept_greedy(tokens, parents, count: int, target) -> dict:
    """Greedy acceptance walk of one request's tree (slots 0..n): the accepted
    slots in order (``path``, length ``accepted``), and the target's bonus token."""
    tok = np.ascontiguousarray(tokens, np.int32)
    par = np.ascontiguousarray(parents, np.int32)
    tgt = np.ascontiguousarray(target, np.int32)
    n = tok.shape[0] - 1
    if par.shape != tok.shape or tgt.shape != tok.shape:
        raise ValueError("tokens, parents and target must all have n + 1 entries")
    path = np.empty(n + 1, np.int32)
    acc = np.zeros(1, np.int32)
    bonus = np.zeros(1, np.int32)
    rc = _load().oracle_accept_greedy(n, int(count), _ptr(tok, C.c_int32), _ptr(par, C.c_int32),
                                      _ptr(tgt, C.c_int32), _ptr(path, C.c_int32),
                                      _ptr(acc, C.c_int32), _ptr(bonus, C.c_int32))
    _check(rc, "oracle_accept_greedy")
    k = int(acc[0])
    return {"path": path[:k].copy(), "accepted": k, "bonus": int(bonus[0])}
