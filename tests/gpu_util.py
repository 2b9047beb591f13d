"""Helpers of the GPU parity tests: run the library, compare with the oracle."""
from __future__ import annotations

import numpy as np

import oracle

SCORE_TOL = 1e-4  # absolute, binary32 node scores vs the double-precision oracle
# Gaps below this are under binary32 resolution of the scores (ulp(16) ~ 2e-6):
# the GPU may see them as exact ties, which it breaks deterministically and
# does not flag.
FP32_RESOLUTION = 2e-6


def run_build(bld, t: dict):
    import torch
    out = bld.build(t["base"], t["emb"], t["w_ih"], t["w_hh"], t.get("b_ih"), t.get("b_hh"),
                    t["C"], t.get("h0"))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def ancestor_mask(parents: np.ndarray, count: int) -> np.ndarray:
    S = parents.shape[0]
    m = np.zeros((S, S), np.uint8)
    for i in range(count + 1):
        j = i
        while j >= 0:
            m[i, j] = 1
            j = parents[j] if j > 0 else -1
    return m


def check_valid_tree(got: dict, b: int, n: int, L: int):
    """Properties every output must have, whatever the ties."""
    cnt = int(got["count"][b])
    tok, par, dep, sc = got["tokens"][b], got["parents"][b], got["depths"][b], got["scores"][b]
    assert 0 <= cnt <= n
    assert tok[0] == -1 and par[0] == -1 and dep[0] == 0 and sc[0] == 0.0
    for v in range(1, cnt + 1):
        q = par[v]
        assert 0 <= q < v, (b, v, q)
        assert dep[v] == dep[q] + 1 and 1 <= dep[v] <= L
        assert sc[v] <= sc[q]
        assert tok[v] >= 0
    # every node is a distinct token path: no two slots share (parent, token)
    pairs = set(zip(par[1:cnt + 1].tolist(), tok[1:cnt + 1].tolist()))
    assert len(pairs) == cnt, f"request {b}: two slots share a (parent, token) pair"
    assert np.all(np.diff(sc[1:cnt + 1]) <= 0), "pop order must be by non-increasing score"
    assert np.all(tok[cnt + 1:] == -1) and np.all(par[cnt + 1:] == -1)
    assert np.all(dep[cnt + 1:] == -1) and np.all(np.isneginf(sc[cnt + 1:]))
    np.testing.assert_array_equal(got["mask"][b], ancestor_mask(par, cnt))


def paths_of(got: dict, b: int):
    cnt = int(got["count"][b])
    tok, par = got["tokens"][b], got["parents"][b]
    out = []
    for v in range(1, cnt + 1):
        p, j = [], v
        while j > 0:
            p.append(int(tok[j]))
            j = par[j]
        out.append(p[::-1])
    return out


def compare_request(got: dict, b_got: int, ref: dict, inp: dict, b_inp: int, cfg: dict,
                    eps: float = 1e-5, tol: float = SCORE_TOL):
    """Compare request b_got of a GPU result with the oracle's tree `ref` of
    request b_inp of `inp`.  Returns ("exact" or "flagged", the largest
    |GPU score - oracle score| over the request's nodes, and that largest
    error per node depth as a dict)."""
    n, L = cfg["n"], cfg["L"]
    check_valid_tree(got, b_got, n, L)
    assert int(got["count"][b_got]) == ref["count"]
    gflag = int(got["flags"][b_got]) & 1
    if ref["min_gap"] > 2 * eps:
        assert gflag == 0, f"GPU flags a near tie the oracle puts at {ref['min_gap']:.3g}"
    if FP32_RESOLUTION <= ref["min_gap"] < eps / 2:
        assert gflag == 1, f"GPU misses a near tie of {ref['min_gap']:.3g}"
    cnt = ref["count"]
    if ref["flags"] == 0:
        for k in ("tokens", "parents", "depths", "mask"):
            np.testing.assert_array_equal(got[k][b_got], ref[k], err_msg=k)
        e = np.abs(got["scores"][b_got][:cnt + 1] - ref["scores"][:cnt + 1])
        err = float(e.max())
        assert err <= tol, f"score error {err}"
        return "exact", err, by_depth(e[1:], ref["depths"][1:cnt + 1])
    # A decision was closer than eps: several trees are correct.  The pops
    # before the first such decision were decided by margins of at least eps,
    # so those slots are unique; so is the multiset of the best scores, and
    # every GPU node must carry its own conditional score.
    k0 = ref["first_flag"]
    assert 1 <= k0 <= cnt, k0
    for k in ("tokens", "parents", "depths"):
        np.testing.assert_array_equal(got[k][b_got][:k0], ref[k][:k0],
                                      err_msg=f"{k} before the first near tie (slot {k0})")
    gs = got["scores"][b_got][1:cnt + 1].astype(np.float64)
    rs = oracle.score_paths(inp, b_inp, cfg["M"], paths_of(got, b_got), cfg["T"],
                            full_vocab=cfg.get("full_vocab", False))
    assert np.all(np.isfinite(rs)), "GPU node outside the top-M candidate tree"
    e = np.abs(gs - rs)
    err = float(e.max())
    assert err <= tol, f"score error {err}"
    assert np.abs(np.sort(gs) - np.sort(ref["scores"][1:cnt + 1])).max() <= tol
    return "flagged", err, by_depth(e, got["depths"][b_got][1:cnt + 1])


def by_depth(err, depths) -> dict:
    out = {}
    for e, d in zip(err.tolist(), depths.tolist()):
        out[int(d)] = max(out.get(int(d), 0.0), float(e))
    return out
