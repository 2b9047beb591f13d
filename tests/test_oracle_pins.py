"""Pins of the CPU oracle to things other than itself (CPU only).

* top-M:        numpy's stable lexsort (library routine), bit-exact;
* GRU step:     torch.nn.GRUCell in float64 (library routine), fp32 and bf16
                storage;
* distribution: torch.log_softmax + numpy.lexsort; sum of probabilities = 1;
* tree:         exhaustive enumeration of the candidate tree (tests/bruteforce.py),
                exact branch-and-bound on the tiny workload, and a search over
                all prefix-closed node sets on very small trees;
* closed forms / special cases: M = 1 chain, n = 1 argmax, L = 1 sorted list,
                zero correction == factorized (DDTree) tree, a hand-derived
                example under tests/golden/;
* metamorphic:  vocabulary relabeling, batch independence;
* acceptance walk: hand-derived cases (tests/golden/hand_accept.json), and the
                accepted path recomputed as the set of nodes whose every root-path
                edge matches the target, on random trees and on oracle trees;
* full-vocabulary mode: tail vs scipy's logsumexp over the non-top-M logits;
                C = 0 children vs torch.log_softmax of the whole row; trees vs
                brute force and branch-and-bound with a torch scorer that adds
                the tail to its softmax; M = V reduces to the M-slice mode.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from bruteforce import (Scorer, as_f64, best_n_branch_and_bound, best_n_bruteforce,
                        factorized_tree, prefix_closed_subsets_best, topm_table, tree_arrays)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def small_cfg(**kw):
    cfg = dict(B=1, V=50, L=4, E=6, H=5, M=4, n=8, dtype="f32", alpha=1.1, T=0.0)
    cfg.update(kw)
    return cfg


def assert_tree_equal(res, ref, n, atol=1e-10):
    tok, par, dep, sc = ref
    np.testing.assert_array_equal(res["tokens"], tok)
    np.testing.assert_array_equal(res["parents"], par)
    np.testing.assert_array_equal(res["depths"], dep)
    fin = np.isfinite(sc)
    np.testing.assert_allclose(res["scores"][fin], sc[fin], atol=atol, rtol=0)
    assert np.all(np.isneginf(res["scores"][~fin]))


# ---------------------------------------------------------------- top-M ----

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,M", [(1000, 8), (257, 64), (64, 64), (5, 1), (3000, 17)])
def test_topm_matches_stable_lexsort(dtype, V, M):
    rng = np.random.default_rng(V * 31 + M)
    x = (rng.normal(0, 2, V)).astype(np.float32)
    x = np.round(x * 4) / 4  # many exact ties
    row = S.f32_to_bf16_bits(x) if dtype == "bf16" else x
    idx, val = oracle.topm_row(row, M)
    vals = as_f64(row)
    ref = np.lexsort((np.arange(V), -vals))[:M]
    np.testing.assert_array_equal(idx, ref)
    np.testing.assert_array_equal(val, vals[ref])


def test_topm_all_equal_takes_lowest_ids():
    row = np.full(100, -3.5, np.float32)
    idx, _ = oracle.topm_row(row, 10)
    np.testing.assert_array_equal(idx, np.arange(10))


def test_topm_bf16_zipf_row():
    cfg = S.CONFIGS["qwen3_4b_single"]
    base = S.make_base(1, 1, cfg["V"], cfg["alpha"], "bf16", seed=3)[0, 0]
    idx, val = oracle.topm_row(base, 64)
    vals = as_f64(base)
    ref = np.argsort(-vals, kind="stable")[:64]
    np.testing.assert_array_equal(idx, ref)
    assert len(np.unique(val)) < 64  # the workload really has bf16 ties in the top-64


# ------------------------------------------------------------ GRU step -----

def _gru_inputs(E, H, dtype, seed):
    cfg = small_cfg(V=7, E=E, H=H, dtype=dtype)
    inp = S.make_inputs(cfg, seed=seed, variant="strong")
    return inp


def _torch_cell(inp):
    E, H = inp["w_ih"].shape[1], inp["w_hh"].shape[1]
    cell = torch.nn.GRUCell(E, H).double()
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(as_f64(inp["w_ih"])))
        cell.weight_hh.copy_(torch.from_numpy(as_f64(inp["w_hh"])))
        cell.bias_ih.copy_(torch.from_numpy(as_f64(inp["b_ih"])))
        cell.bias_hh.copy_(torch.from_numpy(as_f64(inp["b_hh"])))
    return cell


@pytest.mark.parametrize("E,H", [(6, 5), (32, 32), (40, 17)])
def test_gru_f32_matches_torch_grucell(E, H):
    inp = _gru_inputs(E, H, "f32", seed=E + H)
    cell = _torch_cell(inp)
    rng = np.random.default_rng(0)
    for tok in range(inp["emb"].shape[0]):
        h = rng.uniform(-1, 1, H)
        got = oracle.gru(inp["emb"], tok, h, inp["w_ih"], inp["w_hh"], inp["b_ih"], inp["b_hh"])
        with torch.no_grad():
            ref = cell(torch.from_numpy(as_f64(inp["emb"][tok]))[None], torch.from_numpy(h)[None])[0]
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-13)


def test_gru_null_biases_are_zero():
    inp = _gru_inputs(6, 5, "f32", seed=1)
    h = np.linspace(-0.5, 0.5, 5)
    z = np.zeros_like(inp["b_ih"])
    a = oracle.gru(inp["emb"], 2, h, inp["w_ih"], inp["w_hh"], None, None)
    b = oracle.gru(inp["emb"], 2, h, inp["w_ih"], inp["w_hh"], z, z)
    np.testing.assert_array_equal(a, b)


def test_gru_bf16_weights_real_state_matches_torch_grucell():
    """bf16-stored weights and embeddings, a real-valued (unrounded) state."""
    inp = _gru_inputs(16, 8, "bf16", seed=5)
    cell = _torch_cell(inp)
    rng = np.random.default_rng(1)
    for tok in range(7):
        h = rng.uniform(-1, 1, 8)
        got = oracle.gru(inp["emb"], tok, h, inp["w_ih"], inp["w_hh"], inp["b_ih"], inp["b_hh"])
        with torch.no_grad():
            ref = cell(torch.from_numpy(as_f64(inp["emb"][tok]))[None], torch.from_numpy(h)[None])[0]
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-13)


# ------------------------------------------------- children distribution ---

@pytest.mark.parametrize("T", [0.0, 0.5, 1.0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dist_matches_torch_log_softmax(T, dtype):
    cfg = small_cfg(V=300, H=24, M=16, dtype=dtype)
    inp = S.make_inputs(cfg, seed=11, variant="strong")
    idx, val = topm_table(inp["base"][0], cfg["M"])
    rng = np.random.default_rng(2)
    h = rng.normal(0, 1, cfg["H"])
    tok, lp = oracle.dist(idx[2], val[2], inp["C"], h, T)
    z = torch.from_numpy(val[2]) + torch.from_numpy(as_f64(inp["C"]))[torch.from_numpy(idx[2])] @ torch.from_numpy(h)
    if T > 0:
        z = z / T
    ref = torch.log_softmax(z, 0).numpy()
    order = np.lexsort((idx[2], -ref))
    np.testing.assert_array_equal(tok, idx[2][order])
    np.testing.assert_allclose(lp, ref[order], rtol=0, atol=1e-13)
    assert abs(np.exp(lp).sum() - 1.0) < 1e-13
    assert np.all(lp <= 0)


def test_dist_ties_go_to_lower_token():
    V, H, M = 10, 3, 6
    Cm = np.zeros((V, H), np.float32)
    idx = np.array([9, 4, 7, 1, 3, 2], np.int32)
    val = np.array([1.0, 1.0, 0.5, 1.0, 0.5, -2.0])
    tok, lp = oracle.dist(idx, val, Cm, np.ones(H), 0.0)
    np.testing.assert_array_equal(tok, [1, 4, 9, 3, 7, 2])
    np.testing.assert_allclose(np.exp(lp).sum(), 1.0, atol=1e-15)


# ------------------------------------------------------ trees: brute force -

def _oracle_tree(inp, cfg, b=0):
    return oracle.build_request(inp, b, cfg["M"], cfg["n"], cfg["T"])


@pytest.mark.parametrize("L,M,n,T,seed", [
    (4, 4, 8, 0.0, 0), (4, 8, 16, 0.0, 1), (3, 5, 20, 0.5, 2), (6, 3, 12, 0.0, 3),
    (2, 6, 5, 1.0, 4), (4, 3, 40, 0.0, 5),
])
def test_tree_equals_bruteforce_top_n(L, M, n, T, seed):
    cfg = small_cfg(L=L, M=M, n=n, T=T, V=40, E=8, H=6)
    inp = S.make_inputs(cfg, seed=seed, variant="strong")
    sc = Scorer(inp, 0, M, T)
    nodes = best_n_bruteforce(sc, n)
    res = _oracle_tree(inp, cfg)
    assert res["count"] == len(nodes)
    assert_tree_equal(res, tree_arrays(nodes, n), n)


@pytest.mark.parametrize("variant", ["default", "strong"])
def test_tiny_workload_equals_branch_and_bound(variant):
    cfg = S.CONFIGS["tiny"]
    inp = S.make_inputs(cfg, seed=0, variant=variant)
    sc = Scorer(inp, 0, cfg["M"], cfg["T"])
    nodes = best_n_branch_and_bound(sc, cfg["n"])
    res = _oracle_tree(inp, cfg)
    assert res["count"] == cfg["n"]
    assert_tree_equal(res, tree_arrays(nodes, cfg["n"]), cfg["n"])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tree_maximizes_over_all_prefix_closed_sets(seed):
    cfg = small_cfg(L=3, M=3, n=4, V=12, E=4, H=3)
    inp = S.make_inputs(cfg, seed=seed, variant="strong")
    sc = Scorer(inp, 0, 3, 0.0)
    best_p, best_s, _ = prefix_closed_subsets_best(sc, 4)
    res = _oracle_tree(inp, cfg)
    s = res["scores"][1:]
    assert abs(np.exp(s).sum() - best_p) < 1e-12
    assert abs(s.sum() - best_s) < 1e-12


# ------------------------------------------ closed forms / special cases ---

def test_zero_correction_equals_factorized_tree():
    for name, over in [("tiny", {}), ("tiny", dict(T=0.5, M=6)), ("tiny", dict(n=40, L=5))]:
        cfg = S.with_config(name, **over)
        inp = S.make_inputs(cfg, seed=4, variant="zero_c")
        res = _oracle_tree(inp, cfg)
        ref = factorized_tree(inp["base"][0], cfg["M"], cfg["n"], cfg["T"])
        assert_tree_equal(res, ref, cfg["n"], atol=1e-12)


def test_zero_correction_bf16_ties_equal_factorized_tree():
    cfg = S.with_config("tiny", dtype="bf16", V=2000, M=32, n=40, L=6, alpha=2.0)
    inp = S.make_inputs(cfg, seed=9, variant="zero_c")
    res = _oracle_tree(inp, cfg)
    ref = factorized_tree(inp["base"][0], cfg["M"], cfg["n"], cfg["T"])
    assert_tree_equal(res, ref, cfg["n"], atol=1e-12)


def test_zero_gru_weights_equal_factorized_tree():
    cfg = S.with_config("tiny")
    inp = S.make_inputs(cfg, seed=6)
    for k in ("w_ih", "w_hh", "b_ih", "b_hh"):
        inp[k] = np.zeros_like(inp[k])
    res = _oracle_tree(inp, cfg)  # h stays 0 -> correction is 0
    ref = factorized_tree(inp["base"][0], cfg["M"], cfg["n"], cfg["T"])
    assert_tree_equal(res, ref, cfg["n"], atol=1e-12)


def test_m1_is_a_chain_of_top1_tokens():
    cfg = S.with_config("tiny", M=1, n=16, L=8)
    inp = S.make_inputs(cfg, seed=2, variant="strong")
    res = _oracle_tree(inp, cfg)
    idx, _ = topm_table(inp["base"][0], 1)
    assert res["count"] == 8  # min(n, L): the tree runs out of candidates
    np.testing.assert_array_equal(res["tokens"][1:9], idx[:, 0])
    np.testing.assert_array_equal(res["parents"][1:9], np.arange(8))
    np.testing.assert_array_equal(res["depths"][1:9], np.arange(1, 9))
    assert np.all(res["scores"][:9] == 0.0)
    assert np.all(res["tokens"][9:] == -1) and np.all(np.isneginf(res["scores"][9:]))
    assert res["mask"][9:].sum() == 0


def test_n1_is_the_argmax_of_the_first_corrected_slice():
    cfg = S.with_config("tiny", n=1)
    inp = S.make_inputs(cfg, seed=8, variant="strong")
    res = _oracle_tree(inp, cfg)
    idx, val = topm_table(inp["base"][0], cfg["M"])
    z = val[0] + as_f64(inp["C"])[idx[0]] @ inp["h0"][0].astype(np.float64)
    j = np.lexsort((idx[0], -z))[0]
    assert res["tokens"][1] == idx[0][j]
    ref = z[j] - (z.max() + np.log(np.exp(z - z.max()).sum()))
    assert abs(res["scores"][1] - ref) < 1e-12


def test_l1_is_the_sorted_root_list():
    cfg = S.with_config("tiny", L=1, n=5, M=8)
    inp = S.make_inputs(cfg, seed=3, variant="strong")
    res = _oracle_tree(inp, cfg)
    sc = Scorer(inp, 0, cfg["M"], 0.0)
    toks, lps = sc.children(sc.h0, 0)
    np.testing.assert_array_equal(res["tokens"][1:], toks[:5])
    np.testing.assert_allclose(res["scores"][1:], lps[:5], atol=1e-12)
    assert np.all(res["parents"][1:] == 0) and np.all(res["depths"][1:] == 1)


@pytest.mark.parametrize("fixture", ["hand_factorized.json", "hand_depth_tie.json"])
def test_hand_derived_example(fixture):
    """tests/golden/hand_*.json: 4-token, 2-position examples whose trees are
    derived by hand from the definitions (derivations are in the files)."""
    with open(os.path.join(GOLDEN, fixture)) as f:
        g = json.load(f)
    base = np.array(g["base"], np.float32)[None]
    V, E, H = base.shape[2], 2, 2
    inp = dict(base=base, emb=np.zeros((V, E), np.float32), w_ih=np.zeros((3 * H, E), np.float32),
               w_hh=np.zeros((3 * H, H), np.float32), b_ih=None, b_hh=None,
               C=np.zeros((V, H), np.float32), h0=None)
    res = oracle.build_request(inp, 0, g["M"], g["n"], 0.0)
    np.testing.assert_array_equal(res["tokens"], g["tokens"])
    np.testing.assert_array_equal(res["parents"], g["parents"])
    np.testing.assert_array_equal(res["depths"], g["depths"])
    ref = [eval(s, {"log": math.log, "exp": math.exp}) for s in g["scores_closed_form"]]
    np.testing.assert_allclose(res["scores"], ref, atol=1e-15)
    np.testing.assert_array_equal(res["mask"], g["mask"])
    # their exact ties add the same terms: every precision ties them, no flag
    assert res["flags"] == 0


def _zero_model_inputs(base):
    base = np.asarray(base, np.float32)[None]
    V, E, H = base.shape[2], 2, 2
    return dict(base=base, emb=np.zeros((V, E), np.float32), w_ih=np.zeros((3 * H, E), np.float32),
                w_hh=np.zeros((3 * H, H), np.float32), b_ih=None, b_hh=None,
                C=np.zeros((V, H), np.float32), h0=None)


def test_equal_scores_from_different_terms_are_near_ties():
    """Paths (token 0, token 1) and (token 1, token 0) over two positions with
    the same logits have mathematically equal scores built from different
    additions; floating point may break that tie either way, so it is flagged
    even when double precision happens to give an exact tie."""
    inp = _zero_model_inputs([[1.0, 0.5, -9.0, -9.0], [1.0, 0.5, -9.0, -9.0]])
    res = oracle.build_request(inp, 0, 2, 4, 0.0, eps=1e-5)
    assert res["flags"] & 1 and res["min_gap"] < 1e-12


# ---------------------------------------------------------- structure -----

def _check_structure(res, n, L):
    cnt = res["count"]
    par, dep, sc = res["parents"], res["depths"], res["scores"]
    for v in range(1, cnt + 1):
        q = par[v]
        assert 0 <= q < v                         # prefix-closed, parents first
        assert dep[v] == dep[q] + 1 and dep[v] <= L
        assert sc[v] <= sc[q]
    anc = np.zeros((n + 1, n + 1), np.uint8)
    for i in range(cnt + 1):
        j = i
        while j >= 0:
            anc[i, j] = 1
            j = par[j] if j > 0 else -1
    np.testing.assert_array_equal(res["mask"], anc)
    # pop order is the total order: non-increasing scores
    assert np.all(np.diff(sc[1:cnt + 1]) <= 0)


@pytest.mark.parametrize("name,variant", [("tiny", "default"), ("tiny", "strong")])
def test_structure_invariants(name, variant):
    cfg = S.CONFIGS[name]
    inp = S.make_inputs(cfg, seed=12, variant=variant)
    _check_structure(_oracle_tree(inp, cfg), cfg["n"], cfg["L"])


# ---------------------------------------------------------- metamorphic ---

def test_vocabulary_relabeling_maps_tokens():
    cfg = S.with_config("tiny", V=600)
    inp = S.make_inputs(cfg, seed=13, variant="strong")
    perm = np.random.default_rng(0).permutation(cfg["V"])  # old id t -> new id perm[t]
    inv = np.argsort(perm)
    inp2 = dict(inp)
    inp2["base"] = inp["base"][:, :, inv]
    inp2["emb"] = inp["emb"][inv]
    inp2["C"] = inp["C"][inv]
    a, b = _oracle_tree(inp, cfg), _oracle_tree(inp2, cfg)
    assert a["flags"] == 0 and b["flags"] == 0  # continuous fp32 draws: no near ties
    np.testing.assert_array_equal(b["tokens"][1:], perm[a["tokens"][1:]])
    np.testing.assert_array_equal(a["parents"], b["parents"])
    np.testing.assert_allclose(a["scores"], b["scores"], atol=1e-12)


def test_request_independent_of_batch():
    cfg = S.with_config("tiny", B=4)
    full = S.make_inputs(cfg, seed=14, variant="strong")
    one = S.make_inputs(cfg, seed=14, variant="strong", requests=[2])
    a = oracle.build_request(full, 2, cfg["M"], cfg["n"])
    b = oracle.build_request(one, 0, cfg["M"], cfg["n"])
    for k in ("tokens", "parents", "depths", "scores", "mask"):
        np.testing.assert_array_equal(a[k], b[k])


def test_score_paths_rescoring_agrees_with_tree():
    cfg = S.CONFIGS["tiny"]
    inp = S.make_inputs(cfg, seed=15, variant="strong")
    res = _oracle_tree(inp, cfg)
    paths = []
    for v in range(1, res["count"] + 1):
        p, j = [], v
        while j > 0:
            p.append(int(res["tokens"][j]))
            j = res["parents"][j]
        paths.append(p[::-1])
    s = oracle.score_paths(inp, 0, cfg["M"], paths, cfg["T"])
    np.testing.assert_array_equal(s, res["scores"][1:])


def test_near_tie_gap_is_reported():
    # two depth-1 candidates 1e-7 apart: a near tie that the flag must catch
    base = np.array([[0.0, -1e-7, -3.0, -4.0]], np.float32)
    V, E, H = 4, 2, 2
    inp = dict(base=base[None], emb=np.zeros((V, E), np.float32), w_ih=np.zeros((3 * H, E), np.float32),
               w_hh=np.zeros((3 * H, H), np.float32), b_ih=None, b_hh=None,
               C=np.zeros((V, H), np.float32), h0=None)
    res = oracle.build_request(inp, 0, 3, 2, 0.0, eps=1e-5)
    assert res["flags"] & 1
    assert 0 < res["min_gap"] < 1e-5
    # the first pop (slot 1) leaves its sibling 1e-7 below it in the queue
    assert res["first_flag"] == 1
    res = oracle.build_request(inp, 0, 3, 2, 0.0, eps=1e-8)
    assert res["flags"] == 0 and res["first_flag"] == 0


def test_near_tie_behind_an_exact_structural_tie_is_found():
    """After the second pop the queue holds the popped node's sibling (an exact
    tie adding the same terms: no flag) and, 1e-6 lower, the root's second
    child (different terms: a near tie).  Every candidate within eps counts,
    not only the best one."""
    import math as _m
    v1 = np.float32(1.0 - _m.log(2.0) - 1e-6)
    inp = _zero_model_inputs([[1.0, v1, -9.0, -9.0], [0.0, 0.0, -9.0, -9.0]])
    res = oracle.build_request(inp, 0, 2, 2, 0.0, eps=1e-5)
    np.testing.assert_array_equal(res["tokens"], [-1, 0, 0])
    np.testing.assert_array_equal(res["depths"], [0, 1, 2])
    assert res["flags"] & 1 and 5e-7 < res["min_gap"] < 2e-6
    # the first pop's gaps are 0.3 nats and more; the second pop is the near tie
    assert res["first_flag"] == 2


# ---- greedy acceptance walk -------------------------------------------------

def _accept_by_matched_set(tokens, parents, count, target):
    """The accepted path from its definition as a set: node c is accepted iff
    every edge (p -> child) on its root path has token(child) == target(p).
    Accepted nodes form one chain (siblings carry distinct tokens); its
    deepest node ends the walk."""
    S = len(tokens)
    acc = {0}
    changed = True
    while changed:  # fixed point, no assumption on slot order
        changed = False
        for c in range(1, min(count, S - 1) + 1):
            if c not in acc and parents[c] in acc and tokens[c] == target[parents[c]]:
                acc.add(c)
                changed = True
    depth = {0: 0}
    def d(c):
        if c not in depth:
            depth[c] = d(parents[c]) + 1
        return depth[c]
    end = max(acc, key=d)
    chain = []
    c = end
    while c != 0:
        chain.append(c)
        c = parents[c]
    return chain[::-1], int(target[end])


def test_accept_hand_derived_cases():
    g = json.load(open(os.path.join(GOLDEN, "hand_accept.json")))
    tok, par = g["tree"]["tokens"], g["tree"]["parents"]
    for case in g["cases"]:
        r = oracle.accept_greedy(tok, par, case["count"], case["target"])
        assert r["path"].tolist() == case["path"], case["why"]
        assert r["accepted"] == len(case["path"])
        assert r["bonus"] == case["bonus"], case["why"]


def _random_tree(rng, n, V, fanout_tokens=6):
    """A random prefix-closed tree in pop order (parent slot < child slot),
    siblings with distinct tokens drawn from a small alphabet so that
    matches are frequent."""
    tokens = [-1]
    parents = [-1]
    kids = {0: set()}
    for c in range(1, n + 1):
        for _ in range(100):
            p = int(rng.integers(0, c))
            t = int(rng.integers(0, fanout_tokens))
            if t not in kids[p]:
                break
        else:
            p, t = c - 1, 0
        kids[p].add(t)
        kids[c] = set()
        tokens.append(t)
        parents.append(p)
    return np.array(tokens, np.int32), np.array(parents, np.int32)


@pytest.mark.parametrize("seed", range(6))
def test_accept_equals_matched_set_on_random_trees(seed):
    rng = np.random.default_rng(seed)
    for _ in range(50):
        n = int(rng.integers(1, 20))
        tok, par = _random_tree(rng, n, 6)
        count = int(rng.integers(0, n + 1))
        target = rng.integers(0, 6, size=n + 1).astype(np.int32)
        r = oracle.accept_greedy(tok, par, count, target)
        path, bonus = _accept_by_matched_set(tok.tolist(), par.tolist(), count, target.tolist())
        assert r["path"].tolist() == path
        assert r["bonus"] == bonus


def test_accept_on_oracle_trees_with_synthetic_targets():
    cfg = S.CONFIGS["tiny"]
    inp = S.make_inputs(cfg, seed=3)
    res = oracle.build_request(inp, 0, cfg["M"], cfg["n"])
    tok, par, cnt = res["tokens"], res["parents"], res["count"]
    for p_follow in (0.0, 0.5, 1.0):
        tgt = S.make_greedy_targets(tok[None], par[None], np.array([cnt]), cfg["V"], p_follow, seed=1)[0]
        r = oracle.accept_greedy(tok, par, cnt, tgt)
        path, bonus = _accept_by_matched_set(tok.tolist(), par.tolist(), cnt, tgt.tolist())
        assert r["path"].tolist() == path and r["bonus"] == bonus
        if p_follow == 1.0:  # every node follows a child while it has one: the walk ends at a leaf
            end = path[-1] if path else 0
            assert all(par[c] != end for c in range(1, cnt + 1))


def test_accept_special_cases():
    tok = np.array([-1, 4, 5, 6], np.int32)
    par = np.array([-1, 0, 1, 2], np.int32)  # a chain
    # count 0: only the root; bonus is the target's first token
    r = oracle.accept_greedy(tok, par, 0, [4, 5, 6, 9])
    assert r["accepted"] == 0 and r["bonus"] == 4
    # the whole chain accepted: tau = n + 1 tokens in the round
    r = oracle.accept_greedy(tok, par, 3, [4, 5, 6, 9])
    assert r["path"].tolist() == [1, 2, 3] and r["bonus"] == 9
    # a mismatch in the middle stops the walk there
    r = oracle.accept_greedy(tok, par, 3, [4, 7, 6, 9])
    assert r["path"].tolist() == [1] and r["bonus"] == 7


# ---- full-vocabulary normalization (optional mode) -----------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,M,T", [(1000, 8, 0.0), (257, 64, 0.5), (3000, 17, 1.0), (70, 1, 2.0)])
def test_tail_lse_matches_scipy_logsumexp(dtype, V, M, T):
    from scipy.special import logsumexp
    cfg = small_cfg(V=V, L=1, dtype=dtype, alpha=1.1)
    row = S.make_inputs(cfg, seed=V + M)["base"][0, 0]
    x = as_f64(row)
    top = np.lexsort((np.arange(V), -x))[:M]  # numpy's ordering, not the oracle's
    keep = np.ones(V, bool)
    keep[top] = False
    want = logsumexp(x[keep] / (T if T > 0 else 1.0))
    assert oracle.tail_lse(row, M, T) == pytest.approx(want, abs=1e-12, rel=1e-13)


def test_tail_is_empty_when_m_equals_v():
    row = np.linspace(-3, 2, 11).astype(np.float32)
    assert oracle.tail_lse(row, 11) == -np.inf


@pytest.mark.parametrize("T", [0.0, 0.7])
def test_full_vocab_zero_correction_is_the_full_log_softmax(T):
    # with C = 0 the corrected logits are the base logits: the children's
    # log-probs are the log-softmax of the whole row, read at the top-M tokens
    cfg = small_cfg(V=500, L=1, M=12, H=7)
    inp = S.make_inputs(cfg, seed=4)
    row = inp["base"][0, 0]
    idx, val = oracle.topm_row(row, cfg["M"])
    tok, lp = oracle.dist(idx, val, np.zeros_like(inp["C"]), np.ones(cfg["H"]), T,
                          tail=oracle.tail_lse(row, cfg["M"], T))
    full = torch.log_softmax(torch.from_numpy(as_f64(row)) / (T if T > 0 else 1.0), dim=0).numpy()
    np.testing.assert_allclose(lp, full[tok], atol=1e-12)
    # and the M-slice mode differs from it by the slice's total mass
    _, lp_slice = oracle.dist(idx, val, np.zeros_like(inp["C"]), np.ones(cfg["H"]), T)
    assert np.all(lp < lp_slice)


@pytest.mark.parametrize("L,M,n,T,seed", [
    (4, 4, 8, 0.0, 0), (3, 5, 20, 0.5, 2), (6, 3, 12, 0.0, 3), (4, 3, 40, 1.0, 5),
])
def test_full_vocab_tree_equals_bruteforce_top_n(L, M, n, T, seed):
    cfg = small_cfg(L=L, M=M, n=n, T=T, V=40, E=8, H=6)
    inp = S.make_inputs(cfg, seed=seed, variant="strong")
    sc = Scorer(inp, 0, M, T, full_vocab=True)
    nodes = best_n_bruteforce(sc, n)
    res = oracle.build_request(inp, 0, M, n, T, full_vocab=True)
    assert res["count"] == len(nodes)
    assert_tree_equal(res, tree_arrays(nodes, n), n)


def test_full_vocab_tiny_equals_branch_and_bound():
    cfg = S.CONFIGS["tiny"]
    inp = S.make_inputs(cfg, seed=0, variant="strong")
    sc = Scorer(inp, 0, cfg["M"], cfg["T"], full_vocab=True)
    nodes = best_n_branch_and_bound(sc, cfg["n"])
    res = oracle.build_request(inp, 0, cfg["M"], cfg["n"], cfg["T"], full_vocab=True)
    assert res["count"] == cfg["n"]
    assert_tree_equal(res, tree_arrays(nodes, cfg["n"]), cfg["n"])


def test_full_vocab_with_m_equal_v_is_the_slice_mode():
    cfg = small_cfg(V=9, M=9, L=3, n=10)
    inp = S.make_inputs(cfg, seed=8, variant="strong")
    a = oracle.build_request(inp, 0, 9, 10, full_vocab=True)
    b = oracle.build_request(inp, 0, 9, 10)
    assert np.all(a["tail"] == -np.inf)
    for k in ("tokens", "parents", "depths", "scores"):
        np.testing.assert_array_equal(a[k], b[k])


def test_full_vocab_rescoring_agrees_with_tree():
    cfg = S.CONFIGS["tiny"]
    inp = S.make_inputs(cfg, seed=1)
    res = oracle.build_request(inp, 0, cfg["M"], cfg["n"], full_vocab=True)
    paths = []
    for v in range(1, res["count"] + 1):
        p, j = [], v
        while j > 0:
            p.append(int(res["tokens"][j]))
            j = res["parents"][j]
        paths.append(p[::-1])
    sc = oracle.score_paths(inp, 0, cfg["M"], paths, full_vocab=True)
    np.testing.assert_allclose(sc, res["scores"][1:res["count"] + 1], atol=1e-12)
