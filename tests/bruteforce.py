"""Independent cross-checks for the oracle (test helpers, CPU only).

Nothing here imports the oracle or the GPU library.  Scores are computed with
library routines -- ``torch.nn.GRUCell`` and ``torch.log_softmax`` in float64,
``numpy.lexsort`` for orderings -- and the tree is found by exhaustive
enumeration of the candidate tree rather than by a priority queue.

The candidate tree of a request: the root (depth 0), and below a node at depth
d < L one child per token of the depth-(d+1) top-M set (block position d).  A
node's key is its cumulative conditional log-prob; the n best nodes under the
total order (score desc, depth asc, parent's order, sibling rank asc) form the
tree the best-first builder must return, in that order.
"""
from __future__ import annotations

import functools
import heapq
import itertools

import numpy as np
import torch

import synthetic as S


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return S.bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, np.float64)


def topm_table(base_req: np.ndarray, M: int):
    """Per position: (idx, val) of the M best tokens, (value desc, id asc)."""
    vals = as_f64(base_req)
    L, V = vals.shape
    idx = np.empty((L, M), np.int64)
    for p in range(L):
        order = np.lexsort((np.arange(V), -vals[p]))  # last key is primary
        idx[p] = order[:M]
    val = np.take_along_axis(vals, idx, axis=1)
    return idx, val


class Scorer:
    """Conditional child distributions via torch library routines (float64)."""

    def __init__(self, inp: dict, b: int, M: int, T: float, full_vocab: bool = False):
        self.idx, self.val = topm_table(inp["base"][b], M)
        self.L = self.idx.shape[0]
        self.T = T
        # full-vocabulary normalization: every row's logits outside its top M
        # (uncorrected) join the softmax
        self.full_vocab = full_vocab
        if full_vocab:
            rows = as_f64(inp["base"][b])
            keep = np.ones(rows.shape, bool)
            np.put_along_axis(keep, self.idx, False, axis=1)
            self.tail_logits = [torch.from_numpy(rows[p][keep[p]]) for p in range(self.L)]
        self.emb = torch.from_numpy(as_f64(inp["emb"]))
        self.C = torch.from_numpy(as_f64(inp["C"]))
        H, E = inp["w_hh"].shape[1], inp["w_ih"].shape[1]
        cell = torch.nn.GRUCell(E, H, bias=True).double()
        with torch.no_grad():
            cell.weight_ih.copy_(torch.from_numpy(as_f64(inp["w_ih"])))
            cell.weight_hh.copy_(torch.from_numpy(as_f64(inp["w_hh"])))
            cell.bias_ih.copy_(torch.from_numpy(as_f64(inp["b_ih"])) if inp.get("b_ih") is not None
                               else torch.zeros(3 * H, dtype=torch.float64))
            cell.bias_hh.copy_(torch.from_numpy(as_f64(inp["b_hh"])) if inp.get("b_hh") is not None
                               else torch.zeros(3 * H, dtype=torch.float64))
        self.cell = cell
        h0 = inp.get("h0")
        self.h0 = (torch.zeros(H, dtype=torch.float64) if h0 is None
                   else torch.from_numpy(np.asarray(h0[b], np.float64)))

    def children(self, h: torch.Tensor, pos: int):
        """Sorted (tokens, logp) of the children at block position pos."""
        idx = self.idx[pos]
        z = torch.from_numpy(self.val[pos]) + self.C[torch.from_numpy(idx)] @ h
        if self.T > 0:
            z = z / self.T
        if self.full_vocab:
            tail = self.tail_logits[pos] / (self.T if self.T > 0 else 1.0)
            lp = (z - torch.logsumexp(torch.cat([z, tail]), dim=0)).numpy()
        else:
            lp = torch.log_softmax(z, dim=0).numpy()
        order = np.lexsort((idx, -lp))
        return idx[order], lp[order]

    @torch.no_grad()
    def step(self, h: torch.Tensor, tok: int) -> torch.Tensor:
        return self.cell(self.emb[tok][None], h[None])[0]


class Node:
    __slots__ = ("tokens", "score", "depth", "parent", "rank", "h", "kids")

    def __init__(self, tokens, score, depth, parent, rank, h):
        self.tokens, self.score, self.depth = tokens, score, depth
        self.parent, self.rank, self.h, self.kids = parent, rank, h, None


def node_cmp(a: Node, b: Node) -> int:
    """-1 when a precedes b in the total order."""
    if a.score != b.score:
        return -1 if a.score > b.score else 1
    if a.depth != b.depth:
        return -1 if a.depth < b.depth else 1
    if a.parent is not b.parent:
        return node_cmp(a.parent, b.parent)
    return (a.rank > b.rank) - (a.rank < b.rank)


def _expand(sc: Scorer, node: Node):
    if node.kids is None:
        toks, lps = sc.children(node.h, node.depth)
        node.kids = (toks, lps)
    return node.kids


def enumerate_all(sc: Scorer):
    """Every node of the candidate tree (M^1 + ... + M^L of them)."""
    root = Node((), 0.0, 0, None, 0, sc.h0)
    out, stack = [], [root]
    while stack:
        q = stack.pop()
        if q.depth == sc.L:
            continue
        toks, lps = _expand(sc, q)
        for r, (t, lp) in enumerate(zip(toks, lps)):
            child = Node(q.tokens + (int(t),), q.score + float(lp), q.depth + 1, q, r, None)
            if child.depth < sc.L:
                child.h = sc.step(q.h, int(t))
            out.append(child)
            stack.append(child)
    return out


def best_n_bruteforce(sc: Scorer, n: int):
    """The n first nodes of the total order, by full enumeration."""
    nodes = enumerate_all(sc)
    nodes.sort(key=functools.cmp_to_key(node_cmp))
    return nodes[:n]


def best_n_branch_and_bound(sc: Scorer, n: int):
    """Same result as best_n_bruteforce without visiting the whole tree: a
    subtree is skipped when its root already comes after the current n-th
    best node (keys never improve along a path: log-probs are <= 0 and a
    child's depth is larger)."""
    root = Node((), 0.0, 0, None, 0, sc.h0)
    best: list[Node] = []
    key = functools.cmp_to_key(node_cmp)

    def visit(q: Node):
        if q.depth == sc.L:
            return
        toks, lps = _expand(sc, q)
        for r, (t, lp) in enumerate(zip(toks, lps)):
            child = Node(q.tokens + (int(t),), q.score + float(lp), q.depth + 1, q, r, None)
            if len(best) == n and node_cmp(child, best[-1]) > 0:
                break  # this and every later (worse-ranked) sibling is out
            best.append(child)
            best.sort(key=key)
            del best[n:]
            if child.depth < sc.L:
                child.h = sc.step(q.h, int(t))
                visit(child)

    visit(root)
    return best


def tree_arrays(nodes: list, n: int):
    """Tree slots from nodes given in pop order: tokens/parents/depths/scores."""
    slot = {(): 0}
    tokens, parents, depths, scores = [-1], [-1], [0], [0.0]
    for i, nd in enumerate(nodes, start=1):
        slot[nd.tokens] = i
        tokens.append(nd.tokens[-1])
        parents.append(slot[nd.tokens[:-1]])
        depths.append(nd.depth)
        scores.append(nd.score)
    while len(tokens) < n + 1:
        tokens.append(-1); parents.append(-1); depths.append(-1); scores.append(-np.inf)
    return (np.array(tokens), np.array(parents), np.array(depths), np.array(scores))


def factorized_tree(base_req: np.ndarray, M: int, n: int, T: float = 0.0):
    """DDTree's factorized best-first tree over the same per-depth M-slice
    log-softmax, computed with Python's heapq (no GRU, no correction).
    Returns tokens, parents, depths, scores arrays with n+1 slots."""
    idx, val = topm_table(base_req, M)
    L = idx.shape[0]
    dists = []
    for p in range(L):
        z = torch.from_numpy(val[p])
        if T > 0:
            z = z / T
        lp = torch.log_softmax(z, dim=0).numpy()
        order = np.lexsort((idx[p], -lp))
        dists.append((idx[p][order], lp[order]))
    tokens, parents, depths, scores = [-1], [-1], [0], [0.0]
    # heap entries: (-score, depth, parent slot, rank)
    heap = [(-(0.0 + dists[0][1][0]), 1, 0, 0)]
    while len(tokens) <= n and heap:
        negs, d, q, r = heapq.heappop(heap)
        v = len(tokens)
        tokens.append(int(dists[d - 1][0][r]))
        parents.append(q)
        depths.append(d)
        scores.append(-negs)
        if r + 1 < M:
            heapq.heappush(heap, (-(scores[q] + dists[d - 1][1][r + 1]), d, q, r + 1))
        if d < L:
            heapq.heappush(heap, (-(scores[v] + dists[d][1][0]), d + 1, v, 0))
    while len(tokens) < n + 1:
        tokens.append(-1); parents.append(-1); depths.append(-1); scores.append(-np.inf)
    return np.array(tokens), np.array(parents), np.array(depths), np.array(scores)


def prefix_closed_subsets_best(sc: Scorer, n: int):
    """Among ALL prefix-closed sets of n non-root nodes, the largest sum of
    path probabilities sum(exp(score)) and of scores; exhaustive (tiny trees)."""
    nodes = enumerate_all(sc)
    ids = {nd.tokens: i for i, nd in enumerate(nodes)}
    best_p, best_s = -np.inf, -np.inf
    for combo in itertools.combinations(range(len(nodes)), n):
        chosen = {nodes[i].tokens for i in combo}
        if any(len(t) > 1 and t[:-1] not in chosen for t in chosen):
            continue
        best_p = max(best_p, sum(np.exp(nodes[i].score) for i in combo))
        best_s = max(best_s, sum(nodes[i].score for i in combo))
    return best_p, best_s, ids
