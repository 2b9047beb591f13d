"""Seeded synthetic workloads for the conditional draft-tree builder.

This module only draws inputs; it holds none of the method's arithmetic.  It
is the one module both the GPU library's callers (tests, bench) and the CPU
oracle's callers use, so that both sides see identical bytes.

Recipe (stands in for the drafter outputs on the paper's eight benchmark
datasets, which are not available):

* base logits ``[B, L, V]``: for every (request b, block position p) draw an
  independent uniform permutation ``pi`` of the vocabulary and noise
  ``eps_r ~ N(0, 0.5)``; token ``pi[r-1]`` gets ``-alpha * ln(r) + eps_r`` for
  ranks ``r = 1..V`` (a Zipf(alpha)-shaped logit profile with noise);
* GRU weights ``W_ih [3H,E]``, ``W_hh [3H,H]``, embedding ``emb [V,E]`` and
  correction matrix ``C [V,H]`` are ``N(0, 1/sqrt(fan_in))`` with fan_in the
  input width of each matrix; biases ``[3H]`` are ``N(0, 1/sqrt(H))``;
* ``h0 = 0`` unless a variant says otherwise;
* everything is drawn in float32 (logits in float64 then rounded to float32)
  and, for bf16 configurations, rounded to bf16 with round-to-nearest-even.
  bf16 arrays are carried as ``uint16`` bit patterns.

* greedy target tokens ``[B, n+1]`` for the acceptance walk (the target
  model's argmax after each tree node, which needs the target model): for
  every slot of a given tree, with probability ``p_follow`` the token of that
  node's earliest child (lowest slot: the draft's own first choice there),
  otherwise a token drawn uniformly from the vocabulary (slots past
  ``count``: -1);
* random trees ``[B, n+1]`` in the builder's output format (for the acceptance
  walk on its own): slot c > 0 gets a parent drawn uniformly from slots < c
  and a token drawn from a small alphabet, distinct among siblings; the node
  count is drawn uniformly from 0..n, or is n.

Seeds: ``numpy.random.default_rng(SeedSequence([seed, tensor_id, b + 1]))`` for
per-request tensors (positions drawn in order from that stream); shared
matrices are drawn in blocks of 8192 rows, block i from
``SeedSequence([seed, tensor_id, 0, i])``.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Named workloads.  dtype "f32" or "bf16"; T = 0 means unscaled logits.
CONFIGS = {
    # small case the oracle finishes in well under a second
    "tiny": dict(B=1, V=1000, L=8, E=32, H=32, M=8, n=16, dtype="f32", alpha=1.1, T=0.0),
    # Qwen3-4B-shaped drafter, one request
    "qwen3_4b_single": dict(B=1, V=151936, L=16, E=2560, H=1024, M=64, n=16, dtype="bf16",
                            alpha=1.1, T=0.0),
    # Qwen3-4B-shaped drafter, 64 independent requests (the measured workload)
    "qwen3_4b_batched": dict(B=64, V=151936, L=16, E=2560, H=1024, M=64, n=16, dtype="bf16",
                             alpha=1.1, T=0.0),
    # Qwen3-8B-shaped drafter, T = 1.0, flatter logits
    "qwen3_8b": dict(B=32, V=151936, L=16, E=4096, H=1024, M=64, n=16, dtype="bf16",
                     alpha=0.8, T=1.0),
    # Qwen3-4B shapes with a 256-wide GRU state, so that the correction head
    # C = W_2 is [V, 256] (the 256 x M slice the pages print)
    "qwen3_4b_head256": dict(B=64, V=151936, L=16, E=2560, H=256, M=64, n=16, dtype="bf16",
                             alpha=1.1, T=0.0),
    # large batch, large budget, peaked logits (long chains)
    "stress": dict(B=256, V=151936, L=16, E=2560, H=1024, M=64, n=64, dtype="bf16",
                   alpha=2.0, T=0.0),
}

_TID = {"base": 1, "emb": 2, "w_ih": 3, "w_hh": 4, "b_ih": 5, "b_hh": 6, "C": 7, "h0": 8,
        "target": 9, "tree": 10}


def _rng(seed: int, name: str, b: int | None):
    return np.random.default_rng(np.random.SeedSequence([seed, _TID[name], 0 if b is None else b + 1]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); uint16 bits.

    Adding 0x7FFF plus the lowest kept bit and truncating is round-to-nearest-
    even on the 16 dropped bits.  Done in place on 8M-element chunks."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).reshape(-1)
    out = np.empty(u.shape, np.uint16)
    step = 1 << 23
    for s in range(0, u.size, step):
        c = u[s:s + step]
        t = c >> np.uint32(16)
        t &= np.uint32(1)
        t += np.uint32(0x7FFF)
        t += c
        t >>= np.uint32(16)
        out[s:s + step] = t
    return out.reshape(np.shape(x))


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _cast(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def zipf_row(rng, V: int, alpha: float, noise_std: float = 0.5) -> np.ndarray:
    perm = rng.permutation(V)
    noise = rng.normal(0.0, noise_std, V)
    ranks = np.arange(1, V + 1, dtype=np.float64)
    row = np.empty(V, np.float64)
    row[perm] = -alpha * np.log(ranks) + noise
    return row.astype(np.float32)


def make_base(B, L, V, alpha, dtype, seed=0, requests=None) -> np.ndarray:
    reqs = list(range(B)) if requests is None else list(requests)
    out = np.empty((len(reqs), L, V), np.uint16 if dtype == "bf16" else np.float32)

    def one(i):
        rng = _rng(seed, "base", reqs[i])
        for p in range(L):
            out[i, p] = _cast(zipf_row(rng, V, alpha), dtype)

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(one, range(len(reqs))))
    return out


_ROWS_PER_BLOCK = 8192


def _normal(seed, name, shape, std, dtype):
    """N(0, std) matrix drawn in blocks of 8192 rows; block i uses
    SeedSequence([seed, tensor_id, 0, i]).  Blocks run on worker threads."""
    rows = shape[0]
    out = np.empty(shape, np.uint16 if dtype == "bf16" else np.float32)
    nblk = (rows + _ROWS_PER_BLOCK - 1) // _ROWS_PER_BLOCK

    def blk(i):
        r0, r1 = i * _ROWS_PER_BLOCK, min(rows, (i + 1) * _ROWS_PER_BLOCK)
        rng = np.random.default_rng(np.random.SeedSequence([seed, _TID[name], 0, i]))
        x = rng.standard_normal((r1 - r0,) + tuple(shape[1:]), dtype=np.float32)
        x *= np.float32(std)
        out[r0:r1] = _cast(x, dtype)

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(blk, range(nblk)))
    return out


def make_inputs(cfg: dict, seed: int = 0, variant: str = "default", requests=None, skip=()) -> dict:
    """Inputs of a workload as numpy arrays.

    variant: "default"; "strong" (h0 ~ N(0,1) and C scaled by 10, to make the
    correction change trees); "zero_c" (C = 0: the factorized ablation).
    ``requests`` restricts the per-request tensors to those request ids
    (their values equal those of the full batch).  Tensors named in ``skip``
    ("base", "emb") are not drawn (None): they depend on neither H nor the
    variant, so a caller can reuse them from another workload of the same
    B, L, V, E, alpha and seed.
    """
    B, V, L, E, H = cfg["B"], cfg["V"], cfg["L"], cfg["E"], cfg["H"]
    dt = cfg["dtype"]
    reqs = list(range(B)) if requests is None else list(requests)
    inp = {
        "base": None if "base" in skip else make_base(B, L, V, cfg["alpha"], dt, seed, reqs),
        "emb": None if "emb" in skip else _normal(seed, "emb", (V, E), 1.0 / math.sqrt(E), dt),
        "w_ih": _normal(seed, "w_ih", (3 * H, E), 1.0 / math.sqrt(E), dt),
        "w_hh": _normal(seed, "w_hh", (3 * H, H), 1.0 / math.sqrt(H), dt),
        "b_ih": _normal(seed, "b_ih", (3 * H,), 1.0 / math.sqrt(H), dt),
        "b_hh": _normal(seed, "b_hh", (3 * H,), 1.0 / math.sqrt(H), dt),
    }
    cscale = 10.0 if variant == "strong" else 1.0
    if variant == "zero_c":
        inp["C"] = np.zeros((V, H), np.uint16 if dt == "bf16" else np.float32)
    else:
        inp["C"] = _normal(seed, "C", (V, H), cscale / math.sqrt(H), dt)
    h0 = np.zeros((len(reqs), H), np.float32)
    if variant == "strong":
        for i, b in enumerate(reqs):
            h0[i] = _rng(seed, "h0", b).standard_normal(H, dtype=np.float32)
    inp["h0"] = h0
    return inp


def with_config(name: str, **over) -> dict:
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    return cfg


def to_torch(inp: dict, device) -> dict:
    """The same inputs as torch tensors on `device` (uint16 bf16 patterns become
    torch.bfloat16; None stays None)."""
    import torch

    out = {}
    for k, v in inp.items():
        if v is None:
            out[k] = None
        elif v.dtype == np.uint16:
            out[k] = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).to(device)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(v)).to(device)
    return out


def make_greedy_targets(tokens: np.ndarray, parents: np.ndarray, count: np.ndarray, V: int,
                        p_follow: float, seed: int = 0) -> np.ndarray:
    """Synthetic greedy target tokens ``[B, n+1]`` int32 for trees ``tokens`` /
    ``parents`` ``[B, n+1]`` with ``count[b]`` nodes: slot i takes the token of
    node i's earliest child with probability ``p_follow``, else a uniform
    vocabulary token; slots past ``count[b]`` hold -1."""
    tokens = np.asarray(tokens)
    parents = np.asarray(parents)
    B, S = tokens.shape
    out = np.full((B, S), -1, np.int32)
    for b in range(B):
        rng = _rng(seed, "target", b)
        c = int(count[b])
        kids = [[] for _ in range(S)]
        for j in range(1, c + 1):
            if 0 <= parents[b, j] < S:
                kids[int(parents[b, j])].append(int(tokens[b, j]))
        for i in range(c + 1):
            follow = rng.random() < p_follow
            pick = rng.integers(0, 1 << 30)
            if follow and kids[i]:
                out[b, i] = kids[i][0]
            else:
                out[b, i] = pick % V
    return out


def make_random_trees(B: int, n: int, V: int, seed: int = 0, alphabet: int = 6,
                      full: bool = False):
    """Random prefix-closed trees in pop order: (tokens, parents) [B, n+1] int32
    and count [B] int32.  Tokens come from an alphabet of ``alphabet`` ids
    spread over the vocabulary, distinct among the children of one node."""
    alphabet = max(1, min(alphabet, V))
    step = max(1, V // alphabet)
    tok = np.full((B, n + 1), -1, np.int32)
    par = np.full((B, n + 1), -1, np.int32)
    cnt = np.zeros(B, np.int32)
    for b in range(B):
        rng = _rng(seed, "tree", b)
        kids = {0: set()}
        for c in range(1, n + 1):
            p, t = c - 1, None
            for _ in range(64):
                p = int(rng.integers(0, c))
                a = int(rng.integers(0, alphabet))
                if a not in kids[p]:
                    t = a
                    break
            if t is None:  # every draw collided: hang the node under its predecessor
                p = c - 1
                t = int(rng.integers(0, alphabet))
            kids[p].add(t)
            kids[c] = set()
            tok[b, c] = t * step
            par[b, c] = p
        cnt[b] = n if full else int(rng.integers(0, n + 1))
    return tok, par, cnt
