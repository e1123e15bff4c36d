"""Draft trees for tree verification: shapes, node rows and i.i.d. children.

A tree of branching factor t and depth d has its nodes numbered breadth first
(node 0 is the last committed token). Node n's target logits follow the recipe of
the chain's rows; its draft logits are the target's plus noise; the token of node
n is drawn from the draft distribution at its parent, independently for siblings
(the drafting the tree walk assumes). Like the rest of this package it only draws
numbers and lays them out.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from .gen import Preset, draft_from_logits, make_attention_inputs, make_reject_inputs


def tree_parents(t: int, depth: int) -> np.ndarray:
    """parents [N] of the full t-ary tree of the given depth, breadth first."""
    parents, frontier, n = [], [0], 0
    for _ in range(depth):
        nxt = []
        for v in frontier:
            for _ in range(t):
                n += 1
                parents.append(v)
                nxt.append(n)
        frontier = nxt
    return np.array(parents, dtype=np.int32)


def random_parents(rng: np.random.Generator, N: int, max_children: int = 4) -> np.ndarray:
    """A random tree of N draft nodes (parent of n uniform over earlier nodes with room)."""
    parents, kids = [], [0] * (N + 1)
    for n in range(1, N + 1):
        choices = [v for v in range(n) if kids[v] < max_children]
        v = int(rng.choice(choices))
        parents.append(v)
        kids[v] += 1
    return np.array(parents, dtype=np.int32)


def random_paths(rng: np.random.Generator, parents: np.ndarray, stop: float = 0.25) -> tuple:
    """A random root-to-node path in each sequence's tree: from the root, stop with probability
    `stop` (or at a leaf), else step to a uniformly chosen child. Returns (accepted_nodes [B][N],
    path order then -1; depth [B]) for parents [B][N]."""
    par = np.asarray(parents)
    B, N = par.shape
    nodes = np.full((B, N), -1, dtype=np.int32)
    depth = np.zeros(B, dtype=np.int32)
    for b in range(B):
        v, d = 0, 0
        while True:
            kids = [n for n in range(1, N + 1) if int(par[b, n - 1]) == v]
            if not kids or rng.random() < stop:
                break
            v = int(rng.choice(kids))
            nodes[b, d] = v
            d += 1
        depth[b] = d
    return nodes, depth


def make_tree_reject_inputs(preset: Preset, parents: np.ndarray, seed: int | None = None, B: int | None = None) -> dict:
    """target [B][N+1][V], draft [B][N+1][V], tokens [B][N] drawn from q at each parent,
    parents [B][N] (the same tree for every sequence if a 1-d array is given)."""
    s = preset.index if seed is None else seed
    par = np.asarray(parents, dtype=np.int32)
    N = par.shape[-1]
    base = make_reject_inputs(dataclasses.replace(preset, k=N), seed=s, B=B)
    B = base["B"]
    rng = np.random.Generator(np.random.PCG64(7000 + s))
    target = base["target_logits"]                                  # [B][N+1][V]
    noise = rng.standard_normal(target.shape, dtype=np.float32) * np.float32(preset.draft_sigma)
    draft = np.ascontiguousarray(target + noise, dtype=np.float32)  # one draft row per node
    par_b = np.broadcast_to(par, (B, N)).copy() if par.ndim == 1 else par.copy()
    tokens = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        for n in range(1, N + 1):
            tokens[b, n - 1] = draft_from_logits(rng, draft[b, par_b[b, n - 1]][None], preset.temperature)[0]
    out = dict(base)
    out.update(k=N, target_logits=target, draft_logits=draft, draft_tokens=tokens, parents=par_b)
    return out


def make_tree_attention_inputs(preset: Preset, N: int, seed: int | None = None, B: int | None = None) -> dict:
    """Attention inputs for N draft nodes: the cache holds L_b + N + 1 keys, the KV rows of
    nodes 0 .. N at slots L_b .. L_b + N; q [B][N+1][Hq][D]."""
    return make_attention_inputs(dataclasses.replace(preset, k=N), seed=seed, B=B)
