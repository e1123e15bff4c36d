"""Tree verification: one target pass over a tree of drafts, then a lossless walk (fp64 oracle).

Test infrastructure: only tests/, the smoke check and the benchmark's CPU
baseline use this module; the GPU path shares no code with it.

What the pages fix: "ReSpec: Towards Optimizing Speculative Decoding in
Reinforcement Learning Systems" (talk notes), GAP 1: the speculation
configuration (s, t, n) has a branching factor t, i.e. the drafts form a tree
that the target checks in one pass; "Accelerating RL Post-Training Rollouts
via System-Integrated Speculative Decoding" (gist.science summary), section 2:
verification is rejection sampling that keeps the rollout distribution equal to
the target's. The pages give neither the tree mask nor the tree acceptance rule;
the readings taken (plainest ones consistent with the lossless guarantee):

T1  Tree.  Node 0 is the root (the last committed token, position L); nodes
    1 .. N are drafts, node n with parent parents[n-1] in [0, n) and depth
    d(n) = d(parent) + 1, at position L + d(n). The children of a node, in index
    order, are its candidates; they were drawn independently from the draft
    distribution q_v at their parent v.
T2  Attention.  The caller has appended the KV rows of nodes 0 .. N at cache
    slots L .. L + N (node n at L + n). Node n's query row attends to the
    committed keys 0 .. L-1 and to the slots of its ancestors and itself
    (including the root): the tree mask.
T3  Walk (multi-candidate rejection sampling, as in SpecInfer, Miao et al.
    2024).  Start at the root. At node v with target distribution p_v:
      if v has no children, emit a bonus token from p_v and stop;
      otherwise r = p_v; for each child c_i (token x_i) in order: accept x_i iff
      u_i < r(x_i) / q_v(x_i) (q = 0: +inf if r > 0, else 0); on acceptance emit
      x_i and continue the walk at c_i; on rejection r = max(0, r - q_v)
      normalised (kept as is if that sum is 0). If every child is rejected,
      emit a sample of r and stop.
    With i.i.d. candidates this emits exactly p_v at every step; a chain-shaped
    tree (one child per node) is the ordinary chain.
T4  Uniforms.  The children of the node at depth d are decided at position
    P = L + d + 1; candidate 1 uses word 0 of Philox(P, seq, stream 0) (the
    chain's u_acc), candidate i >= 2 word 0 of stream i (stream 1 belongs to the
    draft generator); the final sample or bonus uses word 1 of stream 0 (the
    chain's u_smp). So a chain-shaped tree reproduces the chain's decisions.
T5  Outputs.  Emitted tokens (the accepted path, then the sampled token), a =
    depth of the last accepted node, the accepted node indices, p_v of every
    emitted token at its node, and min(1, r(x)/q(x)) of every tested node.
T6  Commit.  The committed prefix after the step is the root and the accepted
    path, so the KV rows of the accepted nodes n_1 .. n_a (path order) move to
    slots L+1 .. L+a (slot L+j takes what slot L+n_j held before the move; the
    root stays at L), then L' = L + a + 1 as for the chain. A commit that would
    pass the capacity is refused (the chain's rule) and then nothing moves;
    a <= 0 moves nothing. Slots past L+a keep their old rows: they lie beyond
    L' and the next step's append overwrites them.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

from .attention import attend, bf16_to_f64, gather_sequence_kv
from .commit import commit_lengths
from .philox import verify_uniforms
from .reject import Decision, inverse_cdf, softmax_t


def depths(parents) -> list:
    """d(n) for n = 0 .. N (T1)."""
    d = [0]
    for n, par in enumerate(parents, start=1):
        assert 0 <= par < n, (n, par)
        d.append(d[par] + 1)
    return d


def ancestors_or_self(parents, n: int) -> list:
    """Nodes on the path from the root to n, root first (T2)."""
    path = [n]
    while path[-1] != 0:
        path.append(int(parents[path[-1] - 1]))
    return path[::-1]


def children(parents, v: int) -> list:
    return [n for n in range(1, len(parents) + 1) if int(parents[n - 1]) == v]


def verify_attention_tree(q, k_cache, v_cache, block_table, seq_lens, parents, Hq: int, Hkv: int,
                          block_size: int, sm_scale: float, pairs=None) -> np.ndarray:
    """fp64 output [B][N+1][Hq][D]: node n attends keys 0..L-1 and the slots of its ancestors (T2).
    ``pairs`` restricts the work to a list of (b, kv_head); other rows are left as NaN."""
    B, N1, _, D = q.shape
    G = Hq // Hkv
    out = np.full((B, N1, Hq, D), np.nan, dtype=np.float64)
    todo = pairs if pairs is not None else [(b, g) for b in range(B) for g in range(Hkv)]
    for b, g in todo:
        L = int(seq_lens[b])
        K, Vv = gather_sequence_kv(k_cache, v_cache, block_table, b, g, L + N1, block_size)
        for n in range(N1):
            keys = list(range(L)) + [L + m for m in ancestors_or_self(parents[b], n)]
            for h in range(g * G, (g + 1) * G):
                out[b, n, h] = attend(bf16_to_f64(q[b, n, h]), K[keys], Vv[keys], sm_scale)
    return out


@dataclasses.dataclass
class TreeResult:
    tokens: list            # emitted tokens: accepted path, then the sampled / bonus token
    num_accepted: int       # a = depth of the last accepted node
    nodes: list             # accepted node indices, root excluded
    out_probs: list         # p_v(token) at the node each token was decided at
    accept_probs: dict      # node -> min(1, r(x)/q(x)) for every tested node
    decisions: list
    decision_nodes: list    # the tested node of each acceptance decision (-1 for a draw)


def walk(p_of, q_of, tokens, parents, L: int, uni) -> TreeResult:
    """The walk of T3. p_of(v) / q_of(v): target / draft distributions at node v;
    tokens[n-1]: token of node n; uni(P, stream) -> (word-0 unit, word-1 unit) (T4)."""
    v, depth = 0, 0
    out, nodes, probs, acc_probs, dec, dnodes = [], [], [], {}, [], []
    while True:
        P = L + depth + 1
        p = p_of(v)
        ch = children(parents, v)
        if not ch:
            y, margin = inverse_cdf(p, uni(P, 0)[1])
            dec.append(Decision("sample", depth, y, margin))
            dnodes.append(-1)
            out.append(y)
            probs.append(float(p[y]))
            return TreeResult(out, depth, nodes, probs, acc_probs, dec, dnodes)
        q = q_of(v)
        r = p
        moved = False
        for i, c in enumerate(ch, start=1):
            x = int(tokens[c - 1])
            rx, qx = float(r[x]), float(q[x])
            ratio = rx / qx if qx > 0.0 else (math.inf if rx > 0.0 else 0.0)
            u = uni(P, 0 if i == 1 else i)[0]
            acc_probs[c] = min(1.0, ratio)
            accepted = u < ratio
            dec.append(Decision("accept", depth, int(accepted), math.inf if math.isinf(ratio) else abs(u - ratio)))
            dnodes.append(c)
            if accepted:
                out.append(x)
                probs.append(float(p[x]))
                nodes.append(c)
                v, depth, moved = c, depth + 1, True
                break
            res = np.maximum(0.0, r - q)
            s = math.fsum(res)
            r = res / s if s > 0.0 else r
        if not moved:
            y, margin = inverse_cdf(r, uni(P, 0)[1])
            dec.append(Decision("sample", depth, y, margin))
            dnodes.append(-1)
            out.append(y)
            probs.append(float(p[y]))
            return TreeResult(out, depth, nodes, probs, acc_probs, dec, dnodes)


def verify_batch_tree(target_logits, draft_logits, draft_tokens, parents, seq_ids, seq_lens,
                      temperature: float, seed: int, rows_cache=None):
    """Batch driver; target_logits [B][N+1][V] (row n = node n), draft_logits [B][N+1][V] (row v =
    q at node v; rows of leaves unused), draft_tokens [B][N], parents [B][N]. Outputs padded like
    the C-ABI: out_tokens [B][N+1] (-1 after), accepted_nodes [B][N] (-1 after), out_probs
    [B][N+1] (0 after), accept_probs [B][N] (-1 for untested nodes).

    rows_cache: optional list of B empty dicts, kept by the caller across calls on the same logits
    and temperature (many seeds): the softmax rows of each sequence are then computed once."""
    B, N1, _ = target_logits.shape
    N = N1 - 1
    out_tokens = np.full((B, N1), -1, dtype=np.int32)
    accepted_nodes = np.full((B, max(N, 0)), -1, dtype=np.int32)
    out_probs = np.zeros((B, N1), dtype=np.float64)
    accept_probs = np.full((B, max(N, 0)), -1.0, dtype=np.float64)
    num_accepted = np.zeros(B, dtype=np.int32)
    results = []
    for b in range(B):
        if rows_cache is None:
            cache_p, cache_q = {}, {}
        else:
            cache_p = rows_cache[b].setdefault("p", {})
            cache_q = rows_cache[b].setdefault("q", {})

        def p_of(v, b=b, cache=cache_p):
            if v not in cache:
                cache[v] = softmax_t(target_logits[b, v], temperature)
            return cache[v]

        def q_of(v, b=b, cache=cache_q):
            if v not in cache:
                cache[v] = softmax_t(draft_logits[b, v], temperature)
            return cache[v]

        sid = int(seq_ids[b])
        res = walk(p_of, q_of, draft_tokens[b], parents[b], int(seq_lens[b]),
                   lambda P, stream, sid=sid: verify_uniforms(seed, sid, P, stream))
        n = len(res.tokens)
        out_tokens[b, :n] = res.tokens
        out_probs[b, :n] = res.out_probs
        accepted_nodes[b, : len(res.nodes)] = res.nodes
        for node, ap in res.accept_probs.items():
            accept_probs[b, node - 1] = ap
        num_accepted[b] = res.num_accepted
        results.append(res)
    return dict(out_tokens=out_tokens, num_accepted=num_accepted, accepted_nodes=accepted_nodes,
                out_probs=out_probs, accept_probs=accept_probs, results=results)


def commit_tree(k_cache, v_cache, block_table, seq_lens, accepted_nodes, num_accepted, capacity_tokens: int):
    """T6 on the paged caches (K [pages][Hkv][bs][D], V [pages][Hkv][D][bs]). Every row is read
    from the caches as they were before the call and written into copies, so the order of the
    moves cannot matter. Returns (k_cache', v_cache', new lengths, overflow flags)."""
    kc, vc = k_cache.copy(), v_cache.copy()
    new_L, overflow = commit_lengths(seq_lens, num_accepted, capacity_tokens)
    bs = k_cache.shape[2]

    def where(b, s):
        return int(block_table[b, s // bs]), s % bs

    for b in range(len(seq_lens)):
        L, a = int(seq_lens[b]), int(num_accepted[b])
        if overflow[b] or a <= 0:
            continue
        for j in range(1, a + 1):
            ps, os_ = where(b, L + int(accepted_nodes[b, j - 1]))
            pd, od = where(b, L + j)
            kc[pd, :, od, :] = k_cache[ps, :, os_, :]
            vc[pd, :, :, od] = v_cache[ps, :, :, os_]
    return kc, vc, new_L, overflow
