"""Pins for the tree-verification oracle (CPU only).

* A chain-shaped tree (one child per node) is the ordinary chain: the walk
  reproduces the chain oracle's outputs decision for decision, and the tree mask
  reproduces the causal verify attention.
* A star (every draft a child of the root) sees only the cache, the root and
  itself; attention is checked against a dense masked softmax built from scratch.
* Over the 2^24 grid of one candidate's uniform, with the earlier candidates
  rejected, the accept count equals ceil(r(x)/q(x) 2^24) for the residual r left by
  those rejections, and the final draw's counts equal the residual's interval
  widths: the walk uses the right uniform and the right residual at every step.
* Monte Carlo, multi-round with the commit: generating tokens by repeated tree
  rounds (branching 2, depth 2, children drawn i.i.d. from the draft) gives the
  target Markov chain's joint law (chi-squared, fixed seeds): the walk is lossless.
* The tree commit: after moving the accepted path, plain causal attention over
  the cache at depth j of the path gives exactly what the tree mask gave that
  node before the move (the mask's definition, not the move's code); a
  chain-shaped path moves nothing; only the slots L+1 .. L+a change, and an
  overflowing commit changes nothing.
"""

import math

import numpy as np
from scipy import stats

from oracle import attention as oatt
from oracle import commit as ocommit
from oracle import reject as orej
from oracle import tree as otree
from oracle.philox import verify_uniforms
from workloads import (PRESETS, draft_from_logits, make_attention_inputs, make_reject_inputs,
                       make_tree_attention_inputs, random_parents, random_paths)

GRID = 1 << 24


def test_chain_shaped_tree_is_the_chain():
    inp = make_reject_inputs(PRESETS["tiny"], B=6)
    B, k = inp["B"], inp["k"]
    parents = np.tile(np.arange(k, dtype=np.int32), (B, 1))          # node n's parent is n - 1
    draft_rows = np.concatenate([inp["draft_logits"], inp["draft_logits"][:, :1]], axis=1)   # leaf row unused
    for seed in range(40):
        t = otree.verify_batch_tree(inp["target_logits"], draft_rows, inp["draft_tokens"], parents, inp["seq_ids"],
                                    inp["seq_lens"], 1.0, seed)
        c = orej.verify_batch(inp["target_logits"], inp["draft_logits"], inp["draft_tokens"], inp["seq_ids"],
                              inp["seq_lens"], k, 1.0, seed)
        for key in ("out_tokens", "num_accepted", "out_probs", "accept_probs"):
            np.testing.assert_array_equal(t[key], c[key], err_msg=key)
        for b in range(B):
            a = int(t["num_accepted"][b])
            assert list(t["accepted_nodes"][b, :a]) == list(range(1, a + 1))


def test_chain_shaped_tree_attention_is_causal_verify_attention():
    a = make_attention_inputs(PRESETS["tiny"], B=3)
    k = a["k"]
    parents = np.tile(np.arange(k, dtype=np.int32), (3, 1))
    t = otree.verify_attention_tree(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], parents,
                                    a["Hq"], a["Hkv"], a["block_size"], a["sm_scale"])
    c = oatt.verify_attention(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], k, a["Hq"],
                              a["Hkv"], a["block_size"], a["sm_scale"])
    np.testing.assert_allclose(t, c, rtol=0, atol=1e-14)


def test_star_tree_attention_against_a_dense_masked_softmax():
    a = make_attention_inputs(PRESETS["tiny"], B=2)
    k, Hq, Hkv, D, bs = a["k"], a["Hq"], a["Hkv"], a["D"], a["block_size"]
    parents = np.zeros((2, k), dtype=np.int32)                        # every draft hangs off the root
    t = otree.verify_attention_tree(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], parents,
                                    Hq, Hkv, bs, a["sm_scale"])
    G = Hq // Hkv
    for b in range(2):
        L = int(a["seq_lens"][b])
        n_keys = L + k + 1
        for h in range(Hq):
            g = h // G
            # dense K, V from the block table, key by key
            K = np.array([oatt.bf16_to_f64(a["k_cache"][a["block_table"][b, s // bs], g, s % bs]) for s in range(n_keys)])
            Vv = np.array([oatt.bf16_to_f64(a["v_cache"][a["block_table"][b, s // bs], g, :, s % bs])
                           for s in range(n_keys)])
            for n in range(k + 1):
                mask = np.zeros(n_keys, bool)
                mask[:L + 1] = True                                   # cache and root
                mask[L + n] = True                                    # itself
                s = a["sm_scale"] * (K @ oatt.bf16_to_f64(a["q"][b, n, h]))
                s[~mask] = -np.inf
                w = np.exp(s - s.max())
                want = (w / w.sum()) @ Vv
                np.testing.assert_allclose(t[b, n, h], want, rtol=0, atol=1e-12)


def _first_grid_point(pred):
    lo, hi = 0, GRID
    while lo < hi:
        mid = (lo + hi) // 2
        if pred(mid):
            hi = mid
        else:
            lo = mid + 1
    return lo


def test_multi_candidate_step_over_the_uniform_grid():
    rng = np.random.default_rng(3)
    V = 6
    p = orej.softmax_t(rng.standard_normal(V) * 1.5, 1.0)
    q = orej.softmax_t(rng.standard_normal(V) * 1.5, 1.0)
    # residuals after rejecting candidates, written out independently of the walk
    r1 = np.maximum(0.0, p - q); r1 /= math.fsum(r1)
    r2 = np.maximum(0.0, r1 - q); r2 /= math.fsum(r2)
    # every candidate can be rejected (ratio < 1); candidate 3 still has residual mass
    x1 = int(np.argmin(p / q))
    x2 = int(np.argmin(r1 / q))
    ok3 = np.where((r2 > 0) & (r2 / q < 1), r2 / q, -1.0)
    x3 = int(np.argmax(ok3))
    tokens = [x1, x2, x3]
    assert p[x1] / q[x1] < 1 and r1[x2] / q[x2] < 1 and 0 < r2[x3] < q[x3]
    r3 = np.maximum(0.0, r2 - q); r3 /= math.fsum(r3)
    parents = [0, 0, 0]                                              # three candidates at the root
    leaf = orej.softmax_t(np.zeros(V), 1.0)
    p_of = lambda v: p if v == 0 else leaf
    q_of = lambda v: q
    REJ = 1.0 - 2.0 ** -24                                           # rejects unless the ratio is >= 1
    for i, r in ((1, p), (2, r1), (3, r2)):
        x = tokens[i - 1]
        want = min(GRID, math.ceil(r[x] / q[x] * GRID))

        def rejects(m, i=i):      # candidate i is node i
            def uni(P, stream):
                return (m / GRID if stream == (0 if i == 1 else i) else REJ, 0.0)
            return otree.walk(p_of, q_of, tokens, parents, 10, uni).nodes[:1] != [i]
        assert _first_grid_point(rejects) == want, (i, want)
    # all three rejected: the final draw over the grid of u_smp has the widths of r3
    C = np.cumsum(r3)

    def draw(m):
        return otree.walk(p_of, q_of, tokens, parents, 10, lambda P, s: (REJ, m / GRID)).tokens[0]
    edges = [_first_grid_point(lambda m, y=y: draw(m) > y) for y in range(V)]
    widths = np.diff([0] + edges)
    want = np.diff(np.concatenate([[0], np.minimum([math.ceil(C[y] / C[-1] * GRID) for y in range(V)], GRID)]))
    np.testing.assert_array_equal(widths, want)
    assert np.all(widths[r3 == 0] == 0)


def _tree_round(A, Bm, last, rng, t=2, depth=2):
    """A draft tree of branching t and the given depth, children drawn i.i.d. from the draft
    chain Bm at their parent's token; returns parents, tokens, target rows, draft rows."""
    parents, toks, node_tok = [], [], [last]
    frontier = [0]
    for _ in range(depth):
        nxt = []
        for v in frontier:
            for _ in range(t):
                tok = int(draft_from_logits(rng, Bm[node_tok[v]][None], 1.0)[0])
                parents.append(v)
                toks.append(tok)
                node_tok.append(tok)
                nxt.append(len(node_tok) - 1)
        frontier = nxt
    tl = np.array([A[x] for x in node_tok], np.float32)
    dl = np.array([Bm[x] for x in node_tok], np.float32)
    return np.array(parents, np.int32), np.array(toks, np.int32), tl, dl


def test_monte_carlo_lossless_tree_rounds_with_commit():
    rng = np.random.default_rng(12)
    V, n_tok, n = 3, 3, 20_000
    A = (rng.standard_normal((V, V)) * 1.2).astype(np.float32)
    Bm = (A + rng.standard_normal((V, V)) * 1.0).astype(np.float32)
    P = np.array([orej.softmax_t(A[i], 1.0) for i in range(V)])
    x0 = 2
    counts = np.zeros((V,) * n_tok)
    used = set()
    for s in range(n):
        seq, L = [x0], 10
        while len(seq) - 1 < n_tok:
            par, toks, tl, dl = _tree_round(A, Bm, seq[-1], rng)
            out = otree.verify_batch_tree(tl[None], dl[None], toks[None], par[None], np.array([s]), np.array([L]),
                                          1.0, 4321)
            a = int(out["num_accepted"][0])
            if s < 100:
                for j in range(a + 1):
                    assert (s, L + 1 + j) not in used
                    used.add((s, L + 1 + j))
            seq.extend(int(x) for x in out["out_tokens"][0, :a + 1])
            L = int(ocommit.commit_lengths([L], [a], 10**9)[0][0])
        counts[tuple(seq[1:n_tok + 1])] += 1
    want = np.zeros_like(counts)
    for idx in np.ndindex(*counts.shape):
        pr, prev = 1.0, x0
        for tkn in idx:
            pr *= P[prev, tkn]
            prev = tkn
        want[idx] = pr
    assert stats.chisquare(counts.ravel(), n * want.ravel()).pvalue > 1e-4


def _tree_commit_case(seed: int, N: int = 9):
    p = PRESETS["tiny"]
    a = make_tree_attention_inputs(p, N, seed=seed)
    rng = np.random.Generator(np.random.PCG64(8100 + seed))
    parents = np.stack([random_parents(rng, N) for _ in range(p.B)])
    nodes, depth = random_paths(rng, parents, stop=0.2)
    return p, a, parents, nodes, depth


def test_tree_commit_then_causal_attention_equals_the_tree_mask():
    for seed in range(3):
        p, a, parents, nodes, depth = _tree_commit_case(seed)
        L = a["seq_lens"]
        cap = a["max_blocks"] * p.block_size
        kc, vc, newL, over = otree.commit_tree(a["k_cache"], a["v_cache"], a["block_table"], L, nodes, depth, cap)
        assert not over.any()
        np.testing.assert_array_equal(newL, L + depth + 1)
        tree = otree.verify_attention_tree(a["q"], a["k_cache"], a["v_cache"], a["block_table"], L, parents,
                                           p.Hq, p.Hkv, p.block_size, a["sm_scale"])
        G = p.Hq // p.Hkv
        for b in range(p.B):
            path = [0] + [int(x) for x in nodes[b, :depth[b]]]
            for g in range(p.Hkv):
                K, Vv = oatt.gather_sequence_kv(kc, vc, a["block_table"], b, g, int(L[b]) + len(path),
                                                p.block_size)
                for j, n in enumerate(path):
                    vis = int(L[b]) + j + 1          # causal: keys 0 .. L + j
                    for h in range(g * G, (g + 1) * G):
                        got = oatt.attend(oatt.bf16_to_f64(a["q"][b, n, h]), K[:vis], Vv[:vis], a["sm_scale"])
                        np.testing.assert_array_equal(got, tree[b, n, h])


def test_tree_commit_chain_path_moves_nothing():
    p = PRESETS["tiny"]
    N = 6
    a = make_tree_attention_inputs(p, N, seed=1)
    depth = np.array([0, 2, 6, 4], dtype=np.int32)[: p.B]
    nodes = np.full((p.B, N), -1, dtype=np.int32)
    for b in range(p.B):
        nodes[b, :depth[b]] = np.arange(1, depth[b] + 1)
    kc, vc, newL, over = otree.commit_tree(a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], nodes, depth,
                                           10 ** 6)
    np.testing.assert_array_equal(kc, a["k_cache"])
    np.testing.assert_array_equal(vc, a["v_cache"])
    np.testing.assert_array_equal(newL, a["seq_lens"] + depth + 1)


def test_tree_commit_touches_only_the_new_prefix_and_refuses_overflow():
    p, a, parents, nodes, depth = _tree_commit_case(5)
    L = a["seq_lens"].astype(np.int64)
    cap = int(L[1] + depth[1])                  # sequence 1 would pass the capacity by one token
    kc, vc, newL, over = otree.commit_tree(a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], nodes, depth,
                                           cap)
    bs = p.block_size
    allowed = set()
    for b in range(p.B):
        if over[b]:
            assert newL[b] == L[b]
            continue
        for j in range(1, int(depth[b]) + 1):
            allowed.add((int(a["block_table"][b, (L[b] + j) // bs]), int((L[b] + j) % bs)))
    assert over[1] == 1
    changed_k = {(int(pg), int(o)) for pg, _, o in zip(*np.nonzero((kc != a["k_cache"]).any(axis=3)))}
    changed_v = {(int(pg), int(o)) for pg, _, o in zip(*np.nonzero((vc != a["v_cache"]).any(axis=2)))}
    assert changed_k <= allowed and changed_v <= allowed
    # every moved slot holds the old row of its node
    for b in range(p.B):
        if over[b]:
            continue
        for j in range(1, int(depth[b]) + 1):
            sp, so = int(a["block_table"][b, (L[b] + nodes[b, j - 1]) // bs]), int((L[b] + nodes[b, j - 1]) % bs)
            dp, do = int(a["block_table"][b, (L[b] + j) // bs]), int((L[b] + j) % bs)
            np.testing.assert_array_equal(kc[dp, :, do, :], a["k_cache"][sp, :, so, :])
            np.testing.assert_array_equal(vc[dp, :, :, do], a["v_cache"][sp, :, :, so])


def test_rows_cache_changes_nothing():
    # the optional per-sequence row cache only memoises the softmax rows: every output over many
    # seeds equals the uncached call's
    from workloads import make_tree_reject_inputs
    inp = make_tree_reject_inputs(PRESETS["tiny"], np.array([0, 0, 1, 1, 2], dtype=np.int32), seed=5, B=5)
    args = (inp["target_logits"], inp["draft_logits"], inp["draft_tokens"], inp["parents"], inp["seq_ids"],
            inp["seq_lens"], 1.0)
    rows = [{} for _ in range(inp["target_logits"].shape[0])]
    for seed in range(30):
        plain = otree.verify_batch_tree(*args, seed)
        cached = otree.verify_batch_tree(*args, seed, rows_cache=rows)
        for key in ("out_tokens", "num_accepted", "accepted_nodes", "out_probs", "accept_probs"):
            np.testing.assert_array_equal(plain[key], cached[key], err_msg=key)
    assert all(r["p"] for r in rows)
