"""GPU parity of tree verification against the fp64 oracle.

spec_verify_attn_tree (the tree mask) element by element on full binary trees,
random trees, stars and chain-shaped trees (the last also bit-equal to the
causal spec_verify_attn); spec_reject_sample_tree decision by decision (each
candidate test and the final draw, mismatches only below the margin) on tiny and
8B-sized rows, random and full trees, and over steps with the commit;
spec_commit_tree bit-exact on the whole caches (random paths, a = 0, a = -1,
refused commits, every page size and both head sizes, the 8B shape), and composed
with the attention calls: causal attention over the moved cache reproduces the
tree-masked rows of the accepted path.
"""

import numpy as np
import pytest

from oracle import commit as ocommit
from oracle import tree as otree
from tests.parity import ATTN_TOL, MARGIN, MISMATCH_BUDGET, PROB_TOL, Tally, bf16_dev, dev, run_attention, say, seed_count
from workloads import (PRESETS, make_tree_attention_inputs, make_tree_reject_inputs, random_parents, random_paths,
                       tree_parents)

pytestmark = pytest.mark.gpu


def _tree_attn(a, parents, device):
    import torch
    import speculative_decoding_verification_14_amd as sv
    q = bf16_dev(a["q"], device)
    out = torch.empty_like(q)
    sv.verify_attn_tree(q, bf16_dev(a["k_cache"], device), bf16_dev(a["v_cache"], device),
                        dev(a["block_table"], device), dev(a["seq_lens"], device), dev(parents, device), out,
                        a["max_seq_len"], a["sm_scale"])
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _shapes():
    rng = np.random.default_rng(1)
    return [("binary d3", tree_parents(2, 3)), ("ternary d2", tree_parents(3, 2)),
            ("random 15", random_parents(rng, 15)), ("random 9", random_parents(rng, 9)),
            ("star 4", np.zeros(4, np.int32)), ("chain 5", np.arange(5, dtype=np.int32))]


@pytest.mark.parametrize("label,par", _shapes())
@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (64, 8, 2)])
def test_tree_attention(device, label, par, D, Hq, Hkv):
    import dataclasses
    N = len(par)
    p = dataclasses.replace(PRESETS["tiny"], D=D, Hq=Hq, Hkv=Hkv, B=5, ctx=("uniform", 1, 700))
    a = make_tree_attention_inputs(p, N, seed=N + D)
    parents = np.broadcast_to(par, (5, N)).copy()
    got = _tree_attn(a, parents, device)
    want = otree.verify_attention_tree(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], parents,
                                       Hq, Hkv, a["block_size"], a["sm_scale"])
    err = np.abs(got - want).max()
    say(f"[tree attn] {label} D{D} Hq{Hq}: max err {err:.2e}")
    assert np.all(np.isfinite(got)) and err <= ATTN_TOL
    if label.startswith("chain"):
        np.testing.assert_array_equal(got, run_attention(a, device))


@pytest.mark.parametrize("t,d", [(2, 2), (2, 3)])
def test_tree_attention_8b_every_row(device, t, d):
    """The bench's tree shapes at the 8B size (two- and four-tile row groups, contexts 1K-8K), every
    node row of every sequence against the oracle."""
    par = tree_parents(t, d)
    N = len(par)
    p = PRESETS["8b"]
    a = make_tree_attention_inputs(p, N, seed=40 + N)
    parents = np.broadcast_to(par, (p.B, N)).copy()
    got = _tree_attn(a, parents, device)
    want = otree.verify_attention_tree(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], parents,
                                       p.Hq, p.Hkv, a["block_size"], a["sm_scale"])
    err = float(np.abs(got - want).max())
    say(f"[tree attn] 8b t{t} d{d}: all {got.shape[0] * got.shape[1] * got.shape[2]} rows, max err {err:.2e}")
    assert np.all(np.isfinite(got)) and err <= ATTN_TOL


class TreeDevice:
    def __init__(self, inp, device):
        import torch
        self.inp = inp
        self.t, self.d = dev(inp["target_logits"], device), dev(inp["draft_logits"], device)
        self.dt, self.par = dev(inp["draft_tokens"], device), dev(inp["parents"], device)
        self.sid, self.sl = dev(inp["seq_ids"], device), dev(inp["seq_lens"], device)
        B, N = inp["draft_tokens"].shape
        self.out_tokens = torch.empty((B, N + 1), dtype=torch.int32, device=device)
        self.out_probs = torch.empty((B, N + 1), dtype=torch.float32, device=device)
        self.nodes = torch.empty((B, N), dtype=torch.int32, device=device)
        self.acc = torch.empty((B, N), dtype=torch.float32, device=device)
        self.num_acc = torch.empty(B, dtype=torch.int32, device=device)

    def call(self, seed):
        import torch
        import speculative_decoding_verification_14_amd as sv
        for t, v in ((self.out_tokens, -7), (self.out_probs, -7.0), (self.nodes, -7), (self.acc, -7.0),
                     (self.num_acc, -7)):
            t.fill_(v)
        sv.reject_sample_tree(self.t, self.d, self.dt, self.par, self.sid, self.sl, self.inp["temperature"], seed,
                              self.out_tokens, self.num_acc, self.nodes, self.out_probs, self.acc)
        torch.cuda.synchronize()
        return dict(out_tokens=self.out_tokens.cpu().numpy(), num_accepted=self.num_acc.cpu().numpy(),
                    accepted_nodes=self.nodes.cpu().numpy(),
                    out_probs=self.out_probs.cpu().numpy().astype(np.float64),
                    accept_probs=self.acc.cpu().numpy().astype(np.float64))


def _compare_tree(g, o, tally):
    for b, res in enumerate(o["results"]):
        a_g = int(g["num_accepted"][b])
        nodes_g = g["accepted_nodes"][b]
        toks_g = g["out_tokens"][b]
        bad = False
        for d, node in zip(res.decisions, res.decision_nodes):
            tally.decisions += 1
            if d.kind == "accept":
                got_acc = a_g > d.j and int(nodes_g[d.j]) == node
                same = got_acc == bool(d.outcome)
            else:
                same = a_g == d.j and int(toks_g[d.j]) == d.outcome
            if not same:
                tally.mismatches += 1
                tally.mismatch_margins.append(d.margin)
                if not (d.margin < MARGIN):
                    tally.bad.append((b, d.kind, d.j, node, d.margin))
                bad = True
                break
        if bad:
            continue
        n = res.num_accepted + 1
        if (not np.array_equal(toks_g[:n], res.tokens) or np.any(toks_g[n:] != -1)
                or not np.array_equal(nodes_g[:n - 1], res.nodes) or np.any(nodes_g[n - 1:] != -1)):
            tally.bad.append((b, "outputs", -1, -1, 0.0))
            continue
        tally.prob_err = max(tally.prob_err, float(np.abs(g["out_probs"][b, :n] - res.out_probs).max()))
        if np.any(g["out_probs"][b, n:] != 0.0):
            tally.bad.append((b, "out_probs_pad", -1, -1, 0.0))
        want_acc = np.full(len(nodes_g), -1.0)
        for node, ap in res.accept_probs.items():
            want_acc[node - 1] = ap
        tested = want_acc >= 0
        if np.any(g["accept_probs"][b, ~tested] != -1.0):
            tally.bad.append((b, "accept_probs_pad", -1, -1, 0.0))
        if tested.any():
            tally.prob_err = max(tally.prob_err, float(np.abs(g["accept_probs"][b, tested] - want_acc[tested]).max()))


def _check_tree(inp, device, seeds, label):
    td = TreeDevice(inp, device)
    tally = Tally()
    rows = [{} for _ in range(inp["B"])]   # each sequence's softmax rows, computed once for all seeds
    for i, s in enumerate(seeds):
        g = td.call(s)
        o = otree.verify_batch_tree(inp["target_logits"], inp["draft_logits"], inp["draft_tokens"], inp["parents"],
                                    inp["seq_ids"], inp["seq_lens"], inp["temperature"], s, rows_cache=rows)
        _compare_tree(g, o, tally)
        if (i + 1) % 25 == 0:
            say(f"[tree reject] {label}: {i + 1} of {len(seeds)} seeds")
    say(f"[tree reject] {label}: {tally.summary()}")
    tally.record(f"tree walk {label}")
    assert not tally.bad, tally.bad[:10]
    assert tally.mismatches <= MISMATCH_BUDGET * max(1, tally.decisions) and tally.prob_err <= PROB_TOL
    return tally


@pytest.mark.parametrize("label,par", _shapes())
def test_tree_reject_tiny(device, label, par):
    inp = make_tree_reject_inputs(PRESETS["tiny"], par, B=8)
    _check_tree(inp, device, [inp["seed"] + i for i in range(60)], f"tiny {label}")


def test_tree_reject_random_trees_per_sequence(device):
    rng = np.random.default_rng(9)
    par = np.stack([random_parents(rng, 12) for _ in range(16)])
    inp = make_tree_reject_inputs(PRESETS["tiny"], par, B=16)
    _check_tree(inp, device, [inp["seed"] + 3 * i for i in range(60)], "tiny random per sequence")


@pytest.mark.parametrize("t,d", [(2, 2), (2, 3), (4, 1)])
def test_tree_reject_8b(device, t, d):
    inp = make_tree_reject_inputs(PRESETS["8b"], tree_parents(t, d), B=64)
    _check_tree(inp, device, [inp["seed"] + 11 * i for i in range(seed_count(20))], f"8b t{t} d{d}")


@pytest.mark.parametrize("t,d", [(2, 2), (4, 1)])
def test_tree_reject_batch_invariant_across_workgroup_sizes(device, t, d):
    """The full batch of 64 runs eight-wavefront workgroups, its first 4 and first 16
    sequences four-wavefront ones (each workgroup on a CU of its own): the walk's exchanges
    go through quads of units, so those sequences' outputs are bit-identical."""
    inp = make_tree_reject_inputs(PRESETS["8b"], tree_parents(t, d), B=64)
    full = TreeDevice(inp, device)
    for n in (4, 16):
        small = dict(inp)
        for key in ("target_logits", "draft_logits", "draft_tokens", "parents", "seq_ids", "seq_lens"):
            small[key] = np.ascontiguousarray(inp[key][:n])
        part = TreeDevice(small, device)
        for seed in (5, 77, 9001):
            a, c = full.call(seed), part.call(seed)
            for key in a:
                np.testing.assert_array_equal(c[key], a[key][:n])


def test_tree_steps_with_commit(device):
    import torch
    import speculative_decoding_verification_14_amd as sv
    inp = make_tree_reject_inputs(PRESETS["tiny"], tree_parents(2, 2), B=6)
    td = TreeDevice(inp, device)
    L = inp["seq_lens"].copy()
    tally = Tally()
    for step in range(3):
        td.sl.copy_(torch.from_numpy(L))
        g = td.call(8)
        o = otree.verify_batch_tree(inp["target_logits"], inp["draft_logits"], inp["draft_tokens"], inp["parents"],
                                    inp["seq_ids"], L, 1.0, 8)
        _compare_tree(g, o, tally)
        sv.commit_lengths(td.sl, td.num_acc, 15, 10**6)
        torch.cuda.synchronize()
        L, _ = ocommit.commit_lengths(L, o["num_accepted"], 10**6)
        np.testing.assert_array_equal(td.sl.cpu().numpy(), L)
    tally.record("test_gpu_tree::test_tree_steps_with_commit")
    assert not tally.bad and tally.mismatches <= MISMATCH_BUDGET * tally.decisions, tally.summary()


def _commit_tree_case(p, N: int, seed: int, B: int):
    a = make_tree_attention_inputs(p, N, seed=seed, B=B)
    rng = np.random.Generator(np.random.PCG64(8200 + seed))
    parents = np.stack([random_parents(rng, N) for _ in range(B)])
    nodes, depth = random_paths(rng, parents, stop=0.2)
    return a, parents, nodes, depth


def _gpu_commit_tree(a, nodes, depth, cap, device):
    import torch
    import speculative_decoding_verification_14_amd as sv
    kc, vc = bf16_dev(a["k_cache"], device), bf16_dev(a["v_cache"], device)
    sl = dev(a["seq_lens"], device)
    over = torch.full((len(depth),), 7, dtype=torch.int32, device=device)
    sv.commit_tree(kc, vc, dev(a["block_table"], device), sl, dev(nodes, device), dev(depth, device), cap, over)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    return bits(kc), bits(vc), sl.cpu().numpy(), over.cpu().numpy()


def _check_commit_tree(a, nodes, depth, cap, device, label):
    gk, gv, gl, go = _gpu_commit_tree(a, nodes, depth, cap, device)
    wk, wv, wl, wo = otree.commit_tree(a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], nodes, depth, cap)
    moved = int(sum(d for d, o in zip(depth, wo) if d > 0 and not o))
    say(f"[tree commit] {label}: cap {cap}, {int(wo.sum())} refused, {moved} rows moved")
    np.testing.assert_array_equal(gl, wl)
    np.testing.assert_array_equal(go, wo)
    np.testing.assert_array_equal(gk, wk)
    np.testing.assert_array_equal(gv, wv)


@pytest.mark.parametrize("N,D,bs", [(1, 64, 16), (6, 64, 32), (15, 64, 16), (9, 128, 64), (15, 128, 16)])
def test_tree_commit_bit_exact(device, N, D, bs):
    import dataclasses
    p = dataclasses.replace(PRESETS["tiny"], D=D, Hq=8, Hkv=4, block_size=bs, ctx=("uniform", 0, 300))
    a, parents, nodes, depth = _commit_tree_case(p, N, seed=N + D + bs, B=12)
    depth[0], nodes[0] = 0, -1                     # nothing accepted
    depth[1], nodes[1] = -1, -1                    # the walk's error value
    L = a["seq_lens"].astype(np.int64)
    _check_commit_tree(a, nodes, depth, a["max_blocks"] * bs, device, f"N{N} D{D} bs{bs}")
    b = int(np.argmax(depth))
    cap = int(L[b] + depth[b])                     # sequence b (and any longer) would pass it
    _check_commit_tree(a, nodes, depth, cap, device, f"N{N} D{D} bs{bs} refused")


def test_tree_commit_8b_shape(device):
    p = PRESETS["8b"]
    a, parents, nodes, depth = _commit_tree_case(p, 14, seed=3, B=p.B)
    _check_commit_tree(a, nodes, depth, a["max_blocks"] * p.block_size, device, "8b N14")


def test_tree_commit_then_causal_attention_is_the_tree_rows(device):
    """Tree attention before the move (GPU), causal attention of the path after it (GPU, the ragged
    call with k_b = a_b), and the oracle's tree rows agree on every node of the accepted path."""
    import dataclasses
    import torch
    import speculative_decoding_verification_14_amd as sv
    N = 12
    p = dataclasses.replace(PRESETS["tiny"], D=128, Hq=16, Hkv=4, ctx=("uniform", 1, 900))
    a, parents, nodes, depth = _commit_tree_case(p, N, seed=21, B=10)
    B = len(depth)
    tree_gpu = _tree_attn(a, parents, device)
    want = otree.verify_attention_tree(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], parents,
                                       p.Hq, p.Hkv, a["block_size"], a["sm_scale"])
    gk, gv, gl, go = _gpu_commit_tree(a, nodes, depth, a["max_blocks"] * p.block_size, device)
    assert not go.any()
    paths = [[0] + [int(x) for x in nodes[b, :depth[b]]] for b in range(B)]
    cu = np.concatenate([[0], np.cumsum(depth)]).astype(np.int32)
    q_rows = np.concatenate([a["q"][b, path] for b, path in enumerate(paths)])        # [R][Hq][D]
    q = bf16_dev(q_rows, device)
    out = torch.empty_like(q)
    sv.verify_attn_ragged(q, bf16_dev(gk, device), bf16_dev(gv, device), dev(a["block_table"], device),
                          dev(a["seq_lens"], device), dev(cu, device), out, N, a["max_seq_len"], a["sm_scale"])
    torch.cuda.synchronize()
    causal = out.float().cpu().numpy().astype(np.float64)
    r = 0
    worst = 0.0
    for b, path in enumerate(paths):
        for n in path:
            worst = max(worst, np.abs(causal[r] - want[b, n]).max(), np.abs(tree_gpu[b, n] - want[b, n]).max())
            r += 1
    say(f"[tree commit + attention] {r} path rows, max err {worst:.2e}")
    assert worst <= ATTN_TOL


def test_tree_reject_broken_trees_then_a_valid_call(device):
    """A node with five children and a parent index out of range end their sequences with -1 (the
    failure comes before any exchange); the valid trees in the same call match the oracle, and a
    following call on the same workspace with other logits still matches it (the failing call stored
    its epoch, so no slot of it is taken for one of the next call)."""
    good = [random_parents(np.random.default_rng(5), 6), np.arange(6, dtype=np.int32)]
    wide = np.array([0, 0, 0, 0, 0, 1], dtype=np.int32)
    out_of_range = np.array([0, 5, 1, 2, 3, 4], dtype=np.int32)
    parents = np.stack([good[0], wide, out_of_range, good[1]])
    inp = make_tree_reject_inputs(PRESETS["tiny"], parents, B=4)     # one workgroup per sequence
    g = TreeDevice(inp, device).call(inp["seed"])
    np.testing.assert_array_equal(g["num_accepted"][[1, 2]], [-1, -1])
    sub = {k: inp[k][[0, 3]] for k in ("target_logits", "draft_logits", "draft_tokens", "parents", "seq_ids",
                                       "seq_lens")}
    o = otree.verify_batch_tree(sub["target_logits"], sub["draft_logits"], sub["draft_tokens"], sub["parents"],
                                sub["seq_ids"], sub["seq_lens"], inp["temperature"], inp["seed"])
    tally = Tally()
    _compare_tree({k: v[[0, 3]] for k, v in g.items()}, o, tally)
    inp2 = make_tree_reject_inputs(PRESETS["tiny"], np.stack([good[0], good[1], good[0], good[1]]), seed=77, B=4)
    g2 = TreeDevice(inp2, device).call(inp2["seed"] + 1)
    o2 = otree.verify_batch_tree(inp2["target_logits"], inp2["draft_logits"], inp2["draft_tokens"], inp2["parents"],
                                 inp2["seq_ids"], inp2["seq_lens"], inp2["temperature"], inp2["seed"] + 1)
    _compare_tree(g2, o2, tally)
    say(f"[tree reject] broken trees, then a valid call: {tally.summary()}")
    tally.record("test_gpu_tree::test_tree_reject_broken_trees_then_a_valid_call")
    assert not tally.bad and tally.mismatches == 0, tally.summary()
