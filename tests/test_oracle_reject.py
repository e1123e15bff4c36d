"""Pins for the oracle's acceptance chain, residual / bonus sampling and commit (CPU only).

Each pin is fixed by the pages or by mathematics, not by the oracle itself:
* softmax: sums to one (exactly rounded sum), shift invariance, temperature.
* q = p accepts every draft; k = 3 then adopts four tokens in one step (worked
  example in the explainer of "Accelerating RL Post-Training Rollouts via
  System-Integrated Speculative Decoding"; fixture tests/golden/pages_facts.json).
* one-hot special cases, q(x) = 0 handling.
* exhaustive 2^24 uniform grid: accept counts equal the grid points below p/q,
  and every token's sample count equals its interval width (inverse CDF).
* acceptance frequency equals the closed form beta = sum_x min(p(x), q(x)).
* Monte-Carlo lossless guarantee (one round): each emitted token ~ p_j.
* Monte-Carlo lossless guarantee across rounds with commit, on a Markov
  target/draft pair: the joint law of the first tokens equals the target chain.
* expected emitted length equals sum_j prod_{i<j} beta_i.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy import stats

from oracle import commit as ocommit
from oracle import philox
from oracle import reject as orej
from workloads import draft_from_logits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(V, k, rng, sigma=1.0, noise=0.7):
    target = (rng.standard_normal((k + 1, V)) * sigma).astype(np.float32)
    draft = (target[:k] + rng.standard_normal((k, V)) * noise).astype(np.float32)
    return target, draft


# ----------------------------------------------------------------------------- softmax

def test_softmax_sums_to_one_and_is_shift_invariant():
    rng = np.random.default_rng(0)
    for V in (3, 1000, 128256):
        z = (rng.standard_normal(V) * 3).astype(np.float32)
        p = orej.softmax_t(z, 1.0)
        assert abs(math.fsum(p) - 1.0) < 1e-15
        np.testing.assert_allclose(orej.softmax_t(z.astype(np.float64) + 5.0, 1.0), p, rtol=1e-12, atol=1e-300)
        # temperature T on z equals T = 1 on z / T (T a power of two keeps z / T exact)
        np.testing.assert_allclose(orej.softmax_t(z, 2.0), orej.softmax_t(z / np.float32(2.0), 1.0),
                                   rtol=1e-13, atol=0)
    # two-token closed form: p(0) = 1 / (1 + e^(z1 - z0))
    p = orej.softmax_t(np.array([0.5, -1.25], np.float32), 1.0)
    assert abs(p[0] - 1.0 / (1.0 + math.exp(-1.75))) < 1e-16


# ----------------------------------------------------------------------------- special cases

def test_q_equals_p_accepts_everything_and_k3_adopts_four_tokens():
    facts = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))
    k = facts["full_acceptance"]["k"]
    want_tokens = facts["full_acceptance"]["tokens_adopted"]
    rng = np.random.default_rng(1)
    for V in (7, 1000):
        target, _ = _rows(V, k, rng)
        draft = target[:k].copy()
        dt = draft_from_logits(rng, draft, 1.0)
        for seed in range(200):
            res = orej.verify_batch(target[None], draft[None], dt[None], np.array([seed * 3 + 1]),
                                    np.array([100 + seed]), k, 1.0, seed)
            assert res["num_accepted"][0] == k
            assert np.count_nonzero(res["out_tokens"][0] >= 0) == want_tokens
            np.testing.assert_array_equal(res["out_tokens"][0, :k], dt)
            new_len, ovf = ocommit.commit_lengths(np.array([100 + seed]), res["num_accepted"], 10**6)
            assert new_len[0] == 100 + seed + want_tokens and ovf[0] == 0


def test_one_hot_target_always_accepts_its_token():
    V, k = 11, 3
    rng = np.random.default_rng(2)
    target, draft = _rows(V, k, rng)
    dt = np.array([4, 9, 0], np.int32)
    for j in range(k):
        target[j] = -np.inf
        target[j, dt[j]] = 0.0
    for seed in range(100):
        res = orej.verify_batch(target[None], draft[None], dt[None], np.array([5]), np.array([seed]),
                                k, 1.0, seed)
        assert res["num_accepted"][0] == k
        np.testing.assert_array_equal(res["accept_probs"][0], 1.0)


def test_one_hot_draft_on_impossible_token_rejects_and_residual_is_p():
    V, k = 9, 2
    rng = np.random.default_rng(3)
    target, draft = _rows(V, k, rng)
    x = 6
    target[0, x] = -np.inf          # p_0(x) = 0
    draft[0] = -np.inf
    draft[0, x] = 0.0               # q_0 one-hot on x
    dt = np.array([x, 1], np.int32)
    rows = orej.SequenceRows(target, draft, 1.0)
    np.testing.assert_array_equal(rows.residual(0), rows.p(0))
    counts = np.zeros(V)
    n = 4000
    for s in range(n):
        res = orej.verify_batch(target[None], draft[None], dt[None], np.array([s]), np.array([0]), k, 1.0, 77)
        assert res["num_accepted"][0] == 0 and res["accept_probs"][0, 0] == 0.0
        counts[res["out_tokens"][0, 0]] += 1
    assert counts[x] == 0
    p = rows.p(0)
    assert stats.chisquare(counts[p > 0], n * p[p > 0]).pvalue > 1e-4


def test_zero_draft_probability_with_positive_target_is_accepted():
    V, k = 5, 1
    target = np.zeros((2, V), np.float32)
    draft = np.full((1, V), -np.inf, np.float32)
    draft[0, 2] = 0.0               # q_0 one-hot on token 2
    dt = np.array([3], np.int32)    # q_0(3) = 0 while p_0(3) = 1/5
    for s in range(50):
        res = orej.verify_batch(target[None], draft[None], dt[None], np.array([s]), np.array([9]), k, 1.0, s)
        assert res["num_accepted"][0] == 1 and res["accept_probs"][0, 0] == 1.0


# ----------------------------------------------------------------------------- exhaustive uniform grid

GRID = 1 << 24


def _first_grid_point(pred):
    """Smallest m in [0, 2^24] with pred(m) True, for a predicate monotone in m (bisection)."""
    lo, hi = 0, GRID
    while lo < hi:
        mid = (lo + hi) // 2
        if pred(mid):
            hi = mid
        else:
            lo = mid + 1
    return lo


def test_exhaustive_grid_acceptance_and_inverse_cdf():
    """Over all 2^24 values of u the oracle's outcomes partition the grid in exactly the
    proportions the weights prescribe (monotonicity in u lets bisection count each cell)."""
    rng = np.random.default_rng(4)
    V, k = 6, 1
    target, draft = _rows(V, k, rng, sigma=1.5, noise=1.0)
    rows = orej.SequenceRows(target, draft, 1.0)
    p0, q0 = rows.p(0), rows.q(0)
    for x in range(V):
        ratio = p0[x] / q0[x]

        def rejects(m, x=x):
            r = orej.decide(rows, [x], k, [(m / GRID, 0.0), (0.0, 0.0)])
            return r.num_accepted == 0

        n_accept = _first_grid_point(rejects)
        assert n_accept == min(GRID, math.ceil(ratio * GRID)), (x, n_accept, ratio)

    # residual sampling after a reject: counts per token = interval widths on the grid
    for weights in (rows.residual(0), rows.p(1)):
        C = np.cumsum(weights)
        edges = [_first_grid_point(lambda m, y=y: orej.inverse_cdf(weights, m / GRID)[0] > y)
                 for y in range(V)]
        counts = np.diff([0] + edges)
        want = np.array([math.ceil(C[y] / C[-1] * GRID) for y in range(V)])
        want = np.diff(np.concatenate([[0], np.minimum(want, GRID)]))
        np.testing.assert_array_equal(counts, want)
        assert np.all(counts[weights == 0] == 0)
        # spot check monotonicity on random grid points
        ms = np.sort(rng.integers(0, GRID, 2000))
        ys = [orej.inverse_cdf(weights, m / GRID)[0] for m in ms]
        assert all(a <= b for a, b in zip(ys, ys[1:]))


def test_plain_decoding_k0_is_inverse_cdf_of_p0_over_the_whole_grid():
    """k = 0 tests no draft: the step emits one token, the inverse CDF of p_0 at u_smp
    (word 1 of the uniforms at P = L+1, never u_acc). Over all 2^24 grid values of u_smp
    each token's count is its interval width ceil(C(y) 2^24) - ceil(C(y-1) 2^24), and
    u_acc changes nothing."""
    rng = np.random.default_rng(11)
    V = 7
    target = (rng.standard_normal((1, V)) * 1.5).astype(np.float32)
    rows = orej.SequenceRows(target, np.zeros((0, V), np.float32), 1.0)
    p0 = np.exp(target[0].astype(np.float64) - target[0].max())
    p0 /= math.fsum(p0)
    C = np.cumsum(p0)
    edges = [_first_grid_point(lambda m, y=y: orej.decide(rows, [], 0, [(0.5, m / GRID)]).tokens[0] > y)
             for y in range(V)]
    counts = np.diff([0] + edges)
    want = np.diff(np.concatenate([[0], np.minimum([math.ceil(C[y] / C[-1] * GRID) for y in range(V)], GRID)]))
    np.testing.assert_array_equal(counts, want)
    for u_acc in (0.0, 0.3, 1.0 - 2.0 ** -24):
        for m in rng.integers(0, GRID, 50):
            r0 = orej.decide(rows, [], 0, [(0.5, m / GRID)])
            r1 = orej.decide(rows, [], 0, [(u_acc, m / GRID)])
            assert r1.tokens == r0.tokens and r1.num_accepted == 0 and len(r1.tokens) == 1
            assert [d.kind for d in r1.decisions] == ["sample"] and r1.accept_probs == []
    # batch form: positions L+1, outputs [B][1], no acceptance outputs; commit adds one
    B = 5
    tl = (rng.standard_normal((B, 1, 40)) * 2).astype(np.float32)
    sid = np.arange(B, dtype=np.int64) * 31 + 7
    L = rng.integers(0, 1000, B).astype(np.int32)
    out = orej.verify_batch(tl, np.zeros((B, 0, 40), np.float32), np.zeros((B, 0), np.int32), sid, L, 0, 1.0, 77)
    assert out["out_tokens"].shape == (B, 1) and out["accept_probs"].shape == (B, 0)
    assert np.all(out["num_accepted"] == 0)
    for b in range(B):
        u_acc, u_smp = philox.verify_uniforms(77, int(sid[b]), int(L[b]) + 1)
        pb = orej.softmax_t(tl[b, 0], 1.0)
        assert out["out_tokens"][b, 0] == orej.inverse_cdf(pb, u_smp)[0]
    np.testing.assert_array_equal(ocommit.commit_lengths(L, out["num_accepted"], 10**6)[0], L + 1)


def test_exact_boundary_hits_are_strict():
    """Dyadic weights make u * R land exactly on a CDF edge: the rule is C(y) > u * R (strict),
    zero-weight tokens are never emitted, and acceptance is u < p/q (strict)."""
    w = np.array([0.0, 0.0, 0.25, 0.0, 0.75, 0.0])
    assert orej.inverse_cdf(w, 0.0)[0] == 2
    assert orej.inverse_cdf(w, 0.25)[0] == 4          # t == C(2) exactly -> next positive token
    assert orej.inverse_cdf(w, 0.25 - 2**-24)[0] == 2
    assert orej.inverse_cdf(w, 1.0 - 2**-24)[0] == 4
    assert orej.inverse_cdf(w, 0.25)[1] == 0.0        # exact edge hit has zero margin
    rows = orej.SequenceRows(np.zeros((2, 2), np.float32), np.zeros((1, 2), np.float32), 1.0)
    rows._p[0] = np.array([0.5, 0.5])
    rows._q[0] = np.array([1.0, 0.0])                # p/q = 0.5 on token 0
    assert orej.decide(rows, [0], 1, [(0.5, 0.0), (0.0, 0.0)]).num_accepted == 0
    assert orej.decide(rows, [0], 1, [(0.5 - 2**-24, 0.0), (0.0, 0.0)]).num_accepted == 1


def test_acceptance_uses_temperature_on_both_distributions():
    """beta = sum min(p, q) with p, q = softmax(z / T) from scipy, at T != 1."""
    from scipy.special import softmax
    rng = np.random.default_rng(11)
    V, k, T, n = 40, 1, 0.6, 30_000
    target, draft = _rows(V, k, rng, sigma=1.0, noise=0.9)
    p = softmax(target[0].astype(np.float64) / T)
    q = softmax(draft[0].astype(np.float64) / T)
    beta = float(np.minimum(p, q).sum())
    rows = orej.SequenceRows(target, draft, T)
    drafts = np.stack([draft_from_logits(rng, draft, T) for _ in range(n)])
    ua, us = philox.verify_uniforms_np(31, np.arange(n), np.full(n, 8))
    acc = np.mean([orej.decide(rows, drafts[t], k, [(ua[t], us[t]), (0.0, 0.0)]).num_accepted == 1
                   for t in range(n)])
    assert abs(acc - beta) < 5 * math.sqrt(beta * (1 - beta) / n), (acc, beta)


# ----------------------------------------------------------------------------- Monte Carlo: one round

def _mc_round(target, draft, k, n, seed, rng):
    rows = orej.SequenceRows(target, draft, 1.0)
    drafts = np.stack([draft_from_logits(rng, draft, 1.0) for _ in range(n)])
    sids = np.arange(n, dtype=np.int64) + 1000
    Lc = 50
    ua, us = philox.verify_uniforms_np(seed, sids[:, None], Lc + 1 + np.arange(k + 1)[None, :])
    out = []
    for t in range(n):
        unis = list(zip(ua[t], us[t]))
        out.append(orej.decide(rows, drafts[t], k, unis))
    return rows, out


def test_monte_carlo_lossless_single_round():
    rng = np.random.default_rng(5)
    V, k, n = 5, 3, 60_000
    target, draft = _rows(V, k, rng, sigma=1.2, noise=1.0)
    rows, results = _mc_round(target, draft, k, n, 0x5EED, rng)
    betas = [float(np.minimum(rows.p(j), rows.q(j)).sum()) for j in range(k)]
    for j in range(k + 1):
        reached = [r for r in results if len(r.tokens) > j]
        # P(reach index j) = prod_{i<j} beta_i
        want_frac = float(np.prod(betas[:j]))
        frac = len(reached) / n
        assert abs(frac - want_frac) < 5 * math.sqrt(want_frac * (1 - want_frac) / n) + 1e-12, (j, frac, want_frac)
        # token emitted at j, given j is reached, is distributed as p_j
        counts = np.bincount([r.tokens[j] for r in reached], minlength=V)
        assert stats.chisquare(counts, len(reached) * rows.p(j)).pvalue > 1e-4, j
    # acceptance frequency at each tested position = closed form beta_j
    for j in range(k):
        tested = [r for r in results if len(r.accept_probs) > j]
        acc = np.mean([r.num_accepted > j for r in tested])
        sd = math.sqrt(betas[j] * (1 - betas[j]) / len(tested))
        assert abs(acc - betas[j]) < 5 * sd, (j, acc, betas[j])
    # expected emitted length = sum_j prod_{i<j} beta_i
    mean_len = np.mean([len(r.tokens) for r in results])
    want = sum(float(np.prod(betas[:j])) for j in range(k + 1))
    assert abs(mean_len - want) < 0.02 * want


def test_acceptance_frequency_matches_closed_form_on_wide_vocab():
    rng = np.random.default_rng(6)
    V, k, n = 2000, 1, 20_000
    target, draft = _rows(V, k, rng, sigma=2.0, noise=0.8)
    rows, results = _mc_round(target, draft, k, n, 99, rng)
    beta = float(np.minimum(rows.p(0), rows.q(0)).sum())
    acc = np.mean([r.num_accepted >= 1 for r in results])
    assert abs(acc - beta) < 5 * math.sqrt(beta * (1 - beta) / n)


# ----------------------------------------------------------------------------- Monte Carlo: rounds + commit

def _markov_rollout(A, Bm, x0, seq_id, seed, k, n_tokens, rng, log_positions=None):
    """Generate n_tokens after x0 with repeated verify rounds; drafts from the draft chain."""
    tokens = [x0]
    L = 10                                   # committed length before the first round
    V = A.shape[0]
    while len(tokens) - 1 < n_tokens:
        last = tokens[-1]
        drafts, q_logits = [], []
        ctx = last
        for _ in range(k):
            q_logits.append(Bm[ctx])
            d = int(draft_from_logits(rng, Bm[ctx][None], 1.0)[0])
            drafts.append(d)
            ctx = d
        p_logits = [A[last]] + [A[d] for d in drafts]
        rows = orej.SequenceRows(np.array(p_logits, np.float32), np.array(q_logits, np.float32).reshape(k, V), 1.0)
        unis = orej.sequence_uniforms(seed, seq_id, L, k)
        res = orej.decide(rows, drafts, k, unis)
        if log_positions is not None:   # positions whose uniforms this round consumed
            log_positions.extend((seq_id, L + 1 + j) for j in range(res.num_accepted + 1))
        tokens.extend(res.tokens)
        L = int(ocommit.commit_lengths([L], [res.num_accepted], 10**9)[0][0])
        assert V == A.shape[1]
    return tokens[1: n_tokens + 1]


@pytest.mark.parametrize("k", [2, 0])
def test_monte_carlo_lossless_across_rounds_with_commit(k):
    """k = 2 is speculative decoding; k = 0 is plain decoding (one token per round, the
    length advanced by one): both must generate the target chain's joint law."""
    rng = np.random.default_rng(7 + k)
    V, n_tok, n = 3, 4, 20_000
    A = (rng.standard_normal((V, V)) * 1.2).astype(np.float32)
    Bm = (A + rng.standard_normal((V, V)) * 1.0).astype(np.float32)
    x0 = 1
    P = np.array([orej.softmax_t(A[i], 1.0) for i in range(V)])
    counts = np.zeros((V,) * n_tok)
    positions = []
    for s in range(n):
        seq = _markov_rollout(A, Bm, x0, seq_id=s, seed=2024, k=k, n_tokens=n_tok, rng=rng,
                              log_positions=positions if s < 200 else None)
        counts[tuple(seq)] += 1
    want = np.zeros_like(counts)
    for idx in np.ndindex(*counts.shape):
        pr, prev = 1.0, x0
        for t in idx:
            pr *= P[prev, t]
            prev = t
        want[idx] = pr
    assert stats.chisquare(counts.ravel(), n * want.ravel()).pvalue > 1e-4
    # every (sequence, position) is decided exactly once over the rollout: the positions
    # consumed by successive rounds are disjoint and contiguous
    assert len(positions) == len(set(positions))
    for s in range(200):
        ps = sorted(p for (sid, p) in positions if sid == s)
        assert ps == list(range(ps[0], ps[0] + len(ps)))


def test_resume_equals_uninterrupted():
    rng = np.random.default_rng(8)
    V, k = 50, 3
    target, draft = _rows(V, k, rng)
    dt = draft_from_logits(rng, draft, 1.0)
    a = orej.verify_batch(target[None], draft[None], dt[None], np.array([42]), np.array([1234]), k, 1.0, 9)
    b = orej.verify_batch(target[None], draft[None], dt[None], np.array([42]), np.array([1234]), k, 1.0, 9)
    for key in ("out_tokens", "num_accepted", "out_probs", "accept_probs"):
        np.testing.assert_array_equal(a[key], b[key])


def test_batch_invariance():
    rng = np.random.default_rng(9)
    V, k, B = 40, 3, 6
    target = (rng.standard_normal((B, k + 1, V)) * 2).astype(np.float32)
    draft = (target[:, :k] + rng.standard_normal((B, k, V))).astype(np.float32)
    dt = draft_from_logits(rng, draft, 1.0)
    sid = np.arange(B, dtype=np.int64) * 11 + 3
    L = np.arange(B, dtype=np.int32) * 5 + 100
    full = orej.verify_batch(target, draft, dt, sid, L, k, 1.0, 5)
    perm = rng.permutation(B)[:4]
    sub = orej.verify_batch(target[perm], draft[perm], dt[perm], sid[perm], L[perm], k, 1.0, 5)
    for key in ("out_tokens", "num_accepted", "out_probs", "accept_probs"):
        np.testing.assert_array_equal(sub[key], full[key][perm])


def test_margins_recorded_for_every_decision():
    rng = np.random.default_rng(10)
    V, k = 300, 3
    target, draft = _rows(V, k, rng)
    dt = draft_from_logits(rng, draft, 1.0)
    res = orej.verify_batch(target[None], draft[None], dt[None], np.array([1]), np.array([7]), k, 1.0, 3)
    r = res["results"][0]
    n_tests = min(r.num_accepted + 1, k)
    assert sum(d.kind == "accept" for d in r.decisions) == n_tests
    assert sum(d.kind == "sample" for d in r.decisions) == 1
    assert all(d.margin >= 0 for d in r.decisions)


# ----------------------------------------------------------------------------- commit

def test_commit_adds_accepted_plus_one_and_flags_overflow():
    L = np.array([10, 20, 30, 98], np.int32)
    a = np.array([0, 3, 2, 3], np.int32)
    new, ovf = ocommit.commit_lengths(L, a, capacity_tokens=100)
    np.testing.assert_array_equal(new, [11, 24, 33, 98])
    np.testing.assert_array_equal(ovf, [0, 0, 0, 1])
    assert np.all((new - L)[ovf == 0] >= 1) and np.all((new - L)[ovf == 0] <= 4)
