"""GPU parity of the ragged-draft-length entry points against the fp64 oracle.

spec_verify_attn_ragged and spec_reject_sample_ragged take per-sequence draft
counts k_b (rows packed by offsets). Checked element by element on small shapes
(mixed k_b from 0 to 15, one and two 16-row tiles, one and two row groups, NaN
in every cache slot past L_b + k_b), on sampled rows at the 8B shape, decision
by decision for the sampler at 8B and tiny sizes, against the uniform entry
points when every k_b is equal, and over steps with the commit.
"""

import dataclasses

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import commit as ocommit
from oracle import reject as orej
from tests.parity import ATTN_TOL, MARGIN, MISMATCH_BUDGET, PROB_TOL, Tally, bf16_dev, dev, run_attention, say, seed_count
from workloads import PRESETS, make_ragged_attention_inputs, make_ragged_reject_inputs, make_reject_inputs
from workloads import pack_reject_inputs

pytestmark = pytest.mark.gpu


def _run_attn_ragged(a, device):
    import torch
    import speculative_decoding_verification_14_amd as sv
    q = bf16_dev(a["q"], device)
    out = torch.empty_like(q)
    sv.verify_attn_ragged(q, bf16_dev(a["k_cache"], device), bf16_dev(a["v_cache"], device),
                          dev(a["block_table"], device), dev(a["seq_lens"], device), dev(a["cu_drafts"], device),
                          out, a["k"], a["max_seq_len"], a["sm_scale"])
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _oracle_attn(a):
    return oatt.verify_attention_ragged(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"],
                                        a["cu_drafts"], a["Hq"], a["Hkv"], a["block_size"], a["sm_scale"])


def _preset(**kw):
    return dataclasses.replace(PRESETS["tiny"], **kw)


@pytest.mark.parametrize("D,Hq,Hkv,k_max,bs", [
    (128, 32, 8, 3, 16),     # 8B heads: 4..16 rows, one tile
    (128, 32, 8, 7, 16),     # up to 32 rows: two tiles
    (64, 16, 2, 15, 32),     # up to 128 rows: four row groups
    (128, 28, 4, 5, 64),     # G = 7
])
def test_attention_ragged_small(device, D, Hq, Hkv, k_max, bs):
    p = _preset(D=D, Hq=Hq, Hkv=Hkv, block_size=bs, B=9, ctx=("uniform", 1, 900))
    a = make_ragged_attention_inputs(p, k_max, seed=D + Hq + k_max)
    got = _run_attn_ragged(a, device)
    want = _oracle_attn(a)
    err = np.abs(got - want).max()
    say(f"[ragged attn] D{D} Hq{Hq} Hkv{Hkv} k_max{k_max} lens {a['draft_lens'].tolist()}: max err {err:.2e}")
    assert np.all(np.isfinite(got)) and err <= ATTN_TOL


def test_attention_ragged_equal_lengths_matches_uniform(device):
    p = _preset(D=128, Hq=32, Hkv=8, block_size=16, B=7, ctx=("uniform", 100, 3000))
    a = make_ragged_attention_inputs(p, 3, draft_lens=np.full(7, 3))
    got = _run_attn_ragged(a, device)
    u = dict(a)
    u["q"] = a["q"].reshape(7, 4, a["Hq"], a["D"])
    uni = run_attention(u, device)
    np.testing.assert_array_equal(got, uni.reshape(got.shape))


def test_attention_ragged_8b_every_row(device):
    """8B shape (B = 64, contexts 1K-8K) with k_b in 0..7, every packed row against the oracle."""
    a = make_ragged_attention_inputs(PRESETS["8b"], 7)
    got = _run_attn_ragged(a, device)
    want = oatt.verify_attention_ragged(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"],
                                        a["cu_drafts"], a["Hq"], a["Hkv"], a["block_size"], a["sm_scale"])
    err = float(np.abs(got - want).max())
    say(f"[ragged attn] 8b: all {got.shape[0] * got.shape[1]} rows, max err {err:.2e}")
    assert np.all(np.isfinite(got)) and err <= ATTN_TOL


class RaggedRejectDevice:
    def __init__(self, inp, device):
        import torch
        self.inp = inp
        self.t = dev(inp["target_logits"], device)
        self.d = dev(inp["draft_logits"], device) if inp["draft_logits"].shape[0] else None
        self.dt = dev(inp["draft_tokens"], device) if inp["draft_tokens"].shape[0] else None
        self.cu = dev(inp["cu_drafts"], device)
        self.sid = dev(inp["seq_ids"], device)
        self.sl = dev(inp["seq_lens"], device)
        T, K, B = self.t.shape[0], int(inp["cu_drafts"][-1]), inp["B"]
        self.max_k = int(np.max(np.diff(inp["cu_drafts"]))) if B else 0
        self.out_tokens = torch.empty(T, dtype=torch.int32, device=device)
        self.out_probs = torch.empty(T, dtype=torch.float32, device=device)
        self.acc_probs = torch.empty(K, dtype=torch.float32, device=device)
        self.num_acc = torch.empty(B, dtype=torch.int32, device=device)

    def call(self, seed):
        import torch
        import speculative_decoding_verification_14_amd as sv
        self.out_tokens.fill_(-7)
        self.out_probs.fill_(-7.0)
        self.acc_probs.fill_(-7.0)
        self.num_acc.fill_(-7)
        sv.reject_sample_ragged(self.t, self.d, self.dt, self.cu, self.sid, self.sl, self.max_k,
                                self.inp["temperature"], seed, self.out_tokens, self.num_acc, self.out_probs,
                                self.acc_probs)
        torch.cuda.synchronize()
        return dict(out_tokens=self.out_tokens.cpu().numpy(), num_accepted=self.num_acc.cpu().numpy(),
                    out_probs=self.out_probs.cpu().numpy().astype(np.float64),
                    accept_probs=self.acc_probs.cpu().numpy().astype(np.float64))


def _compare_ragged(g, o, cu, tally):
    """Decision by decision per sequence (mismatches allowed only below the margin), then
    the packed outputs of every sequence without a mismatch."""
    B = len(cu) - 1
    for b, res in enumerate(o["results"]):
        kb, t0, d0 = int(cu[b + 1] - cu[b]), int(cu[b] + b), int(cu[b])
        a_g = int(g["num_accepted"][b])
        toks = g["out_tokens"][t0:t0 + kb + 1]
        bad = False
        for d in res.decisions:
            tally.decisions += 1
            same = ((a_g > d.j) == bool(d.outcome)) if d.kind == "accept" else (
                a_g == d.j and int(toks[d.j]) == d.outcome)
            if not same:
                tally.mismatches += 1
                tally.mismatch_margins.append(d.margin)
                if not (d.margin < MARGIN):
                    tally.bad.append((b, d.kind, d.j, d.margin))
                bad = True
                break
        if bad:
            continue
        n = res.num_accepted + 1
        if not np.array_equal(toks[:n], res.tokens) or np.any(toks[n:] != -1):
            tally.bad.append((b, "tokens", -1, 0.0))
            continue
        op = g["out_probs"][t0:t0 + kb + 1]
        tally.prob_err = max(tally.prob_err, float(np.abs(op[:n] - res.out_probs).max()))
        if np.any(op[n:] != 0.0):
            tally.bad.append((b, "out_probs_pad", -1, 0.0))
        ap = g["accept_probs"][d0:d0 + kb]
        nt = len(res.accept_probs)
        if nt:
            tally.prob_err = max(tally.prob_err, float(np.abs(ap[:nt] - res.accept_probs).max()))
        if np.any(ap[nt:] != -1.0):
            tally.bad.append((b, "accept_probs_pad", -1, 0.0))
    assert B == len(o["results"])


def _check_ragged(inp, device, seeds, label):
    rd = RaggedRejectDevice(inp, device)
    cu = inp["cu_drafts"]
    rows = [orej.SequenceRows(inp["target_logits"][cu[b] + b: cu[b + 1] + b + 1],
                              inp["draft_logits"][cu[b]: cu[b + 1]], inp["temperature"]) for b in range(inp["B"])]
    tally = Tally()
    for n, s in enumerate(seeds, 1):
        g = rd.call(s)
        o = orej.verify_batch_ragged(inp["target_logits"], inp["draft_logits"], inp["draft_tokens"], cu,
                                     inp["seq_ids"], inp["seq_lens"], inp["temperature"], s, rows_cache=rows)
        _compare_ragged(g, o, cu, tally)
        if n % 500 == 0:
            say(f"[ragged reject] {label}: {n} of {len(seeds)} seeds")
    say(f"[ragged reject] {label} lens {np.diff(cu).tolist()[:16]}: {tally.summary()}")
    tally.record(f"ragged reject {label}")
    assert not tally.bad, tally.bad[:10]
    assert tally.mismatches <= MISMATCH_BUDGET * max(1, tally.decisions) and tally.prob_err <= PROB_TOL
    return tally


def test_reject_ragged_8b(device):
    inp = make_ragged_reject_inputs(PRESETS["8b"], 7)
    _check_ragged(inp, device, [inp["seed"] + 13 * i for i in range(seed_count(120))], "8b k_max 7")


def test_reject_ragged_tiny_k15(device):
    inp = make_ragged_reject_inputs(PRESETS["tiny"], 15, B=16)
    _check_ragged(inp, device, [inp["seed"] + i for i in range(200)], "tiny k_max 15")


def test_reject_ragged_all_zero_lengths(device):
    inp = make_ragged_reject_inputs(PRESETS["tiny"], 3, B=8, draft_lens=np.zeros(8, np.int32))
    _check_ragged(inp, device, [inp["seed"] + i for i in range(50)], "tiny all k_b = 0")


def test_reject_ragged_equal_lengths_matches_uniform(device):
    from tests.parity import RejectDevice
    base = make_reject_inputs(PRESETS["8b"], B=32)
    k = base["k"]
    rag = RaggedRejectDevice(pack_reject_inputs(base, np.full(32, k)), device)
    uni = RejectDevice(base, device)
    for s in (1, 2, 3):
        g, u = rag.call(s), uni.call(s)
        np.testing.assert_array_equal(g["out_tokens"], u["out_tokens"].ravel())
        np.testing.assert_array_equal(g["num_accepted"], u["num_accepted"])
        np.testing.assert_array_equal(g["out_probs"], u["out_probs"].ravel().astype(np.float64))
        np.testing.assert_array_equal(g["accept_probs"], u["accept_probs"].ravel().astype(np.float64))


def test_reject_ragged_level_parallel_matches_full_batch(device):
    """Four ragged sequences of the 8B rows run every level at once (the groups past a
    sequence's k_b only count themselves); the same sequences inside a batch of 64 run
    the chain. Their packed outputs are bit-identical."""
    base = make_reject_inputs(PRESETS["8b"], B=64)
    lens = np.random.default_rng(17).integers(0, base["k"] + 1, size=64).astype(np.int32)
    lens[:4] = [3, 0, 2, 1]
    full = RaggedRejectDevice(pack_reject_inputs(base, lens), device)
    small = dict(base)
    for key in ("target_logits", "draft_logits", "draft_tokens", "seq_ids", "seq_lens"):
        small[key] = np.ascontiguousarray(base[key][:4])
    small["B"] = 4
    part = RaggedRejectDevice(pack_reject_inputs(small, lens[:4]), device)
    rows, drafts = int(np.sum(lens[:4] + 1)), int(np.sum(lens[:4]))
    for seed in (2, 29, 311):
        g, c = full.call(seed), part.call(seed)
        np.testing.assert_array_equal(c["num_accepted"], g["num_accepted"][:4])
        np.testing.assert_array_equal(c["out_tokens"], g["out_tokens"][:rows])
        np.testing.assert_array_equal(c["out_probs"], g["out_probs"][:rows])
        np.testing.assert_array_equal(c["accept_probs"], g["accept_probs"][:drafts])


def test_reject_ragged_steps_with_commit(device):
    import torch
    import speculative_decoding_verification_14_amd as sv
    inp = make_ragged_reject_inputs(PRESETS["tiny"], 6, B=8)
    rd = RaggedRejectDevice(inp, device)
    cu = inp["cu_drafts"]
    L = inp["seq_lens"].copy()
    tally = Tally()
    for step in range(3):
        rd.sl.copy_(torch.from_numpy(L))
        g = rd.call(21)
        o = orej.verify_batch_ragged(inp["target_logits"], inp["draft_logits"], inp["draft_tokens"], cu,
                                     inp["seq_ids"], L, 1.0, 21)
        _compare_ragged(g, o, cu, tally)
        sv.commit_lengths(rd.sl, rd.num_acc, rd.max_k, 10**6)
        torch.cuda.synchronize()
        L, _ = ocommit.commit_lengths(L, o["num_accepted"], 10**6)
        np.testing.assert_array_equal(rd.sl.cpu().numpy(), L)
    tally.record("test_gpu_ragged::test_reject_ragged_steps_with_commit")
    assert not tally.bad and tally.mismatches <= MISMATCH_BUDGET * tally.decisions, tally.summary()
