"""Pins for the oracle's ragged-draft-length layout (CPU only).

The ragged functions add only row packing on top of the uniform-k oracle, which
is pinned by its own tests (dense brute force, library attention, exhaustive
uniform grids, Monte Carlo). What is new is the offset arithmetic, so each
ragged result is checked, sequence by sequence, against the uniform oracle run
on that sequence alone with its own k_b, and a batch whose draft lengths are
all equal against the uniform batch call.
"""

import dataclasses

import numpy as np

from oracle import attention as oatt
from oracle import reject as orej
from workloads import PRESETS, make_ragged_attention_inputs, make_ragged_reject_inputs, make_reject_inputs
from workloads import pack_reject_inputs


def test_ragged_reject_equals_each_sequence_alone():
    inp = make_ragged_reject_inputs(PRESETS["tiny"], 7, B=9, draft_lens=np.array([0, 7, 3, 1, 0, 5, 2, 7, 4]))
    cu = inp["cu_drafts"]
    for seed in (3, 17, 29):
        r = orej.verify_batch_ragged(inp["target_logits"], inp["draft_logits"], inp["draft_tokens"], cu,
                                     inp["seq_ids"], inp["seq_lens"], 1.0, seed)
        assert r["out_tokens"].shape == (cu[-1] + 9,) and r["accept_probs"].shape == (cu[-1],)
        for b in range(9):
            kb, t0, d0 = cu[b + 1] - cu[b], cu[b] + b, cu[b]
            one = orej.verify_batch(inp["target_logits"][None, t0:t0 + kb + 1],
                                    inp["draft_logits"][None, d0:d0 + kb], inp["draft_tokens"][None, d0:d0 + kb],
                                    inp["seq_ids"][b:b + 1], inp["seq_lens"][b:b + 1], kb, 1.0, seed)
            np.testing.assert_array_equal(r["out_tokens"][t0:t0 + kb + 1], one["out_tokens"][0])
            np.testing.assert_array_equal(r["out_probs"][t0:t0 + kb + 1], one["out_probs"][0])
            np.testing.assert_array_equal(r["accept_probs"][d0:d0 + kb], one["accept_probs"][0])
            assert r["num_accepted"][b] == one["num_accepted"][0] <= kb


def test_ragged_reject_with_equal_lengths_is_the_uniform_call():
    base = make_reject_inputs(PRESETS["tiny"], B=6)
    k = base["k"]
    inp = pack_reject_inputs(base, np.full(6, k))
    r = orej.verify_batch_ragged(inp["target_logits"], inp["draft_logits"], inp["draft_tokens"], inp["cu_drafts"],
                                 inp["seq_ids"], inp["seq_lens"], 1.0, 5)
    u = orej.verify_batch(base["target_logits"], base["draft_logits"], base["draft_tokens"], base["seq_ids"],
                          base["seq_lens"], k, 1.0, 5)
    np.testing.assert_array_equal(r["out_tokens"], u["out_tokens"].ravel())
    np.testing.assert_array_equal(r["accept_probs"], u["accept_probs"].ravel())
    np.testing.assert_array_equal(r["num_accepted"], u["num_accepted"])


def test_ragged_attention_equals_each_sequence_alone():
    p = dataclasses.replace(PRESETS["tiny"], B=5)
    a = make_ragged_attention_inputs(p, 4, draft_lens=np.array([4, 0, 2, 1, 3]))
    cu = a["cu_drafts"]
    out = oatt.verify_attention_ragged(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], cu,
                                       a["Hq"], a["Hkv"], a["block_size"], a["sm_scale"])
    assert np.all(np.isfinite(out))         # the NaN-filled slots past L_b + k_b were never read
    for b in range(5):
        kb, r0 = cu[b + 1] - cu[b], cu[b] + b
        one = oatt.verify_attention(a["q"][None, r0:r0 + kb + 1], a["k_cache"], a["v_cache"],
                                    a["block_table"][b:b + 1], a["seq_lens"][b:b + 1], kb, a["Hq"], a["Hkv"],
                                    a["block_size"], a["sm_scale"])
        np.testing.assert_array_equal(out[r0:r0 + kb + 1], one[0])
