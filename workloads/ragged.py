"""Ragged draft lengths: per-sequence k_b in one batch, rows packed by offsets.

The draft length of each sequence is drawn uniformly from 0 .. k_max (the pages
give no distribution; EfficientRollout's abstract only says the draft length
adapts to acceptance). Inputs are the uniform-k inputs at k = k_max, sliced and
packed: sequence b's rows sit at cu[b] + b + i (query, target logits, outputs)
and cu[b] + j (draft logits, draft tokens, acceptance outputs). Like the rest of
this package it only draws numbers and lays them out.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from .gen import BF16_NAN, Preset, make_attention_inputs, make_reject_inputs


def ragged_draft_lengths(B: int, k_max: int, seed: int) -> np.ndarray:
    """k_b ~ U{0 .. k_max}, int32 [B]."""
    rng = np.random.Generator(np.random.PCG64(5000 + seed))
    return rng.integers(0, k_max + 1, size=B).astype(np.int32)


def offsets(draft_lens: np.ndarray) -> np.ndarray:
    """cu [B+1]: cu[0] = 0, cu[b+1] - cu[b] = k_b."""
    cu = np.zeros(len(draft_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(draft_lens, dtype=np.int64))
    return cu


def make_ragged_attention_inputs(preset: Preset, k_max: int, seed: int | None = None, B: int | None = None,
                                 draft_lens: np.ndarray | None = None) -> dict:
    """Attention inputs with packed query rows q [R][Hq][D], R = cu[B] + B.

    The cache is laid out for L_b + k_max + 1 keys; the slots of keys past
    L_b + k_b are filled with bf16 NaN, so any read of them shows in the output.
    """
    s = preset.index if seed is None else seed
    a = make_attention_inputs(dataclasses.replace(preset, k=k_max), seed=s, B=B, garbage="nan")
    B = a["B"]
    kb = ragged_draft_lengths(B, k_max, s) if draft_lens is None else np.asarray(draft_lens, dtype=np.int32)
    cu = offsets(kb)
    q = np.concatenate([a["q"][b, : kb[b] + 1] for b in range(B)], axis=0)
    kc, vc, bt, bs = a["k_cache"], a["v_cache"], a["block_table"], a["block_size"]
    for b in range(B):
        L = int(a["seq_lens"][b])
        for t in range(L + int(kb[b]) + 1, L + k_max + 1):
            page = bt[b, t // bs]
            kc[page, :, t % bs, :] = BF16_NAN
            vc[page, :, :, t % bs] = BF16_NAN
    out = dict(a)
    out.update(q=np.ascontiguousarray(q), cu_drafts=cu, draft_lens=kb, k=k_max)
    return out


def pack_reject_inputs(inp: dict, draft_lens: np.ndarray) -> dict:
    """Packs uniform-k reject inputs ([B][k+1][V], [B][k][V], [B][k]) to the ragged layout."""
    kb = np.asarray(draft_lens, dtype=np.int32)
    B = inp["B"]
    cu = offsets(kb)
    V = inp["V"]
    target = np.concatenate([inp["target_logits"][b, : kb[b] + 1] for b in range(B)], axis=0)
    drafts = [inp["draft_logits"][b, : kb[b]] for b in range(B)]
    draft = np.concatenate(drafts, axis=0) if cu[B] > 0 else np.zeros((0, V), np.float32)
    toks = [inp["draft_tokens"][b, : kb[b]] for b in range(B)]
    tokens = np.concatenate(toks).astype(np.int32) if cu[B] > 0 else np.zeros(0, np.int32)
    out = dict(inp)
    out.update(target_logits=np.ascontiguousarray(target), draft_logits=np.ascontiguousarray(draft),
               draft_tokens=np.ascontiguousarray(tokens), cu_drafts=cu, draft_lens=kb)
    return out


def make_ragged_reject_inputs(preset: Preset, k_max: int, seed: int | None = None, B: int | None = None,
                              draft_lens: np.ndarray | None = None) -> dict:
    """Reject inputs in the ragged layout, from the uniform inputs at k = k_max."""
    s = preset.index if seed is None else seed
    inp = make_reject_inputs(dataclasses.replace(preset, k=k_max), seed=s, B=B)
    kb = ragged_draft_lengths(inp["B"], k_max, s) if draft_lens is None else draft_lens
    return pack_reject_inputs(inp, kb)
