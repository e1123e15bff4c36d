"""Paged-KV verify attention, written out as its definition (fp64).

Follows: "Accelerating RL Post-Training Rollouts via System-Integrated
Speculative Decoding" (gist.science technical summary), section 2 "Method",
core mechanism: the target (verifier) checks all k drafted tokens in a single
forward pass. For one attention layer that pass is: each sequence b has a
committed cache of L_b tokens plus the k+1 verify tokens [x_last, d_1 .. d_k]
at positions L_b .. L_b+k, whose keys and values the caller has already
appended; query row i (0 <= i <= k) attends to keys 0 .. L_b+i (causal inside
the draft). Query head h reads KV head h // (Hq / Hkv). Scores are scaled by
sm_scale (1/sqrt(D) by default); no soft-cap, bias, window or sink.

Memory layouts read here (the same bytes the GPU reads):
* q        bf16 [B][k+1][Hq][D]
* k_cache  bf16 [num_blocks][Hkv][block_size][D]
* v_cache  bf16 [num_blocks][Hkv][D][block_size]
* block_table int32 [B][max_blocks]: logical page -> physical page

Ragged draft lengths (per-sequence k_b, "EfficientRollout: System-Aware
Self-Speculative Decoding for RL Rollouts", abstract: acceptance-aware draft
length) change only which rows exist: sequence b contributes rows i = 0 .. k_b,
packed at row cu[b] + b + i of q [R][Hq][D], and reads L_b + k_b + 1 keys.
"""

from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def gather_sequence_kv(k_cache, v_cache, block_table, b: int, g: int, n_keys: int, block_size: int):
    """Keys and values 0..n_keys-1 of sequence b, KV head g, walking the block table page by page."""
    D = k_cache.shape[-1]
    K = np.empty((n_keys, D), dtype=np.float64)
    Vv = np.empty((n_keys, D), dtype=np.float64)
    for t0 in range(0, n_keys, block_size):
        page = int(block_table[b, t0 // block_size])
        n = min(block_size, n_keys - t0)
        K[t0:t0 + n] = bf16_to_f64(k_cache[page, g, :n, :])
        Vv[t0:t0 + n] = bf16_to_f64(v_cache[page, g, :, :n]).T
    return K, Vv


def attend(qrow: np.ndarray, K: np.ndarray, Vv: np.ndarray, sm_scale: float) -> np.ndarray:
    """softmax(sm_scale * K q) weighted sum of V rows; K and V hold exactly the visible keys."""
    s = sm_scale * (K @ qrow)
    w = np.exp(s - s.max())
    w /= w.sum()
    return w @ Vv


def verify_attention(q, k_cache, v_cache, block_table, seq_lens, k: int, Hq: int, Hkv: int,
                     block_size: int, sm_scale: float, pairs=None) -> np.ndarray:
    """fp64 output [B][k+1][Hq][D]; ``pairs`` restricts the work to a list of (b, kv_head).

    Rows not covered by ``pairs`` are left as NaN.
    """
    B = q.shape[0]
    D = q.shape[-1]
    G = Hq // Hkv
    out = np.full((B, k + 1, Hq, D), np.nan, dtype=np.float64)
    todo = pairs if pairs is not None else [(b, g) for b in range(B) for g in range(Hkv)]
    for b, g in todo:
        L = int(seq_lens[b])
        K, Vv = gather_sequence_kv(k_cache, v_cache, block_table, b, g, L + k + 1, block_size)
        for i in range(k + 1):
            visible = L + i + 1
            for h in range(g * G, (g + 1) * G):
                qrow = bf16_to_f64(q[b, i, h, :])
                out[b, i, h, :] = attend(qrow, K[:visible], Vv[:visible], sm_scale)
    assert out.shape[-1] == D
    return out


def verify_attention_row(q, k_cache, v_cache, block_table, seq_lens, k: int, Hq: int, Hkv: int,
                         block_size: int, sm_scale: float, b: int, i: int, h: int) -> np.ndarray:
    """One output row (b, draft index i, query head h) - for spot checks at full size."""
    G = Hq // Hkv
    g = h // G
    L = int(seq_lens[b])
    K, Vv = gather_sequence_kv(k_cache, v_cache, block_table, b, g, L + i + 1, block_size)
    return attend(bf16_to_f64(q[b, i, h, :]), K, Vv, sm_scale)


def verify_attention_ragged(q, k_cache, v_cache, block_table, seq_lens, cu_drafts, Hq: int, Hkv: int,
                            block_size: int, sm_scale: float) -> np.ndarray:
    """fp64 output [R][Hq][D] for packed rows: sequence b has k_b = cu[b+1] - cu[b] drafts and
    its query row i (0 <= i <= k_b) is row cu[b] + b + i; row i attends keys 0 .. L_b + i."""
    B = len(seq_lens)
    R, _, D = q.shape
    G = Hq // Hkv
    out = np.full((R, Hq, D), np.nan, dtype=np.float64)
    for b in range(B):
        kb = int(cu_drafts[b + 1]) - int(cu_drafts[b])
        r0 = int(cu_drafts[b]) + b
        L = int(seq_lens[b])
        for g in range(Hkv):
            K, Vv = gather_sequence_kv(k_cache, v_cache, block_table, b, g, L + kb + 1, block_size)
            for i in range(kb + 1):
                visible = L + i + 1
                for h in range(g * G, (g + 1) * G):
                    out[r0 + i, h, :] = attend(bf16_to_f64(q[r0 + i, h, :]), K[:visible], Vv[:visible], sm_scale)
    return out
