"""Cache-length commit after a verify step (oracle side).

Follows: "Accelerating RL Post-Training Rollouts via System-Integrated
Speculative Decoding" (gist.science explainer): accepted drafts plus the
verifier's own token are adopted together (up to k+1 per step), and the
accepted length is the per-step progress measure; "ReSpec: Towards Optimizing
Speculative Decoding in Reinforcement Learning Systems" (talk notes), section
"Adaptive Server": speculation extends the KV cache in place.

Reading: before the step the cache holds L committed tokens and the k+1 verify
rows at L .. L+k. After accepting a drafts, x_last and the a accepted drafts
have valid KV, and the newly emitted token becomes the next x_last, so
L' = L + a + 1. A commit that would pass ``capacity_tokens`` is refused for
that sequence (length unchanged, overflow flag set).
"""

from __future__ import annotations

import numpy as np


def commit_lengths(seq_lens, num_accepted, capacity_tokens: int):
    """Returns (new_lengths int32 [B], overflow_flags int32 [B])."""
    L = np.asarray(seq_lens, dtype=np.int64)
    a = np.asarray(num_accepted, dtype=np.int64)
    proposed = L + a + 1
    overflow = proposed > capacity_tokens
    new = np.where(overflow, L, proposed)
    return new.astype(np.int32), overflow.astype(np.int32)
