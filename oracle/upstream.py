"""The verify pass's upstream steps: RoPE and KV append of the new rows, and the LM head (fp64 oracle).

Test infrastructure: only tests/, the smoke check and the benchmark's CPU
baseline use this module; the GPU path shares no code with it.

What the pages fix: "Accelerating RL Post-Training Rollouts via System-Integrated
Speculative Decoding" (gist.science summary), section 2: the target checks all k
drafts in a single forward pass, whose output distribution the rejection sampler
reads; "ReSpec" (talk notes), Adaptive Server: the KV cache is extended in place.
The pages name no position encoding and no output head; the readings taken are
the plainest ones for the decoder models they train (Qwen, Llama-style):

R1  RoPE.  Rotary position embedding in its rotate-half form: for j in
    [0, D/2), the pair (x_j, x_{j+D/2}) is rotated by the angle
    pos * theta^(-2j/D), theta given by the caller (500000 for the 8B shape,
    1000000 for the Qwen shapes). Applied to every query head and every KV head
    of the new rows; V is not rotated. Outputs are rounded once to bfloat16
    (nearest, ties to even) from the exact rotation.
R2  Positions and slots.  Row i of sequence b (the last committed token and the
    k drafts) has position L_b + i and its K, V go to cache slot L_b + i. For a
    tree, node n has position L_b + depth(n) and slot L_b + n (the tree layout of
    the tree readings).
R3  LM head.  logits[r][v] = sum_h hidden[r][h] * W[v][h] for the bf16 hidden
    states of the verify rows (after the model's final norm, which is not part of
    this step) and the bf16 output weight W [V][H]; no bias, no soft-cap; fp32
    logits, which the sampler reads as they are (temperature is the sampler's).
"""

from __future__ import annotations

import numpy as np

from .attention import bf16_to_f64


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 values to bfloat16 bit patterns: nearest, ties to even (finite inputs).

    Works on the float64 bit pattern directly, so there is no intermediate float32 rounding."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    for i, v in enumerate(flat_in):
        flat_out[i] = _round_one(float(v))
    return out


def _round_one(v: float) -> int:
    if v == 0.0:
        return 0x8000 if np.signbit(v) else 0
    sign = 0x8000 if v < 0 else 0
    m, e = np.frexp(abs(v))            # |v| = m * 2^e, m in [0.5, 1)
    e = int(e)
    # bfloat16 normal numbers: 1.f (7 fraction bits) * 2^(E-127), E in [1, 254]
    exp_unbiased = e - 1               # |v| = (2m) * 2^(e-1), 2m in [1, 2)
    if exp_unbiased < -126:            # subnormal range: fixed quantum 2^-133
        q = abs(v) / 2.0 ** -133
    else:
        q = (2.0 * m) * 128.0          # significand scaled to 8 bits: [128, 256)
    n = int(np.floor(q))
    frac = q - n
    if frac > 0.5 or (frac == 0.5 and (n & 1)):
        n += 1
    if exp_unbiased < -126:
        if n >= 128:                   # rounded up into the smallest normal
            return sign | (1 << 7) | (n - 128)
        return sign | n
    if n == 256:                       # carried into the next binade
        n = 128
        exp_unbiased += 1
    E = exp_unbiased + 127
    if E >= 255:
        return sign | 0x7F80           # overflow to infinity
    return sign | (E << 7) | (n - 128)


def rope_exact(x, pos, theta: float) -> np.ndarray:
    """R1 in float64, unrounded: x [..., D] (float64), pos broadcastable to x.shape[:-1]."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    j = np.arange(half, dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * j / D)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def row_positions(seq_lens, k: int, parents=None) -> tuple:
    """R2: (positions [B][k+1], slots [B][k+1]) of the new rows; parents [B][k] for a tree."""
    L = np.asarray(seq_lens, dtype=np.int64)
    B = L.shape[0]
    i = np.arange(k + 1, dtype=np.int64)
    slots = L[:, None] + i[None, :]
    if parents is None:
        return slots.copy(), slots
    depth = np.zeros((B, k + 1), dtype=np.int64)
    for b in range(B):
        for n in range(1, k + 1):
            depth[b, n] = depth[b, int(parents[b][n - 1])] + 1
    return L[:, None] + depth, slots


def rope_append(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, theta: float, parents=None):
    """R1 + R2 on the new rows: q [B][k+1][Hq][D], k_new / v_new [B][k+1][Hkv][D] (bf16 bits).

    Returns (q rotated, k_cache', v_cache'), all bf16 bits; the caches are copies with the new
    rows written at their slots (K rotated, V as given)."""
    B, K1, Hq, D = q.shape
    pos, slots = row_positions(seq_lens, K1 - 1, parents)
    q_rot = f64_to_bf16(rope_exact(bf16_to_f64(q), pos[:, :, None], theta))
    k_rot = f64_to_bf16(rope_exact(bf16_to_f64(k_new), pos[:, :, None], theta))
    kc, vc = k_cache.copy(), v_cache.copy()
    bs = k_cache.shape[2]
    for b in range(B):
        for i in range(K1):
            s = int(slots[b, i])
            page, off = int(block_table[b, s // bs]), s % bs
            kc[page, :, off, :] = k_rot[b, i]
            vc[page, :, :, off] = v_new[b, i]
    return q_rot, kc, vc


def lm_head(hidden, weight) -> np.ndarray:
    """R3 in float64: hidden [R][H], weight [V][H] (bf16 bits) -> logits [R][V] float64."""
    return bf16_to_f64(hidden) @ bf16_to_f64(weight).T


def lm_head_error_bound(hidden, weight) -> np.ndarray:
    """Bound on |fp32-accumulated sum - exact sum| for each logit: the products of two bfloat16
    values are exact in fp32, and a sum of H terms in any order with fp32 additions is within
    gamma_H * sum |terms|, gamma_H = H u / (1 - H u), u = 2^-24 (Higham, Accuracy and Stability
    of Numerical Algorithms, 2nd ed., section 4.2); one more u for rounding the result."""
    H = hidden.shape[-1]
    u = 2.0 ** -24
    gamma = H * u / (1.0 - H * u)
    mag = np.abs(bf16_to_f64(hidden)) @ np.abs(bf16_to_f64(weight)).T
    return gamma * mag + u * mag


def lm_head_stat_bound(hidden, weight, lam: float = 9.0, chunk: int = 64) -> np.ndarray:
    """A probabilistic bound on the fp32 accumulation error of each logit, far tighter than
    the worst case above.

    Model: the device sums the H exact products t_k = hidden[r][k] W[v][k] with fp32
    additions in some order, in blocks of at most `chunk` consecutive k (in any order inside
    a block) whose running total may start at any block. Each addition a rounds its exact
    result p_a by a factor (1 + d_a), |d_a| <= u = 2^-24, the d_a independent with mean zero
    (round to nearest on data without structure). The error is then sum_a p_a d_a, and
    Hoeffding's inequality gives |error| <= lam u sqrt(sum_a p_a^2) with probability at least
    1 - 2 exp(-lam^2 / 2) (the approach of Higham and Mary, "A new approach to probabilistic
    rounding error analysis", SIAM J. Sci. Comput. 41 (2019), applied with the partial sums
    themselves instead of sum |t_k|). Every partial result is a difference of two prefix sums
    S_i = t_0 + .. + t_{i-1} (wrapping past H adds S_H), plus at most one block's worth of
    terms, so |p_a| <= P = 2 max_i |S_i| + |S_H| + max over blocks of sum |t_k|; there are at
    most H additions, hence the bound lam u sqrt(H) P, plus u |S_H| for good measure.
    lam = 9: a false alarm has probability below 1e-17 per logit."""
    h = bf16_to_f64(hidden)
    w = bf16_to_f64(weight)
    R, H = h.shape
    if H % chunk:
        raise ValueError("H must be a multiple of the block length")
    u = 2.0 ** -24
    out = np.empty((R, w.shape[0]))
    for r in range(R):
        t = w * h[r]                                    # [V][H] exact products
        S = np.cumsum(t, axis=1)
        total = S[:, -1]
        block = np.abs(t).reshape(t.shape[0], H // chunk, chunk).sum(axis=2).max(axis=1)
        P = 2.0 * np.max(np.abs(S), axis=1) + np.abs(total) + block
        out[r] = lam * u * np.sqrt(H) * P + u * np.abs(total)
    return out
