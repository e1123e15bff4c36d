"""Pins for the upstream oracle (RoPE + KV append, LM head), CPU only.

* bfloat16 rounding: equal to torch's float32 -> bfloat16 conversion on values
  exact in float32 (torch rounds to nearest even), constructed halfway cases go
  to the even neighbour, bfloat16 values round-trip, subnormals and overflow.
* RoPE: position 0 is the identity; every rotated pair keeps its norm; the dot
  product of a rotated query and key depends only on the position difference;
  rotations compose additively; a hand-worked D = 4 case fixes the rotate-half
  pairing (j with j + D/2) and the frequencies theta^(-2j/D).
* Positions and slots: the chain's row i sits at L + i; a tree node's position
  follows its depth (the tree oracle's own depths).
* Append: causal attention over the appended cache equals a dense softmax over
  the original cache's keys followed by the rotated new rows, built from
  scratch; every other slot is unchanged.
* LM head: small-integer inputs give the exact brute-force sums; a one-hot
  weight picks one hidden component (orientation); a float32 product lies within
  the stated rounding bound of the float64 one.
"""

import math

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import tree as otree
from oracle import upstream as oup
from workloads import PRESETS, make_attention_inputs, random_parents


def _f32_to_bf16_torch(x32):
    import torch
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    np.testing.assert_array_equal(oup.f64_to_bf16(x.astype(np.float64)), _f32_to_bf16_torch(x))


def test_bf16_rounding_ties_and_round_trip():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even significand (1.0)
    assert oup.f64_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even): rounds up
    assert oup.f64_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82
    # just above a tie rounds up
    assert oup.f64_to_bf16(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81
    assert oup.f64_to_bf16(np.array([-2.0]))[0] == 0xC000
    assert oup.f64_to_bf16(np.array([0.0, -0.0])).tolist() == [0, 0x8000]
    assert oup.f64_to_bf16(np.array([3.0e38 * 1.2]))[0] == 0x7F80
    # subnormals: the smallest positive bfloat16 is 2^-133
    assert oup.f64_to_bf16(np.array([2.0 ** -133]))[0] == 0x0001
    assert oup.f64_to_bf16(np.array([2.0 ** -134]))[0] == 0x0000         # tie to even (zero)
    assert oup.f64_to_bf16(np.array([3 * 2.0 ** -134]))[0] == 0x0002     # tie to even (two)
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    np.testing.assert_array_equal(oup.f64_to_bf16(oatt.bf16_to_f64(bits)), bits)


def test_rope_closed_forms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 8, 64))
    np.testing.assert_array_equal(oup.rope_exact(x, np.zeros((5, 8)), 10000.0), x)
    pos = rng.integers(0, 300000, size=(5, 8))
    y = oup.rope_exact(x, pos, 500000.0)
    n_in = x[..., :32] ** 2 + x[..., 32:] ** 2
    n_out = y[..., :32] ** 2 + y[..., 32:] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-12, atol=1e-12)
    # hand-worked D = 4, theta = 10000, position 1: pair (x0, x2) turns by 1 rad,
    # pair (x1, x3) by 10000^(-1/2) = 0.01 rad
    v = np.array([1.0, 2.0, 3.0, 4.0])
    c1, s1, c2, s2 = math.cos(1.0), math.sin(1.0), math.cos(0.01), math.sin(0.01)
    want = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 3 * c1 + 1 * s1, 4 * c2 + 2 * s2]
    np.testing.assert_allclose(oup.rope_exact(v, 1, 10000.0), want, rtol=0, atol=1e-15)


def test_rope_relative_position_and_composition():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for m, n, t in [(5, 3, 1000), (70000, 69990, 12345), (0, 4000, 250000)]:
        d1 = oup.rope_exact(q, m, 1e6) @ oup.rope_exact(k, n, 1e6)
        d2 = oup.rope_exact(q, m + t, 1e6) @ oup.rope_exact(k, n + t, 1e6)
        assert abs(d1 - d2) <= 1e-9 * (1 + abs(d1)), (m, n, t, d1, d2)
        np.testing.assert_allclose(oup.rope_exact(oup.rope_exact(q, m, 1e6), t, 1e6), oup.rope_exact(q, m + t, 1e6),
                                   rtol=0, atol=1e-9)


def test_row_positions_chain_and_tree():
    L = np.array([0, 7, 100])
    pos, slots = oup.row_positions(L, 3)
    np.testing.assert_array_equal(pos, L[:, None] + np.arange(4))
    np.testing.assert_array_equal(slots, pos)
    rng = np.random.default_rng(3)
    parents = np.stack([random_parents(rng, 9) for _ in range(3)])
    pos, slots = oup.row_positions(L, 9, parents)
    for b in range(3):
        np.testing.assert_array_equal(pos[b], L[b] + np.array(otree.depths(parents[b])))
        np.testing.assert_array_equal(slots[b], L[b] + np.arange(10))


def _new_rows(p, k, seed):
    rng = np.random.default_rng(seed)
    shape_q, shape_kv = (p.B, k + 1, p.Hq, p.D), (p.B, k + 1, p.Hkv, p.D)
    f = lambda s: oup.f64_to_bf16(rng.standard_normal(s).astype(np.float32).astype(np.float64))
    return f(shape_q), f(shape_kv), f(shape_kv)


def test_append_then_attention_equals_a_dense_softmax():
    p = PRESETS["tiny"]
    k = p.k
    a = make_attention_inputs(p, seed=4)
    q, kn, vn = _new_rows(p, k, 4)
    theta = 500000.0
    q_rot, kc, vc = oup.rope_append(q, kn, vn, a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], theta)
    got = oatt.verify_attention(q_rot, kc, vc, a["block_table"], a["seq_lens"], k, p.Hq, p.Hkv, p.block_size,
                                a["sm_scale"])
    G = p.Hq // p.Hkv
    for b in range(p.B):
        L = int(a["seq_lens"][b])
        pos = L + np.arange(k + 1)
        for g in range(p.Hkv):
            K0, V0 = oatt.gather_sequence_kv(a["k_cache"], a["v_cache"], a["block_table"], b, g, L, p.block_size)
            k_rows = oatt.bf16_to_f64(oup.f64_to_bf16(oup.rope_exact(oatt.bf16_to_f64(kn[b, :, g]), pos, theta)))
            K = np.concatenate([K0, k_rows])
            Vv = np.concatenate([V0, oatt.bf16_to_f64(vn[b, :, g])])
            for i in range(k + 1):
                for h in range(g * G, (g + 1) * G):
                    qr = oatt.bf16_to_f64(oup.f64_to_bf16(oup.rope_exact(oatt.bf16_to_f64(q[b, i, h]), pos[i],
                                                                          theta)))
                    s = a["sm_scale"] * (K[: L + i + 1] @ qr)
                    w = np.exp(s - s.max())
                    np.testing.assert_allclose(got[b, i, h], (w / w.sum()) @ Vv[: L + i + 1], rtol=0, atol=1e-12)
    # only the new slots changed
    bs = p.block_size
    allowed = {(int(a["block_table"][b, (int(a["seq_lens"][b]) + i) // bs]), (int(a["seq_lens"][b]) + i) % bs)
               for b in range(p.B) for i in range(k + 1)}
    changed = {(int(pg), int(o)) for pg, _, o in zip(*np.nonzero((kc != a["k_cache"]).any(axis=3)))}
    changed |= {(int(pg), int(o)) for pg, _, o in zip(*np.nonzero((vc != a["v_cache"]).any(axis=2)))}
    assert changed <= allowed


def test_lm_head_brute_force_on_small_integers():
    rng = np.random.default_rng(5)
    hid = rng.integers(-3, 4, size=(3, 7))
    w = rng.integers(-3, 4, size=(5, 7))
    to_bits = lambda z: oup.f64_to_bf16(z.astype(np.float64))
    got = oup.lm_head(to_bits(hid), to_bits(w))
    for r in range(3):
        for v in range(5):
            assert got[r, v] == sum(int(hid[r, h]) * int(w[v, h]) for h in range(7))


def test_lm_head_orientation_and_rounding_bound():
    R, H, V = 4, 64, 9
    rng = np.random.default_rng(6)
    hid = oup.f64_to_bf16(rng.standard_normal((R, H)))
    w = np.zeros((V, H), dtype=np.uint16)
    w[6, 17] = 0x3F80                                   # W[6][17] = 1
    out = oup.lm_head(hid, w)
    np.testing.assert_array_equal(out[:, 6], oatt.bf16_to_f64(hid[:, 17]))
    assert not out[:, [0, 1, 2, 3, 4, 5, 7, 8]].any()
    H = 4096
    hid = oup.f64_to_bf16(rng.standard_normal((8, H)))
    w = oup.f64_to_bf16(rng.standard_normal((16, H)) * 0.05)
    exact = oup.lm_head(hid, w)
    f32 = oatt.bf16_to_f64(hid).astype(np.float32) @ oatt.bf16_to_f64(w).astype(np.float32).T
    bound = oup.lm_head_error_bound(hid, w)
    assert np.all(np.abs(f32.astype(np.float64) - exact) <= bound)
    # a sequential fp32 sum, the worst order for error growth, stays inside it too
    seq = np.zeros((8, 16), dtype=np.float32)
    prods = (oatt.bf16_to_f64(hid)[:, None, :] * oatt.bf16_to_f64(w)[None, :, :]).astype(np.float32)
    for h in range(H):
        seq += prods[:, :, h]
    assert np.all(np.abs(seq.astype(np.float64) - exact) <= bound)


def _fp32_blocked_sum(prods: np.ndarray, block: int, start_block: int, perm: np.ndarray) -> np.ndarray:
    """fp32 sum over the last axis the way a blocked device sum runs: blocks of `block` terms
    from block `start_block` on (wrapping), each block's terms added in the order `perm`."""
    n = prods.shape[-1]
    nb = n // block
    acc = np.zeros(prods.shape[:-1], dtype=np.float32)
    for bi in range(nb):
        b = (start_block + bi) % nb
        for j in perm:
            acc = (acc + prods[..., b * block + j]).astype(np.float32)
    return acc


def test_lm_head_stat_bound_holds_for_fp32_sums_and_catches_a_lost_block():
    """The statistical bound against fp32 sums actually carried out in float32 (numpy adds
    rounded to nearest): sequential, blocked with a permuted order inside the block, and
    rotated to start at another block; it is much tighter than the worst-case bound, and a
    sum that loses one block of terms, or adds one block twice, breaks it."""
    rng = np.random.default_rng(11)
    R, H, V = 6, 1024, 40
    hid = oup.f64_to_bf16(rng.standard_normal((R, H)))
    w = oup.f64_to_bf16(rng.standard_normal((V, H)) * 0.05)
    w[3] = oup.f64_to_bf16(np.abs(rng.standard_normal(H)) * 0.05)     # one same-sign column
    exact = oup.lm_head(hid, w)
    stat = oup.lm_head_stat_bound(hid, w)
    worst = oup.lm_head_error_bound(hid, w)
    prods = (oatt.bf16_to_f64(hid)[:, None, :] * oatt.bf16_to_f64(w)[None, :, :]).astype(np.float32)
    assert np.array_equal(prods.astype(np.float64),
                          oatt.bf16_to_f64(hid)[:, None, :] * oatt.bf16_to_f64(w)[None, :, :])   # exact in fp32
    perm = np.array([16 * g + 8 * s + j for s in range(2) for g in range(4) for j in range(8)])
    orders = [_fp32_blocked_sum(prods, H, 0, np.arange(H)),          # sequential
              _fp32_blocked_sum(prods, 64, 0, perm),
              _fp32_blocked_sum(prods, 64, 5, perm)]
    for got in orders:
        err = np.abs(got.astype(np.float64) - exact)
        assert np.all(err <= stat)
    assert np.all(stat < worst) and np.median(worst / stat) >= 10.0
    lost = orders[1].astype(np.float64) - prods[..., 64:128].astype(np.float64).sum(axis=-1)
    twice = orders[1].astype(np.float64) + prods[..., 64:128].astype(np.float64).sum(axis=-1)
    for bad in (lost, twice):
        assert np.mean(np.abs(bad - exact) > stat) > 0.9
