"""Pins for the oracle's paged verify attention (CPU only).

* Dense brute force: pages gathered by fancy indexing into dense K and V,
  explicit causal mask matrix, one matrix softmax - equal to the paged oracle.
* Library routine: torch's scaled_dot_product_attention in float64 with a
  boolean mask and repeated KV heads.
* Closed forms: a single visible key returns that key's value row; identical
  keys, or a zero scale, return the mean of the visible value rows.
* Garbage outside the sequence (finite or NaN) never reaches the output.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from workloads import PRESETS, make_attention_inputs
from workloads.gen import bf16_bits


def _dense_reference(inp):
    """Independent formulation: gather all keys at once, mask matrix, matrix softmax."""
    q = oatt.bf16_to_f64(inp["q"])
    kc = oatt.bf16_to_f64(inp["k_cache"])
    vc = oatt.bf16_to_f64(inp["v_cache"])
    bt, L = inp["block_table"], inp["seq_lens"]
    B, k1, Hq, D = q.shape
    Hkv, bs, k = inp["Hkv"], inp["block_size"], inp["k"]
    G = Hq // Hkv
    out = np.empty_like(q)
    for b in range(B):
        n = int(L[b]) + k + 1
        t = np.arange(n)
        phys = bt[b, t // bs]
        Kd = kc[phys, :, t % bs, :]            # [n][Hkv][D]
        Vd = vc[phys, :, :, t % bs]            # [n][Hkv][D]
        mask = t[None, :] <= (int(L[b]) + np.arange(k1))[:, None]   # [k+1][n]
        for h in range(Hq):
            g = h // G
            S = inp["sm_scale"] * q[b, :, h, :] @ Kd[:, g, :].T     # [k+1][n]
            S = np.where(mask, S, -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            out[b, :, h, :] = P @ Vd[:, g, :]
    return out


def _oracle(inp):
    return oatt.verify_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                                 inp["seq_lens"], inp["k"], inp["Hq"], inp["Hkv"],
                                 inp["block_size"], inp["sm_scale"])


@pytest.fixture(scope="module")
def tiny():
    return make_attention_inputs(PRESETS["tiny"], seed=0)


def test_dense_brute_force(tiny):
    np.testing.assert_allclose(_oracle(tiny), _dense_reference(tiny), rtol=0, atol=1e-12)


def test_torch_sdpa_float64(tiny):
    inp = tiny
    q = oatt.bf16_to_f64(inp["q"])
    kc = oatt.bf16_to_f64(inp["k_cache"])
    vc = oatt.bf16_to_f64(inp["v_cache"])
    B, k1, Hq, D = q.shape
    Hkv, bs, k = inp["Hkv"], inp["block_size"], inp["k"]
    got = _oracle(inp)
    for b in range(B):
        n = int(inp["seq_lens"][b]) + k + 1
        t = np.arange(n)
        phys = inp["block_table"][b, t // bs]
        Kd = torch.from_numpy(np.ascontiguousarray(kc[phys, :, t % bs, :].transpose(1, 0, 2)))
        Vd = torch.from_numpy(np.ascontiguousarray(vc[phys, :, :, t % bs].transpose(1, 0, 2)))
        Kd = Kd.repeat_interleave(Hq // Hkv, dim=0)
        Vd = Vd.repeat_interleave(Hq // Hkv, dim=0)
        Q = torch.from_numpy(np.ascontiguousarray(q[b].transpose(1, 0, 2)))      # [Hq][k+1][D]
        mask = torch.from_numpy(t[None, :] <= (int(inp["seq_lens"][b]) + np.arange(k1))[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(Q, Kd, Vd, attn_mask=mask,
                                                               scale=inp["sm_scale"])
        np.testing.assert_allclose(got[b], ref.numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_single_visible_key_returns_its_value():
    # L = 0: draft row 0 sees only key 0.
    inp = make_attention_inputs(PRESETS["tiny"], seed=3, seq_lens=np.array([0, 0, 5, 17]))
    out = _oracle(inp)
    vc = oatt.bf16_to_f64(inp["v_cache"])
    for b in (0, 1):
        page = inp["block_table"][b, 0]
        for h in range(inp["Hq"]):
            g = h // (inp["Hq"] // inp["Hkv"])
            np.testing.assert_array_equal(out[b, 0, h], vc[page, g, :, 0])


def test_identical_keys_and_zero_scale_give_mean_of_visible_values():
    p = PRESETS["tiny"]
    inp = make_attention_inputs(p, seed=4)
    mean_rows = {}
    for variant in ("same_keys", "zero_scale"):
        x = dict(inp)
        if variant == "same_keys":
            kc = inp["k_cache"].copy()
            kc[:] = bf16_bits(np.linspace(-1, 1, p.D, dtype=np.float32))
            x["k_cache"] = kc
        else:
            x["sm_scale"] = 0.0
        out = _oracle(x)
        for b in range(inp["B"]):
            for i in range(p.k + 1):
                for h in range(p.Hq):
                    g = h // p.G
                    n = int(inp["seq_lens"][b]) + i + 1
                    _, Vv = oatt.gather_sequence_kv(inp["k_cache"], inp["v_cache"], inp["block_table"],
                                                    b, g, n, p.block_size)
                    want = mean_rows.setdefault((b, i, h), np.mean(Vv, axis=0))
                    np.testing.assert_allclose(out[b, i, h], want, rtol=0, atol=1e-12)


def test_garbage_never_reaches_output():
    a = make_attention_inputs(PRESETS["tiny"], seed=5, garbage="finite")
    b = make_attention_inputs(PRESETS["tiny"], seed=5, garbage="nan")
    oa, ob = _oracle(a), _oracle(b)
    assert np.all(np.isfinite(ob))
    np.testing.assert_array_equal(oa, ob)


def test_causal_mask_inside_draft_matters():
    """Row i must not see keys L+i+1..L+k: perturbing key L+k changes only row k."""
    inp = make_attention_inputs(PRESETS["tiny"], seed=6)
    base = _oracle(inp)
    kc = inp["k_cache"].copy()
    bs, k = inp["block_size"], inp["k"]
    for b in range(inp["B"]):
        t = int(inp["seq_lens"][b]) + k
        kc[inp["block_table"][b, t // bs], :, t % bs, :] = bf16_bits(np.full(inp["D"], 3.0, np.float32))
    x = dict(inp)
    x["k_cache"] = kc
    out = _oracle(x)
    np.testing.assert_array_equal(out[:, :k], base[:, :k])
    assert np.max(np.abs(out[:, k] - base[:, k])) > 1e-3


def test_default_scale_is_inverse_sqrt_d():
    assert PRESETS["8b"].D == 128
    inp = make_attention_inputs(PRESETS["tiny"], seed=0)
    assert inp["sm_scale"] == 1.0 / math.sqrt(64)
