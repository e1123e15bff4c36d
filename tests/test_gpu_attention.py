"""GPU parity of spec_verify_attn against the fp64 oracle (<= 1e-2 absolute).

Small shapes are compared element by element (several chunks, ragged tails,
every supported head dim / block size, GQA groups giving 1, 2 and more 16-row
tiles, NaN garbage outside the sequences); the full-size workloads are compared
on every row, in the launch configuration the benchmark times.
"""

import math

import numpy as np
import pytest

from oracle import attention as oatt
from tests.parity import ATTN_TOL, run_attention, say
from workloads import PRESETS, Preset, make_attention_inputs

pytestmark = pytest.mark.gpu


def _full_oracle(inp):
    return oatt.verify_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"], inp["seq_lens"],
                                 inp["k"], inp["Hq"], inp["Hkv"], inp["block_size"], inp["sm_scale"])


def _assert_close(got, want, label):
    err = np.abs(got - want)
    say(f"[attn] {label}: max abs err {err.max():.3e}")
    assert np.all(np.isfinite(got)), label
    assert err.max() <= ATTN_TOL, (label, err.max())


def _preset(**kw):
    base = dict(name="t", index=0, B=3, k=3, Hq=8, Hkv=2, D=128, block_size=16, ctx=("uniform", 100, 3000),
                V=10, target_sigma=1.0, boost_prob=0.0, boost=0.0, draft_sigma=1.0)
    base.update(kw)
    return Preset(**base)


def test_tiny_full(device):
    inp = make_attention_inputs(PRESETS["tiny"])
    _assert_close(run_attention(inp, device), _full_oracle(inp), "tiny")


@pytest.mark.parametrize("D,Hq,Hkv,k,bs", [
    (128, 32, 8, 3, 16),    # 16 rows: one tile, 8B-shaped heads
    (128, 28, 4, 3, 16),    # 28 rows: two tiles with padding (7B-shaped heads)
    (128, 64, 8, 3, 64),    # 32 rows: two tiles, 64-token pages (256K shape)
    (128, 32, 8, 7, 16),    # 32 rows, k = 7 (long-tail shape)
    (64, 4, 2, 3, 16),      # tiny heads
    (64, 8, 1, 3, 32),      # G = 8 onto one KV head
    (128, 16, 16, 1, 32),   # G = 1, k = 1: 2 rows
    (128, 64, 4, 7, 16),    # 128 rows: four row groups
    (64, 48, 4, 15, 64),    # k = 15, G = 12: 192 rows
    (128, 32, 8, 0, 16),    # k = 0 (plain decoding), 8B heads: 4 rows
    (128, 16, 16, 0, 32),   # k = 0, G = 1: a single query row
    (64, 48, 4, 0, 64),     # k = 0, G = 12: 12 rows
])
def test_shapes(device, D, Hq, Hkv, k, bs):
    p = _preset(D=D, Hq=Hq, Hkv=Hkv, k=k, block_size=bs, B=3, ctx=("uniform", 300, 5000))
    inp = make_attention_inputs(p, seed=D + Hq + k + bs)
    _assert_close(run_attention(inp, device), _full_oracle(inp), f"D{D} Hq{Hq} Hkv{Hkv} k{k} bs{bs}")


def test_nan_garbage_and_tiny_contexts(device):
    # L = 0 (row 0 sees one key), lengths around page and block edges, NaN in every unused slot
    p = _preset(B=8, Hq=8, Hkv=2, k=3)
    L = np.array([0, 1, 12, 13, 28, 29, 31, 1021])
    inp = make_attention_inputs(p, seed=11, garbage="nan", seq_lens=L)
    got = run_attention(inp, device)
    _assert_close(got, _full_oracle(inp), "nan-garbage")


def test_split_boundaries(device):
    """Contexts that land exactly on and just past KV-split and 32-key block edges."""
    p = _preset(B=6, Hq=32, Hkv=8, k=3)
    L = np.array([252, 253, 508, 1020, 1021, 4092])   # L + k + 1 = 256, 257, 512, 1024, 1025, 4096
    inp = make_attention_inputs(p, seed=12, seq_lens=L)
    _assert_close(run_attention(inp, device), _full_oracle(inp), "split-edges")
    # the same inputs with a larger max_seq_len (more, shorter splits may be chosen)
    _assert_close(run_attention(inp, device, max_seq_len=65536), _full_oracle(inp), "split-edges/msl")


def test_many_tiny_sequences_split_everywhere(device):
    """Hundreds of short sequences: work shares start and end inside segments everywhere."""
    p = _preset(B=700, Hq=8, Hkv=2, D=64, k=3, ctx=("uniform", 0, 300))
    inp = make_attention_inputs(p, seed=21)
    _assert_close(run_attention(inp, device), _full_oracle(inp), "B700 tiny contexts")


def test_batch_above_lds_prefix_limit(device):
    """B = 5000 takes the separate planning launch for the per-sequence work prefix."""
    p = _preset(B=5000, Hq=4, Hkv=1, D=64, k=1, ctx=("uniform", 0, 60))
    inp = make_attention_inputs(p, seed=22)
    got = run_attention(inp, device)
    want = oatt.verify_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"], inp["seq_lens"],
                                 inp["k"], inp["Hq"], inp["Hkv"], inp["block_size"], inp["sm_scale"],
                                 pairs=[(b, 0) for b in range(0, 5000, 7)])
    rows = list(range(0, 5000, 7))
    _assert_close(got[rows], want[rows], "B5000")


def _every_row(inp, got, label):
    """The whole launch against the oracle: every (sequence, row, query head)."""
    want = oatt.verify_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"], inp["seq_lens"],
                                 inp["k"], inp["Hq"], inp["Hkv"], inp["block_size"], inp["sm_scale"])
    assert np.all(np.isfinite(got))
    err = np.abs(got - want)
    say(f"[attn] {label}: all {got.shape[0] * got.shape[1] * got.shape[2]} rows, max abs err {float(err.max()):.3e}")
    assert float(err.max()) <= ATTN_TOL


@pytest.mark.parametrize("name,B", [("8b", 64), ("7b", 256), ("7b", 64), ("7b", 16), ("7b", 4), ("longtail", 8),
                                    ("262k", 2)])
def test_full_size_workloads_every_row(device, name, B):
    """Each workload at its full size, in the launch configuration the benchmark times."""
    inp = make_attention_inputs(PRESETS[name], B=B)
    got = run_attention(inp, device)
    _every_row(inp, got, f"{name}/B{B}")


def test_deterministic(device):
    inp = make_attention_inputs(PRESETS["8b"], B=8)
    a = run_attention(inp, device)
    b = run_attention(inp, device)
    np.testing.assert_array_equal(a, b)
    assert math.isfinite(float(a.sum()))
