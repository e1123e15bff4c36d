"""Seeded synthetic workloads for the verify step (NumPy PCG64 only).

The pages measure on trained Qwen3 / Qwen2.5 policies, EAGLE-3 drafters and
math-reasoning prompt sets; none of those weights or datasets are used. These
arrays stand in for them, with the shapes, sizes and value distributions of the
five verify workloads (tiny chain, 8B-shaped, 7B-shaped large batch, long-tail
deep draft, 256K context):

* Q, K and V entries are i.i.d. N(0, 1), rounded to bfloat16 (round to nearest
  even). K pages are stored ``[num_blocks][Hkv][block_size][D]`` and V pages
  ``[num_blocks][Hkv][D][block_size]`` (key index fastest inside a V page).
* Each sequence's committed length L_b is drawn from the workload's context
  distribution; its k+1 newest KV rows (positions L_b .. L_b+k) are already in
  the cache, so it owns ceil((L_b+k+1)/block_size) pages, scattered by a random
  permutation of the physical pages.
* Page slots past a sequence's last key, spare physical pages and block-table
  entries past a sequence's last page are filled with garbage (large finite
  values, or NaN) and must never influence a result. Unused block-table entries
  point at a garbage page rather than out of bounds.
* Target logits are N(0, sigma^2) in fp32, plus ``boost`` on i.i.d.
  Bernoulli(boost_prob) entries (peaked distributions). Draft logits are the
  target logits plus N(0, draft_sigma^2) noise.
* Draft token j of each sequence is a sample from softmax(draft_logits_j / T),
  drawn with the Gumbel-max construction from PCG64 uniforms, which are
  independent of the verify step's own counter-based uniforms.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Preset:
    name: str
    index: int
    B: int
    k: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    ctx: tuple            # ("uniform", lo, hi) | ("lognormal", median, log_sigma, lo, hi) | ("fixed", n)
    V: int
    target_sigma: float
    boost_prob: float
    boost: float
    draft_sigma: float
    temperature: float = 1.0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def max_context(self) -> int:
        kind = self.ctx[0]
        if kind == "uniform":
            return int(self.ctx[2])
        if kind == "lognormal":
            return int(self.ctx[4])
        return int(self.ctx[1])


PRESETS = {
    p.name: p
    for p in (
        Preset("tiny", 0, B=4, k=3, Hq=4, Hkv=2, D=64, block_size=16, ctx=("uniform", 64, 256),
               V=1000, target_sigma=2.0, boost_prob=0.0, boost=0.0, draft_sigma=0.5),
        Preset("8b", 1, B=64, k=3, Hq=32, Hkv=8, D=128, block_size=16, ctx=("uniform", 1024, 8192),
               V=128256, target_sigma=3.0, boost_prob=0.01, boost=8.0, draft_sigma=1.0),
        Preset("7b", 2, B=256, k=3, Hq=28, Hkv=4, D=128, block_size=16,
               ctx=("lognormal", 3072, 0.5, 512, 8192),
               V=152064, target_sigma=3.0, boost_prob=0.01, boost=8.0, draft_sigma=1.5),
        Preset("longtail", 3, B=8, k=7, Hq=32, Hkv=8, D=128, block_size=16, ctx=("uniform", 32768, 65536),
               V=128256, target_sigma=3.0, boost_prob=0.01, boost=8.0, draft_sigma=2.0),
        Preset("262k", 4, B=2, k=3, Hq=64, Hkv=8, D=128, block_size=64, ctx=("fixed", 262144),
               V=151936, target_sigma=3.0, boost_prob=0.01, boost=8.0, draft_sigma=1.0),
    )
}

BF16_NAN = np.uint16(0x7FC0)


def verify_seed(preset: Preset) -> int:
    """Default 64-bit seed handed to the verify step for a workload."""
    return 0x5EED0000 + preset.index


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even) and return the raw uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def _normal_bf16(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    """N(0,1) bfloat16 bits of the given shape, generated in chunks to bound host memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def _context_lengths(rng: np.random.Generator, preset: Preset, B: int) -> np.ndarray:
    kind = preset.ctx[0]
    if kind == "uniform":
        lo, hi = preset.ctx[1], preset.ctx[2]
        return rng.integers(lo, hi + 1, size=B).astype(np.int32)
    if kind == "lognormal":
        median, log_sigma, lo, hi = preset.ctx[1:]
        x = np.exp(math.log(median) + log_sigma * rng.standard_normal(B))
        return np.clip(np.rint(x), lo, hi).astype(np.int32)
    if kind == "fixed":
        return np.full(B, preset.ctx[1], dtype=np.int32)
    raise ValueError(kind)


def _garbage_fill(rng: np.random.Generator, n: int, garbage: str) -> np.ndarray:
    if garbage == "nan":
        return np.full(n, BF16_NAN, dtype=np.uint16)
    signs = np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    return bf16_bits(signs * np.float32(1000.0))


def make_attention_inputs(preset: Preset, seed: int | None = None, B: int | None = None,
                          garbage: str = "finite", seq_lens: np.ndarray | None = None,
                          extra_capacity: int | None = None) -> dict:
    """Paged-KV inputs for verify attention.

    Returns raw bfloat16 bits (uint16) for q / k_cache / v_cache, an int32 block
    table and the committed lengths ``seq_lens`` (L_b; the cache already holds
    L_b + k + 1 keys per sequence).
    """
    rng = np.random.Generator(np.random.PCG64(preset.index if seed is None else seed))
    B = preset.B if B is None else B
    k, Hq, Hkv, D, bs = preset.k, preset.Hq, preset.Hkv, preset.D, preset.block_size
    L = _context_lengths(rng, preset, B) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    n_keys = L.astype(np.int64) + k + 1
    pages = (n_keys + bs - 1) // bs
    extra = (2 * (k + 1)) if extra_capacity is None else extra_capacity
    max_blocks = int((int(n_keys.max()) + extra + bs - 1) // bs)
    used = int(pages.sum())
    n_spare = max(1, used // 64)
    num_blocks = used + n_spare
    perm = rng.permutation(num_blocks).astype(np.int32)
    garbage_page = perm[used]                      # first spare physical page
    block_table = np.full((B, max_blocks), garbage_page, dtype=np.int32)
    off = 0
    for b in range(B):
        block_table[b, : pages[b]] = perm[off: off + pages[b]]
        off += pages[b]

    q = _normal_bf16(rng, (B, k + 1, Hq, D))
    k_cache = _normal_bf16(rng, (num_blocks, Hkv, bs, D))
    v_cache = _normal_bf16(rng, (num_blocks, Hkv, D, bs))

    # Garbage: whole spare pages, and the slots of each last page past the sequence's keys.
    spare = perm[used:]
    for pg in spare:
        k_cache[pg] = _garbage_fill(rng, Hkv * bs * D, garbage).reshape(Hkv, bs, D)
        v_cache[pg] = _garbage_fill(rng, Hkv * D * bs, garbage).reshape(Hkv, D, bs)
    for b in range(B):
        fill = int(pages[b] * bs - n_keys[b])
        if fill == 0:
            continue
        pg = block_table[b, pages[b] - 1]
        s0 = bs - fill
        k_cache[pg, :, s0:, :] = _garbage_fill(rng, Hkv * fill * D, garbage).reshape(Hkv, fill, D)
        v_cache[pg, :, :, s0:] = _garbage_fill(rng, Hkv * D * fill, garbage).reshape(Hkv, D, fill)

    return dict(preset=preset, B=B, k=k, Hq=Hq, Hkv=Hkv, D=D, block_size=bs,
                q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                seq_lens=L, max_blocks=max_blocks, num_blocks=num_blocks,
                max_seq_len=int(n_keys.max()), sm_scale=1.0 / math.sqrt(D))


def draft_from_logits(rng: np.random.Generator, draft_logits: np.ndarray, temperature: float) -> np.ndarray:
    """One sample per row of softmax(draft_logits / T) by the Gumbel-max construction."""
    rows = draft_logits.reshape(-1, draft_logits.shape[-1])
    out = np.empty(rows.shape[0], dtype=np.int32)
    for r in range(rows.shape[0]):
        u = (rng.integers(1, 1 << 53, size=rows.shape[1]).astype(np.float64)) * (2.0 ** -53)
        g = -np.log(-np.log(u))
        out[r] = int(np.argmax(rows[r].astype(np.float64) / temperature + g))
    return out.reshape(draft_logits.shape[:-1])


def make_reject_inputs(preset: Preset, seed: int | None = None, B: int | None = None,
                       seq_lens: np.ndarray | None = None) -> dict:
    """Target / draft logits, draft tokens, sequence ids and committed lengths."""
    rng = np.random.Generator(np.random.PCG64(1000 + (preset.index if seed is None else seed)))
    B = preset.B if B is None else B
    k, V, T = preset.k, preset.V, preset.temperature
    if seq_lens is None:
        L = _context_lengths(np.random.Generator(np.random.PCG64(preset.index if seed is None else seed)),
                             preset, B)
    else:
        L = np.asarray(seq_lens, dtype=np.int32)
    target = rng.standard_normal((B, k + 1, V), dtype=np.float32) * np.float32(preset.target_sigma)
    if preset.boost_prob > 0:
        target += np.float32(preset.boost) * (rng.random((B, k + 1, V)) < preset.boost_prob).astype(np.float32)
    draft = target[:, :k, :] + rng.standard_normal((B, k, V), dtype=np.float32) * np.float32(preset.draft_sigma)
    draft = np.ascontiguousarray(draft, dtype=np.float32)
    tokens = draft_from_logits(rng, draft, T)
    seq_ids = (np.arange(B, dtype=np.int64) * 7919 + 1_000_003 * (preset.index + 1)).astype(np.int64)
    return dict(preset=preset, B=B, k=k, V=V, temperature=T,
                target_logits=np.ascontiguousarray(target), draft_logits=draft,
                draft_tokens=tokens.astype(np.int32), seq_ids=seq_ids, seq_lens=L,
                seed=verify_seed(preset))


def make_inputs(name: str, seed: int | None = None, B: int | None = None, garbage: str = "finite",
                preset: Preset | None = None) -> dict:
    preset = PRESETS[name] if preset is None else preset
    a = make_attention_inputs(preset, seed=seed, B=B, garbage=garbage)
    r = make_reject_inputs(preset, seed=seed, B=B, seq_lens=a["seq_lens"])
    out = dict(a)
    out.update({kk: vv for kk, vv in r.items() if kk not in ("preset", "B", "k")})
    return out
