"""Lossless acceptance chain of speculative decoding (fp64 oracle).

What the pages fix:
* "Accelerating RL Post-Training Rollouts via System-Integrated Speculative
  Decoding" (gist.science technical summary), section 2 "Method", core
  mechanism: a draft proposes k tokens, the target verifies them in one pass,
  and rejection sampling against the verifier's distribution keeps the rollout
  distribution identical to the target policy. The explainer part of the same
  page: with k = 3 up to four tokens are adopted in one step, and on a miss the
  verifier writes its own token instead.
* "Online Draft Co-Training for Speculative Decoding ..." (ta-paperlens
  commentary), section "比喩: 速記者と校閲者" (stenographer / proofreader
  metaphor): the verifier rewrites from the first draft token that misses, and
  because verification is rejection sampling the output distribution equals the
  verifier writing alone.
* "EfficientRollout: System-Aware Self-Speculative Decoding for RL Rollouts",
  abstract: rollouts are long, high-temperature generations.

The pages never print the acceptance rule. It is taken from the standard
speculative-sampling algorithm (Leviathan, Kalman & Matias 2023; Chen et al.
2023), which is the rule that makes the guarantee above hold:

  for j = 0 .. k-1 (position P = L + 1 + j, uniforms (u_acc, u_smp) = Philox(seed, seq, P)):
      x = d_j;  accept iff u_acc < p_j(x) / q_j(x)      (q_j(x) = 0: ratio +inf if p_j(x) > 0, else 0)
      on accept emit x; on the first reject emit a sample of the normalised
      residual max(0, p_j - q_j) using u_smp, and stop.
  if all k are accepted, emit a bonus token from p_k with u_smp at P = L + 1 + k.

with p_j = softmax(target_logits_j / T) and q_j = softmax(draft_logits_j / T).
Sampling is inverse-CDF in ascending token id: the smallest y with
C(y) > u_smp * R, C the running sum of the weights and R = C(V-1); zero-weight
tokens can never be chosen; if rounding leaves no such y, the largest y with
positive weight. If the residual sums to zero after a rejection (impossible in
exact arithmetic) the sample is taken from p_j.

Every decision records its margin: |u_acc - p/q| for an acceptance test, and
for a sample the distance from u_smp * R to the nearer edge of the chosen
interval, divided by R.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

from .philox import verify_uniforms


def softmax_t(logits: np.ndarray, temperature: float) -> np.ndarray:
    """softmax(z / T) in fp64 with max subtraction; the normaliser is an exactly rounded sum."""
    z = np.asarray(logits, dtype=np.float64)
    x = (z - z.max()) / float(temperature)
    e = np.exp(x)
    return e / math.fsum(e)


def inverse_cdf(weights: np.ndarray, u: float, C: np.ndarray | None = None):
    """(token, margin): smallest y with C(y) > u * C(V-1); margin relative to the total weight.

    ``C`` may pass the running sum of ``weights`` when it is already known.
    """
    if C is None:
        C = np.cumsum(weights)
    R = float(C[-1])
    t = u * R
    y = int(np.searchsorted(C, t, side="right"))
    if y >= len(weights):
        pos = np.nonzero(weights > 0)[0]
        return int(pos[-1]), 0.0
    lower = float(C[y - 1]) if y > 0 else 0.0
    return y, min(t - lower, float(C[y]) - t) / R


@dataclasses.dataclass
class Decision:
    kind: str          # "accept" (an acceptance test) or "sample" (residual or bonus draw)
    j: int             # draft index (for "sample": the index the sampled token is emitted at)
    outcome: int       # 1/0 for accept tests; the token id for samples
    margin: float


@dataclasses.dataclass
class SequenceResult:
    tokens: list
    num_accepted: int
    out_probs: list
    accept_probs: list
    decisions: list


class SequenceRows:
    """The probability rows of one sequence, computed once and reused across many uniforms."""

    def __init__(self, target_logits: np.ndarray, draft_logits: np.ndarray, temperature: float):
        self.target_logits = target_logits
        self.draft_logits = draft_logits
        self.temperature = temperature
        self._p = {}
        self._q = {}
        self._res = {}
        self._cdf = {}

    def p(self, j: int) -> np.ndarray:
        if j not in self._p:
            self._p[j] = softmax_t(self.target_logits[j], self.temperature)
        return self._p[j]

    def q(self, j: int) -> np.ndarray:
        if j not in self._q:
            self._q[j] = softmax_t(self.draft_logits[j], self.temperature)
        return self._q[j]

    def residual(self, j: int) -> np.ndarray:
        if j not in self._res:
            r = np.maximum(0.0, self.p(j) - self.q(j))
            self._res[j] = r if r.sum() > 0 else self.p(j)
        return self._res[j]

    def cdf(self, kind: str, j: int) -> np.ndarray:
        """Running sum of the residual ("res") or of p ("p") of row j, computed once."""
        key = (kind, j)
        if key not in self._cdf:
            self._cdf[key] = np.cumsum(self.residual(j) if kind == "res" else self.p(j))
        return self._cdf[key]


def decide(rows: SequenceRows, draft_tokens, k: int, uniforms) -> SequenceResult:
    """Run the chain for one sequence given its uniforms[j] = (u_acc, u_smp), j = 0..k."""
    tokens, out_probs, accept_probs, decisions = [], [], [], []
    for j in range(k):
        x = int(draft_tokens[j])
        p_x = float(rows.p(j)[x])
        q_x = float(rows.q(j)[x])
        if q_x > 0.0:
            ratio = p_x / q_x
        else:
            ratio = math.inf if p_x > 0.0 else 0.0
        u_acc, u_smp = uniforms[j]
        accept_probs.append(min(1.0, ratio))
        accepted = u_acc < ratio
        decisions.append(Decision("accept", j, int(accepted),
                                  math.inf if math.isinf(ratio) else abs(u_acc - ratio)))
        if accepted:
            tokens.append(x)
            out_probs.append(p_x)
            continue
        y, margin = inverse_cdf(rows.residual(j), u_smp, rows.cdf("res", j))
        decisions.append(Decision("sample", j, y, margin))
        tokens.append(y)
        out_probs.append(float(rows.p(j)[y]))
        return SequenceResult(tokens, j, out_probs, accept_probs, decisions)
    y, margin = inverse_cdf(rows.p(k), uniforms[k][1], rows.cdf("p", k))
    decisions.append(Decision("sample", k, y, margin))
    tokens.append(y)
    out_probs.append(float(rows.p(k)[y]))
    return SequenceResult(tokens, k, out_probs, accept_probs, decisions)


def sequence_uniforms(seed: int, seq_id: int, committed_len: int, k: int):
    """Uniforms for positions L+1 .. L+1+k (the tokens decided in this verify step)."""
    return [verify_uniforms(seed, seq_id, committed_len + 1 + j) for j in range(k + 1)]


def verify_batch(target_logits, draft_logits, draft_tokens, seq_ids, seq_lens, k: int,
                 temperature: float, seed: int, rows_cache=None):
    """Batch driver; returns dict of output arrays (padded like the C-ABI) and per-sequence results.

    out_tokens [B][k+1] (-1 past the emitted tokens), num_accepted [B],
    out_probs [B][k+1] (0 past the emitted tokens), accept_probs [B][k]
    (-1 for positions not tested).
    """
    B = target_logits.shape[0]
    out_tokens = np.full((B, k + 1), -1, dtype=np.int32)
    out_probs = np.zeros((B, k + 1), dtype=np.float64)
    accept_probs = np.full((B, k), -1.0, dtype=np.float64)
    num_accepted = np.zeros(B, dtype=np.int32)
    results = []
    for b in range(B):
        rows = rows_cache[b] if rows_cache is not None else SequenceRows(
            target_logits[b], draft_logits[b], temperature)
        res = decide(rows, draft_tokens[b], k, sequence_uniforms(seed, int(seq_ids[b]), int(seq_lens[b]), k))
        n = len(res.tokens)
        out_tokens[b, :n] = res.tokens
        out_probs[b, :n] = res.out_probs
        accept_probs[b, : len(res.accept_probs)] = res.accept_probs
        num_accepted[b] = res.num_accepted
        results.append(res)
    return dict(out_tokens=out_tokens, num_accepted=num_accepted, out_probs=out_probs,
                accept_probs=accept_probs, results=results)


def verify_batch_ragged(target_logits, draft_logits, draft_tokens, cu_drafts, seq_ids, seq_lens,
                        temperature: float, seed: int, rows_cache=None):
    """Ragged draft lengths ("EfficientRollout: System-Aware Self-Speculative Decoding for RL
    Rollouts", abstract: the draft length adapts to acceptance): sequence b has
    k_b = cu[b+1] - cu[b] drafts and runs the same chain over them. Rows are packed:
    target_logits / out_tokens / out_probs row cu[b] + b + j (j = 0 .. k_b), draft_logits /
    draft_tokens / accept_probs row cu[b] + j (j < k_b). Unused entries are -1 (tokens,
    accept_probs) or 0 (out_probs), as in the uniform layout."""
    cu = [int(c) for c in cu_drafts]
    B = len(seq_ids)
    T, K = cu[B] + B, cu[B]
    out_tokens = np.full(T, -1, dtype=np.int32)
    out_probs = np.zeros(T, dtype=np.float64)
    accept_probs = np.full(K, -1.0, dtype=np.float64)
    num_accepted = np.zeros(B, dtype=np.int32)
    results = []
    for b in range(B):
        kb, t0, d0 = cu[b + 1] - cu[b], cu[b] + b, cu[b]
        rows = rows_cache[b] if rows_cache is not None else SequenceRows(
            target_logits[t0:t0 + kb + 1], draft_logits[d0:d0 + kb], temperature)
        res = decide(rows, draft_tokens[d0:d0 + kb], kb,
                     sequence_uniforms(seed, int(seq_ids[b]), int(seq_lens[b]), kb))
        n = len(res.tokens)
        out_tokens[t0:t0 + n] = res.tokens
        out_probs[t0:t0 + n] = res.out_probs
        accept_probs[d0:d0 + len(res.accept_probs)] = res.accept_probs
        num_accepted[b] = res.num_accepted
        results.append(res)
    return dict(out_tokens=out_tokens, num_accepted=num_accepted, out_probs=out_probs,
                accept_probs=accept_probs, results=results)
