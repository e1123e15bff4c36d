"""Seeded synthetic inputs for the speculative-decoding verify step.

This package is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark. It only draws random numbers and lays them out in memory; it
holds none of the verify step's arithmetic (no softmax, no acceptance test, no
attention, no counter-based uniforms).
"""

from .gen import PRESETS, Preset, make_attention_inputs, make_reject_inputs, make_inputs  # noqa: F401
from .gen import bf16_bits, verify_seed, draft_from_logits  # noqa: F401
from .ragged import (make_ragged_attention_inputs, make_ragged_reject_inputs, pack_reject_inputs,  # noqa: F401
                     ragged_draft_lengths, offsets)
from .tree import make_tree_attention_inputs, make_tree_reject_inputs, random_parents, random_paths, tree_parents  # noqa: F401
from .upstream import ROPE_THETA, make_lm_head_inputs, make_new_rows  # noqa: F401
