"""Python binding of libspecverify.so, the HIP (gfx950) verify step of lossless
speculative decoding: paged-KV verify attention, vocab-wide rejection sampling
and the cache-length commit.

Argument marshalling only: every step runs in the library's kernels. torch
tensors provide device memory and the stream; nothing here computes on them.
The library must be built (``python -m speculative_decoding_verification_14_amd.build``
or ``__graft_entry__.build()``); importing works without it, but every call
raises ``SpecError`` if it is missing.
"""

from __future__ import annotations

import ctypes
import os
import threading

__all__ = ["SpecError", "library", "verify_attn", "verify_attn_workspace_size", "reject_sample",
           "reject_sample_workspace_size", "commit_lengths", "verify_step", "verify_attn_ragged",
           "reject_sample_ragged", "verify_attn_tree", "reject_sample_tree", "reject_sample_tree_workspace_size",
           "commit_tree", "rope_append", "lm_head", "reject_error_flag", "reject_workspace",
           "reject_sample_noalloc", "reject_sample_plan", "REJECT_PLANS",
           "LIB_PATH", "SYMBOLS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspecverify.so")

SPEC_OK = 0
_c_int32, _c_size, _vp = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/specverify.h
SYMBOLS = {
    "spec_status_string": (ctypes.c_char_p, [_c_int32]),
    "spec_abi_version": (_c_int32, []),
    "spec_verify_attn_workspace_size": (_c_int32, [_c_int32] * 6 + [ctypes.POINTER(_c_size)]),
    "spec_verify_attn": (_c_int32, [_vp] * 6 + [_c_int32] * 9 + [ctypes.c_float, _vp, _c_size, _vp]),
    "spec_reject_sample_workspace_size": (_c_int32, [_c_int32] * 3 + [ctypes.POINTER(_c_size)]),
    "spec_reject_sample": (_c_int32, [_vp] * 5 + [_c_int32] * 3 + [ctypes.c_float, ctypes.c_uint64]
                           + [_vp] * 5 + [_c_size, _vp]),
    "spec_commit_lengths": (_c_int32, [_vp, _vp, _c_int32, _c_int32, _c_int32, _vp, _vp]),
    "spec_verify_attn_ragged": (_c_int32, [_vp] * 7 + [_c_int32] * 9 + [ctypes.c_float, _vp, _c_size, _vp]),
    "spec_reject_sample_ragged": (_c_int32, [_vp] * 6 + [_c_int32] * 3 + [ctypes.c_float, ctypes.c_uint64]
                                  + [_vp] * 5 + [_c_size, _vp]),
    "spec_verify_attn_tree": (_c_int32, [_vp] * 7 + [_c_int32] * 9 + [ctypes.c_float, _vp, _c_size, _vp]),
    "spec_reject_sample_tree_workspace_size": (_c_int32, [_c_int32] * 3 + [ctypes.POINTER(_c_size)]),
    "spec_reject_sample_tree": (_c_int32, [_vp] * 6 + [_c_int32] * 3 + [ctypes.c_float, ctypes.c_uint64]
                                + [_vp] * 6 + [_c_size, _vp]),
    "spec_commit_tree": (_c_int32, [_vp] * 6 + [_c_int32] * 8 + [_vp, _vp]),
    "spec_rope_append": (_c_int32, [_vp] * 8 + [_c_int32] * 8 + [ctypes.c_double, _vp]),
    "spec_lm_head": (_c_int32, [_vp] * 3 + [_c_int32] * 3 + [_vp]),
    "spec_reject_error_flag": (_c_int32, [_vp, _vp, _vp]),
    "spec_reject_sample_plan": (_c_int32, [_c_int32] * 3 + [ctypes.POINTER(_c_int32)]),
    "spec_reject_sample_noalloc": (_c_int32, [_vp] * 5 + [_c_int32] * 3 + [ctypes.c_float, ctypes.c_uint64]
                                   + [_vp] * 5),
}


class SpecError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = library().spec_status_string(code).decode() if _lib is not None else f"status {code}"
        super().__init__(f"{where}: {msg} (status {code})")


_lib = None
_lock = threading.Lock()


def library():
    """The loaded libspecverify.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                                       "(python -m speculative_decoding_verification_14_amd.build)")
                lib = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SYMBOLS.items():
                    fn = getattr(lib, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = lib
    return _lib


def _check(code: int, where: str):
    if code != SPEC_OK:
        raise SpecError(code, where)


def _need(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _opt(t, dtype, name):
    return None if t is None else _need(t, dtype, name)


def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


# Per-device workspaces, zero-filled once; every call leaves them ready for the next.
_workspaces: dict = {}


def _workspace(kind: str, device, nbytes: int):
    import torch
    key = (kind, str(device))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def verify_attn_workspace_size(B, k, Hq, Hkv, D, max_seq_len) -> int:
    n = _c_size(0)
    _check(library().spec_verify_attn_workspace_size(B, k, Hq, Hkv, D, max_seq_len, ctypes.byref(n)),
           "spec_verify_attn_workspace_size")
    return n.value


def reject_sample_workspace_size(B, k, V) -> int:
    n = _c_size(0)
    _check(library().spec_reject_sample_workspace_size(B, k, V, ctypes.byref(n)), "spec_reject_sample_workspace_size")
    return n.value


REJECT_PLANS = {0: "chain, 512-thread workgroups", 1: "chain, 256-thread workgroups", 2: "every level at once"}


def reject_sample_plan(B, k, V) -> int:
    """spec_reject_sample_plan: 0 / 1 = the levels one after another (512- / 256-thread
    workgroups), 2 = every level of every sequence at once (all 2k+1 rows read)."""
    m = _c_int32(-1)
    _check(library().spec_reject_sample_plan(B, k, V, ctypes.byref(m)), "spec_reject_sample_plan")
    return m.value


def verify_attn(q, k_cache, v_cache, block_table, seq_lens, out, max_seq_len: int, sm_scale: float | None = None,
                workspace=None, stream=None):
    """spec_verify_attn. q/out bf16 [B][k+1][Hq][D]; k_cache bf16 [NB][Hkv][bs][D];
    v_cache bf16 [NB][Hkv][D][bs]; block_table int32 [B][max_blocks]; seq_lens int32 [B]."""
    import torch
    B, k1, Hq, D = q.shape
    NB, Hkv, bs, _ = k_cache.shape
    max_blocks = block_table.shape[1]
    scale = (1.0 / D ** 0.5) if sm_scale is None else float(sm_scale)
    lib = library()
    need = verify_attn_workspace_size(B, k1 - 1, Hq, Hkv, D, max_seq_len)
    if workspace is None and need > 0:
        workspace = _workspace("attn", q.device, need)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.spec_verify_attn(_need(q, torch.bfloat16, "q"), _need(k_cache, torch.bfloat16, "k_cache"),
                                _need(v_cache, torch.bfloat16, "v_cache"), _need(block_table, torch.int32, "block_table"),
                                _need(seq_lens, torch.int32, "seq_lens"), _need(out, torch.bfloat16, "out"),
                                B, k1 - 1, Hq, Hkv, D, bs, max_blocks, NB, int(max_seq_len), scale,
                                wptr, wbytes, _stream_handle(stream)), "spec_verify_attn")
    return out


def verify_attn_ragged(q, k_cache, v_cache, block_table, seq_lens, cu_drafts, out, max_k: int, max_seq_len: int,
                       sm_scale: float | None = None, workspace=None, stream=None):
    """spec_verify_attn_ragged. q/out bf16 [R][Hq][D] with R = cu_drafts[B] + B (sequence b's
    rows at cu_drafts[b] + b + i); cu_drafts int32 [B+1] on the device; max_k >= every k_b."""
    import torch
    R, Hq, D = q.shape
    NB, Hkv, bs, _ = k_cache.shape
    B = seq_lens.shape[0]
    max_blocks = block_table.shape[1]
    scale = (1.0 / D ** 0.5) if sm_scale is None else float(sm_scale)
    lib = library()
    need = verify_attn_workspace_size(B, max_k, Hq, Hkv, D, max_seq_len)
    if workspace is None and need > 0:
        workspace = _workspace("attn", q.device, need)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.spec_verify_attn_ragged(_need(q, torch.bfloat16, "q"), _need(k_cache, torch.bfloat16, "k_cache"),
                                       _need(v_cache, torch.bfloat16, "v_cache"),
                                       _need(block_table, torch.int32, "block_table"),
                                       _need(seq_lens, torch.int32, "seq_lens"), _need(cu_drafts, torch.int32, "cu_drafts"),
                                       _need(out, torch.bfloat16, "out"),
                                       B, int(max_k), Hq, Hkv, D, bs, max_blocks, NB, int(max_seq_len), scale,
                                       wptr, wbytes, _stream_handle(stream)), "spec_verify_attn_ragged")
    return out


def reject_sample_ragged(target_logits, draft_logits, draft_tokens, cu_drafts, seq_ids, seq_lens, max_k: int,
                         temperature: float, seed: int, out_tokens, num_accepted, out_probs=None, accept_probs=None,
                         workspace=None, stream=None):
    """spec_reject_sample_ragged. target fp32 [T][V], out_tokens int32 [T], out_probs fp32 [T]
    (T = cu_drafts[B] + B); draft fp32 [K][V], draft_tokens int32 [K], accept_probs fp32 [K]
    (K = cu_drafts[B]); cu_drafts int32 [B+1] on the device; max_k >= every k_b."""
    import torch
    V = target_logits.shape[1]
    B = seq_ids.shape[0]
    lib = library()
    need = reject_sample_workspace_size(B, max_k, V)
    if workspace is None:
        workspace = _workspace("reject", target_logits.device, need)
    if max_k == 0 or draft_logits is None or draft_logits.numel() == 0:
        draft_logits = draft_tokens = None
    if accept_probs is not None and accept_probs.numel() == 0:
        accept_probs = None
    _check(lib.spec_reject_sample_ragged(_need(target_logits, torch.float32, "target_logits"),
                                         _opt(draft_logits, torch.float32, "draft_logits"),
                                         _opt(draft_tokens, torch.int32, "draft_tokens"),
                                         _need(cu_drafts, torch.int32, "cu_drafts"),
                                         _need(seq_ids, torch.int64, "seq_ids"), _need(seq_lens, torch.int32, "seq_lens"),
                                         B, int(max_k), V, float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF,
                                         _need(out_tokens, torch.int32, "out_tokens"),
                                         _need(num_accepted, torch.int32, "num_accepted"),
                                         _opt(out_probs, torch.float32, "out_probs"),
                                         _opt(accept_probs, torch.float32, "accept_probs"),
                                         workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                         _stream_handle(stream)), "spec_reject_sample_ragged")
    return out_tokens, num_accepted


def verify_attn_tree(q, k_cache, v_cache, block_table, seq_lens, parents, out, max_seq_len: int,
                     sm_scale: float | None = None, workspace=None, stream=None):
    """spec_verify_attn_tree. q/out bf16 [B][N+1][Hq][D] (node n's row; the cache holds the KV of
    nodes 0 .. N at slots L_b .. L_b + N); parents int32 [B][N] on the device."""
    import torch
    B, N1, Hq, D = q.shape
    NB, Hkv, bs, _ = k_cache.shape
    max_blocks = block_table.shape[1]
    scale = (1.0 / D ** 0.5) if sm_scale is None else float(sm_scale)
    lib = library()
    need = verify_attn_workspace_size(B, N1 - 1, Hq, Hkv, D, max_seq_len)
    if workspace is None and need > 0:
        workspace = _workspace("attn", q.device, need)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.spec_verify_attn_tree(_need(q, torch.bfloat16, "q"), _need(k_cache, torch.bfloat16, "k_cache"),
                                     _need(v_cache, torch.bfloat16, "v_cache"),
                                     _need(block_table, torch.int32, "block_table"),
                                     _need(seq_lens, torch.int32, "seq_lens"), _need(parents, torch.int32, "parents"),
                                     _need(out, torch.bfloat16, "out"),
                                     B, N1 - 1, Hq, Hkv, D, bs, max_blocks, NB, int(max_seq_len), scale,
                                     wptr, wbytes, _stream_handle(stream)), "spec_verify_attn_tree")
    return out


def reject_sample_tree_workspace_size(B, nodes, V) -> int:
    n = _c_size(0)
    _check(library().spec_reject_sample_tree_workspace_size(B, nodes, V, ctypes.byref(n)),
           "spec_reject_sample_tree_workspace_size")
    return n.value


def reject_sample_tree(target_logits, draft_logits, draft_tokens, parents, seq_ids, seq_lens, temperature: float,
                       seed: int, out_tokens, num_accepted, accepted_nodes=None, out_probs=None, accept_probs=None,
                       workspace=None, stream=None):
    """spec_reject_sample_tree. target / draft fp32 [B][N+1][V] (one row per node); draft_tokens,
    parents int32 [B][N]; out_tokens int32 [B][N+1]; accepted_nodes int32 [B][N]; out_probs fp32
    [B][N+1]; accept_probs fp32 [B][N]."""
    import torch
    B, N1, V = target_logits.shape
    lib = library()
    need = reject_sample_tree_workspace_size(B, N1 - 1, V)
    if workspace is None:
        workspace = _workspace("reject_tree", target_logits.device, need)
    _check(lib.spec_reject_sample_tree(_need(target_logits, torch.float32, "target_logits"),
                                       _need(draft_logits, torch.float32, "draft_logits"),
                                       _need(draft_tokens, torch.int32, "draft_tokens"),
                                       _need(parents, torch.int32, "parents"),
                                       _need(seq_ids, torch.int64, "seq_ids"), _need(seq_lens, torch.int32, "seq_lens"),
                                       B, N1 - 1, V, float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF,
                                       _need(out_tokens, torch.int32, "out_tokens"),
                                       _need(num_accepted, torch.int32, "num_accepted"),
                                       _opt(accepted_nodes, torch.int32, "accepted_nodes"),
                                       _opt(out_probs, torch.float32, "out_probs"),
                                       _opt(accept_probs, torch.float32, "accept_probs"),
                                       workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                       _stream_handle(stream)), "spec_reject_sample_tree")
    return out_tokens, num_accepted


def reject_sample(target_logits, draft_logits, draft_tokens, seq_ids, seq_lens, temperature: float, seed: int,
                  out_tokens, num_accepted, out_probs=None, accept_probs=None, workspace=None, stream=None):
    """spec_reject_sample. target fp32 [B][k+1][V]; draft fp32 [B][k][V]; draft_tokens int32 [B][k];
    seq_ids int64 [B]; seq_lens int32 [B]; outputs as in include/specverify.h.

    k = 0 (plain decoding) reads no draft data: draft_logits, draft_tokens and
    accept_probs may then be None (or empty) and are passed as NULL."""
    import torch
    B, k1, V = target_logits.shape
    k = k1 - 1
    if k == 0:
        draft_logits = draft_tokens = accept_probs = None
    lib = library()
    need = reject_sample_workspace_size(B, k, V)
    if workspace is None:
        workspace = _workspace("reject", target_logits.device, need)
    _check(lib.spec_reject_sample(_need(target_logits, torch.float32, "target_logits"),
                                  _opt(draft_logits, torch.float32, "draft_logits"),
                                  _opt(draft_tokens, torch.int32, "draft_tokens"),
                                  _need(seq_ids, torch.int64, "seq_ids"), _need(seq_lens, torch.int32, "seq_lens"),
                                  B, k, V, float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF,
                                  _need(out_tokens, torch.int32, "out_tokens"),
                                  _need(num_accepted, torch.int32, "num_accepted"),
                                  _opt(out_probs, torch.float32, "out_probs"),
                                  _opt(accept_probs, torch.float32, "accept_probs"),
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  _stream_handle(stream)), "spec_reject_sample")
    return out_tokens, num_accepted


def reject_workspace(device, kind: str = "reject"):
    """The binding's own workspace for the sampling calls on `device` (kind "reject" for
    spec_reject_sample and _ragged, "reject_tree" for the tree walk), or None if no call
    has made one yet."""
    return _workspaces.get((kind, str(device)))


def reject_error_flag(workspace, flag_out, stream=None):
    """spec_reject_error_flag: copy the sampling workspace's error word into flag_out (int32
    device tensor of one element) and clear it. Nonzero iff some sequence of a call since the
    last read reported num_accepted = -1."""
    import torch
    if flag_out.numel() < 1:
        raise ValueError("flag_out needs one element")
    _check(library().spec_reject_error_flag(_need(workspace, torch.uint8, "workspace"),
                                            _need(flag_out, torch.int32, "flag_out"), _stream_handle(stream)),
           "spec_reject_error_flag")
    return flag_out


def reject_sample_noalloc(target_logits, draft_logits, draft_tokens, seq_ids, seq_lens, temperature: float,
                          seed: int, out_tokens, num_accepted, out_probs=None, accept_probs=None, stream=None):
    """spec_reject_sample_noalloc: spec_reject_sample on the library's own 16 MiB workspace (one per
    GPU; calls that overlap on one GPU race on it). Arguments as for reject_sample."""
    import torch
    B, k1, V = target_logits.shape
    k = k1 - 1
    if k == 0:
        draft_logits = draft_tokens = accept_probs = None
    _check(library().spec_reject_sample_noalloc(_need(target_logits, torch.float32, "target_logits"),
                                                _opt(draft_logits, torch.float32, "draft_logits"),
                                                _opt(draft_tokens, torch.int32, "draft_tokens"),
                                                _need(seq_ids, torch.int64, "seq_ids"),
                                                _need(seq_lens, torch.int32, "seq_lens"),
                                                B, k, V, float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF,
                                                _need(out_tokens, torch.int32, "out_tokens"),
                                                _need(num_accepted, torch.int32, "num_accepted"),
                                                _opt(out_probs, torch.float32, "out_probs"),
                                                _opt(accept_probs, torch.float32, "accept_probs"),
                                                _stream_handle(stream)), "spec_reject_sample_noalloc")
    return out_tokens, num_accepted


def commit_lengths(seq_lens, num_accepted, k: int, capacity_tokens: int, overflow_flags=None, stream=None):
    """spec_commit_lengths: seq_lens[b] += num_accepted[b] + 1 unless past capacity_tokens."""
    import torch
    B = seq_lens.shape[0]
    _check(library().spec_commit_lengths(_need(seq_lens, torch.int32, "seq_lens"),
                                         _need(num_accepted, torch.int32, "num_accepted"), B, int(k),
                                         int(capacity_tokens), _opt(overflow_flags, torch.int32, "overflow_flags"),
                                         _stream_handle(stream)), "spec_commit_lengths")
    return seq_lens


def commit_tree(k_cache, v_cache, block_table, seq_lens, accepted_nodes, num_accepted, capacity_tokens: int,
                overflow_flags=None, stream=None):
    """spec_commit_tree: move the accepted path's KV rows to L+1 .. L+a, then seq_lens[b] += a + 1
    unless past capacity_tokens. accepted_nodes int32 [B][N] as written by reject_sample_tree."""
    import torch
    B, N = accepted_nodes.shape
    NB, Hkv, bs, D = k_cache.shape
    _check(library().spec_commit_tree(_need(k_cache, torch.bfloat16, "k_cache"),
                                      _need(v_cache, torch.bfloat16, "v_cache"),
                                      _need(block_table, torch.int32, "block_table"),
                                      _need(seq_lens, torch.int32, "seq_lens"),
                                      _need(accepted_nodes, torch.int32, "accepted_nodes"),
                                      _need(num_accepted, torch.int32, "num_accepted"), B, N, Hkv, D, bs,
                                      block_table.shape[1], NB, int(capacity_tokens),
                                      _opt(overflow_flags, torch.int32, "overflow_flags"), _stream_handle(stream)),
           "spec_commit_tree")
    return seq_lens


def rope_append(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, rope_theta: float, parents=None,
                stream=None):
    """spec_rope_append: rotate q (in place) and k_new by RoPE at each row's position, then write the
    rotated K and v_new into cache slots L_b + i. q bf16 [B][k+1][Hq][D]; k_new / v_new bf16
    [B][k+1][Hkv][D]; parents int32 [B][k] for a tree (positions by depth), else None."""
    import torch
    B, K1, Hq, D = q.shape
    NB, Hkv, bs, _ = k_cache.shape
    _check(library().spec_rope_append(_need(q, torch.bfloat16, "q"), _need(k_new, torch.bfloat16, "k_new"),
                                      _need(v_new, torch.bfloat16, "v_new"),
                                      _need(k_cache, torch.bfloat16, "k_cache"),
                                      _need(v_cache, torch.bfloat16, "v_cache"),
                                      _need(block_table, torch.int32, "block_table"),
                                      _need(seq_lens, torch.int32, "seq_lens"), _opt(parents, torch.int32, "parents"),
                                      B, K1 - 1, Hq, Hkv, D, bs, block_table.shape[1], NB, float(rope_theta),
                                      _stream_handle(stream)), "spec_rope_append")
    return q


def lm_head(hidden, weight, logits, stream=None):
    """spec_lm_head: logits fp32 [R][V] = hidden bf16 [R][H] x weight bf16 [V][H]^T."""
    import torch
    R, H = hidden.shape
    V = weight.shape[0]
    if weight.shape[1] != H or logits.numel() != R * V or logits.shape[-1] != V:
        raise ValueError("lm_head: hidden [R][H], weight [V][H] and logits [..][V] with R * V elements")
    _check(library().spec_lm_head(_need(hidden, torch.bfloat16, "hidden"), _need(weight, torch.bfloat16, "weight"),
                                  _need(logits, torch.float32, "logits"), R, H, V, _stream_handle(stream)),
           "spec_lm_head")
    return logits


def verify_step(q, k_cache, v_cache, block_table, seq_lens, attn_out, max_seq_len, target_logits, draft_logits,
                draft_tokens, seq_ids, temperature, seed, out_tokens, num_accepted, capacity_tokens,
                out_probs=None, accept_probs=None, overflow_flags=None, sm_scale=None, stream=None):
    """One verify step on one stream: attention, rejection sampling, commit.

    The logits are taken as given (the LM head between attention and sampling is
    the caller's); seq_lens is read by the first two calls and updated by the third.
    """
    verify_attn(q, k_cache, v_cache, block_table, seq_lens, attn_out, max_seq_len, sm_scale, stream=stream)
    reject_sample(target_logits, draft_logits, draft_tokens, seq_ids, seq_lens, temperature, seed, out_tokens,
                  num_accepted, out_probs, accept_probs, stream=stream)
    commit_lengths(seq_lens, num_accepted, target_logits.shape[1] - 1, capacity_tokens, overflow_flags,
                   stream=stream)
    return out_tokens, num_accepted
