"""ctypes binding of libdflash (include/dflash.h): argument marshalling only.

Every function takes raw device pointers (ints), sizes and a HIP stream handle,
and raises DFlashError on a non-OK status.  The library must have been built
(``__graft_entry__.build()``); loading fails loudly otherwise: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_uint32, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdflash.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1
ARGMAX, ACCEPT = 1, 2
MAX_BATCH, MAX_TGT_LAYERS, MIN_GAMMA, MAX_GAMMA = 64, 8, 2, 33

EXPORTED = ("dflash_version", "dflash_last_error", "dflash_workspace_size", "dflash_fuse_context",
            "dflash_inject_kv", "dflash_draft_forward", "dflash_draft_forward_noalloc",
            "dflash_draft_forward_ragged",
            "dflash_draft_forward_blocks", "dflash_argmax_accept",
            "dflash_argmax_accept_ragged", "dflash_target_verify", "dflash_sample_drafts",
            "dflash_sample_accept", "dflash_profile_events")
(PROF_NONE, PROF_LM_HEAD, PROF_QKV, PROF_O, PROF_GATEUP, PROF_DOWN, PROF_FUSE, PROF_INJECT, PROF_ATTENTION,
 PROF_ROW_STATS, PROF_VERIFY) = range(11)


class Dims(ctypes.Structure):
    _fields_ = [("D", c_int32), ("L", c_int32), ("Hq", c_int32), ("Hkv", c_int32),
                ("head_dim", c_int32), ("F", c_int32), ("V", c_int32), ("n_tgt_layers", c_int32),
                ("mask_id", c_int32), ("rms_eps", c_float), ("dtype", c_int32), ("cache_dtype", c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("w_c", "g_c", "w_qkv", "w_o", "w_gateup", "w_down",
                                        "g_attn", "g_ffn", "g_final", "embed", "lm_head")]


class KVCache(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("B", c_int32), ("cap", c_int32),
                ("len", POINTER(c_int32)), ("len_dev", c_void_p)]


class DFlashError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"dflash status {status}: {msg}")
        self.status = status


_lib = None


def load():
    """Load libdflash.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.dflash_version.restype = c_char_p
    lib.dflash_version.argtypes = []
    lib.dflash_last_error.restype = c_char_p
    lib.dflash_last_error.argtypes = []
    lib.dflash_workspace_size.restype = c_int32
    lib.dflash_workspace_size.argtypes = [POINTER(Dims), c_int32, c_int32, c_int32, POINTER(c_size_t)]
    lib.dflash_fuse_context.restype = c_int32
    lib.dflash_fuse_context.argtypes = [POINTER(Dims), POINTER(Weights), POINTER(c_void_p), c_int64, c_int32,
                                        c_void_p, c_void_p, c_size_t, c_void_p]
    lib.dflash_inject_kv.restype = c_int32
    lib.dflash_inject_kv.argtypes = [POINTER(Dims), POINTER(Weights), c_void_p, POINTER(c_int32),
                                     POINTER(KVCache), c_void_p, c_size_t, c_void_p]
    lib.dflash_draft_forward.restype = c_int32
    lib.dflash_draft_forward.argtypes = [POINTER(Dims), POINTER(Weights), POINTER(KVCache), c_void_p, c_void_p,
                                         c_int32, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.dflash_draft_forward_noalloc.restype = c_int32
    lib.dflash_draft_forward_noalloc.argtypes = [POINTER(Dims), POINTER(Weights), POINTER(KVCache), c_void_p,
                                                 c_void_p, c_int32, c_void_p, c_void_p]
    lib.dflash_target_verify.restype = c_int32
    lib.dflash_target_verify.argtypes = [POINTER(Dims), POINTER(Weights), POINTER(KVCache), c_void_p, c_int32,
                                         POINTER(c_int32), POINTER(c_void_p), c_void_p, c_void_p, c_void_p,
                                         c_size_t, c_void_p]
    lib.dflash_argmax_accept.restype = c_int32
    lib.dflash_argmax_accept.argtypes = [POINTER(Dims), POINTER(Weights), c_uint32, c_void_p, c_int32, c_int32,
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_size_t, c_void_p]
    lib.dflash_draft_forward_ragged.restype = c_int32
    lib.dflash_draft_forward_ragged.argtypes = [POINTER(Dims), POINTER(Weights), POINTER(KVCache), c_void_p,
                                                c_void_p, POINTER(c_int32), c_void_p, c_void_p, c_size_t, c_void_p]
    lib.dflash_draft_forward_blocks.restype = c_int32
    lib.dflash_draft_forward_blocks.argtypes = [POINTER(Dims), POINTER(Weights), POINTER(KVCache), POINTER(c_int32),
                                                POINTER(c_int32), c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                                c_void_p, c_size_t, c_void_p]
    lib.dflash_argmax_accept_ragged.restype = c_int32
    lib.dflash_argmax_accept_ragged.argtypes = [POINTER(Dims), POINTER(Weights), c_uint32, c_void_p, c_int32,
                                                POINTER(c_int32), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                                c_void_p, c_void_p, c_size_t, c_void_p]
    lib.dflash_sample_drafts.restype = c_int32
    lib.dflash_sample_drafts.argtypes = [POINTER(Dims), POINTER(Weights), c_void_p, c_int32, c_int32, c_float,
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.dflash_sample_accept.restype = c_int32
    lib.dflash_sample_accept.argtypes = [POINTER(Dims), c_int32, c_int32, c_float, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                         c_void_p]
    lib.dflash_profile_events.restype = c_int32
    lib.dflash_profile_events.argtypes = [c_int32, POINTER(c_void_p), POINTER(c_void_p), c_int32, POINTER(c_int32)]
    _lib = lib
    return lib


def version() -> str:
    return load().dflash_version().decode()


def last_error() -> str:
    return load().dflash_last_error().decode()


def _check(st: int):
    if st != OK:
        raise DFlashError(st, last_error())


def _p(x):
    return None if x is None or x == 0 else c_void_p(int(x))


def workspace_size(dims: Dims, B: int, gamma: int, max_rows: int) -> int:
    out = c_size_t(0)
    _check(load().dflash_workspace_size(ctypes.byref(dims), B, gamma, max_rows, ctypes.byref(out)))
    return out.value


def fuse_context(dims: Dims, w: Weights, h_tgt, ld: int, T: int, H_t, ws, ws_bytes: int, stream=0):
    arr = (c_void_p * max(1, len(h_tgt)))(*[int(p) for p in h_tgt])
    _check(load().dflash_fuse_context(ctypes.byref(dims), ctypes.byref(w), arr, ld, T, _p(H_t), _p(ws),
                                      ws_bytes, _p(stream)))


def inject_kv(dims: Dims, w: Weights, H_t, rows_per_seq, cache: KVCache, ws, ws_bytes: int, stream=0):
    rows = (c_int32 * max(1, len(rows_per_seq)))(*rows_per_seq)
    _check(load().dflash_inject_kv(ctypes.byref(dims), ctypes.byref(w), _p(H_t), rows, ctypes.byref(cache),
                                   _p(ws), ws_bytes, _p(stream)))


def draft_forward(dims: Dims, w: Weights, cache: KVCache, block_tokens, embed_override, gamma: int, h_final,
                  ws, ws_bytes: int, stream=0):
    _check(load().dflash_draft_forward(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(cache),
                                       _p(block_tokens), _p(embed_override), gamma, _p(h_final), _p(ws),
                                       ws_bytes, _p(stream)))


def argmax_accept(dims: Dims, w: Weights, flags: int, h_final, B: int, gamma: int, draft, target, tau,
                  next_anchor, logits_dbg, top2_gap, ws, ws_bytes: int, stream=0):
    _check(load().dflash_argmax_accept(ctypes.byref(dims), ctypes.byref(w) if w is not None else None, flags,
                                       _p(h_final), B, gamma, _p(draft), _p(target), _p(tau), _p(next_anchor),
                                       _p(logits_dbg), _p(top2_gap), _p(ws), ws_bytes, _p(stream)))


def _gammas(gammas):
    return (c_int32 * max(1, len(gammas)))(*[int(g) for g in gammas])


def draft_forward_noalloc(dims: Dims, w: Weights, cache: KVCache, block_tokens, embed_override, gamma: int,
                          h_final, stream=0):
    _check(load().dflash_draft_forward_noalloc(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(cache),
                                               _p(block_tokens), _p(embed_override), gamma, _p(h_final),
                                               _p(stream)))


def target_verify(dims: Dims, w: Weights, cache: KVCache, block_tokens, gamma: int, tap_layers, taps,
                  target_tokens, top2_gap, ws, ws_bytes: int, stream=0):
    n = len(tap_layers)
    tl = (c_int32 * max(n, 1))(*[int(x) for x in tap_layers])
    tp = (c_void_p * max(n, 1))(*[int(t) if t else None for t in taps])
    _check(load().dflash_target_verify(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(cache), _p(block_tokens),
                                       gamma, tl, tp, _p(target_tokens), _p(top2_gap), _p(ws), ws_bytes,
                                       _p(stream)))


def draft_forward_ragged(dims: Dims, w: Weights, cache: KVCache, block_tokens, embed_override, gammas, h_final,
                         ws, ws_bytes: int, stream=0):
    _check(load().dflash_draft_forward_ragged(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(cache),
                                              _p(block_tokens), _p(embed_override), _gammas(gammas), _p(h_final),
                                              _p(ws), ws_bytes, _p(stream)))


def draft_forward_blocks(dims: Dims, w: Weights, cache: KVCache, block_seq, anchors, gamma: int, block_tokens,
                         embed_override, h_final, ws, ws_bytes: int, stream=0):
    n = len(anchors)
    _check(load().dflash_draft_forward_blocks(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(cache),
                                              _gammas(block_seq), _gammas(anchors), n, gamma, _p(block_tokens),
                                              _p(embed_override), _p(h_final), _p(ws), ws_bytes, _p(stream)))


def argmax_accept_ragged(dims: Dims, w: Weights, flags: int, h_final, gammas, draft, target, tau, next_anchor,
                         logits_dbg, top2_gap, ws, ws_bytes: int, stream=0):
    _check(load().dflash_argmax_accept_ragged(ctypes.byref(dims), ctypes.byref(w) if w is not None else None,
                                              flags, _p(h_final), len(gammas), _gammas(gammas), _p(draft),
                                              _p(target), _p(tau), _p(next_anchor), _p(logits_dbg), _p(top2_gap),
                                              _p(ws), ws_bytes, _p(stream)))


def sample_drafts(dims: Dims, w: Weights, h_final, B: int, gamma: int, temperature: float, uniforms, draft,
                  logits, lse, ws, ws_bytes: int, stream=0):
    _check(load().dflash_sample_drafts(ctypes.byref(dims), ctypes.byref(w) if w is not None else None,
                                       _p(h_final), B, gamma, temperature, _p(uniforms), _p(draft), _p(logits),
                                       _p(lse), _p(ws), ws_bytes, _p(stream)))


def sample_accept(dims: Dims, B: int, gamma: int, temperature: float, draft, draft_logits, draft_lse,
                  target_logits, accept_u, resid_u, tau, next_anchor, ws, ws_bytes: int, stream=0):
    _check(load().dflash_sample_accept(ctypes.byref(dims), B, gamma, temperature, _p(draft), _p(draft_logits),
                                       _p(draft_lse), _p(target_logits), _p(accept_u), _p(resid_u), _p(tau),
                                       _p(next_anchor), _p(ws), ws_bytes, _p(stream)))


_prof_keep = None


def profile_events(role: int, starts=(), stops=()) -> int:
    """Record HIP events around the next len(starts) launches of a kernel role
    (handles as ints, e.g. torch.cuda.Event.cuda_event).  Returns the number of
    launches recorded under the previous setting."""
    global _prof_keep
    n = len(starts)
    a = (c_void_p * max(1, n))(*[int(x) for x in starts])
    b = (c_void_p * max(1, n))(*[int(x) for x in stops])
    rec = c_int32(0)
    _check(load().dflash_profile_events(role, a, b, n, ctypes.byref(rec)))
    _prof_keep = (a, b)
    return rec.value
