"""Seeded generators for every tensor a DFlash drafter run consumes.

Recipe (the same for the oracle and the GPU path):
  * target hidden states ~ N(0, 1); matrices ~ N(0, w_std); gains = 1, or
    1 + N(0, gain_std) for parity variants that must catch a dropped gain;
  * bf16 workloads round every draw to bfloat16 (round to nearest even) once,
    so both sides see identical values; fp32 workloads keep the fp32 draw;
  * anchors ~ U{0..V-2}; the mask token id is V-1;
  * synthetic target tokens per drafting iteration: position j of sequence b
    matches the draft with probability p_j, otherwise it is the draft shifted by
    r ~ U{1..V-1} (mod V); the bonus token is U{0..V-1};
  * sampled decoding: uniforms strictly inside (0, 1) of the form
    (2k + 1) * 2**-24, k ~ U{0..2**23-1} (exact in float32, never 0 or 1), one
    per (row, vocabulary entry) for the draft draws, one per draft for the
    accept tests and one per (sequence, vocabulary entry) for the emitted
    token; synthetic target logits are the draft logits plus N(0, 0.5^2) noise
    at each draft position (per-position acceptance 2 Phi(-0.25 / T), 0.80 at
    T = 1) and N(0, 1) at the bonus position.

Large tensors are drawn in 4M-element chunks, each from its own
``SeedSequence([base_seed, config_id, tensor_id, chunk])``, on a thread pool.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import BASE_SEED, Config

CHUNK = 1 << 22

# tensor ids (seed namespaces)
T_CTX = 1            # 1..n_tgt: context target states, one per tapped layer
T_WC, T_GC = 10, 11
T_GFINAL, T_EMBED = 20, 21
T_ANCHOR = 30
T_APPEND = 40        # + iteration
T_MATCH = 60         # + iteration
T_LAYER = 100        # + 10*layer + {0: qkv, 1: o, 2: gateup, 3: down, 4: g_attn, 5: g_ffn}
T_OVERRIDE = 5000    # + gamma
T_SAMPLE = 7000      # + 100 * gamma + 10 * iteration + {0: draws, 1: accept, 2: emit, 3: noise, 4: logits, 5: ids, 6: h}


def bf16_round_f32(a: np.ndarray) -> np.ndarray:
    """Round an fp32 array to bfloat16 (nearest even) in place; returns it."""
    assert a.dtype == np.float32 and a.flags.c_contiguous
    b = a.view(np.uint32).reshape(-1)
    t = b >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    b += t
    b &= np.uint32(0xFFFF0000)
    return a


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(seed_key: tuple, shape, std: float, mean: float, bf16: bool) -> np.ndarray:
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32)

    def fill(c: int):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_key) + [c])))
        o = out[lo:hi]
        rng.standard_normal(out=o, dtype=np.float32)
        if std != 1.0:
            o *= np.float32(std)
        if mean != 0.0:
            o += np.float32(mean)
        if bf16:
            bf16_round_f32(o)

    nch = (n + CHUNK - 1) // CHUNK
    if nch <= 1:
        for c in range(nch):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nch)))
    return out.reshape(shape)


def _uniform_open(seed_key: tuple, shape) -> np.ndarray:
    """float32 uniforms (2k + 1) * 2**-24 with k ~ U{0..2**23-1}: strictly inside (0, 1)."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32)

    def fill(c: int):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_key) + [c])))
        k = rng.integers(0, 1 << 23, size=hi - lo, dtype=np.int32)
        out[lo:hi] = (2 * k + 1).astype(np.float32) * np.float32(2.0 ** -24)

    nch = (n + CHUNK - 1) // CHUNK
    if nch <= 1:
        for c in range(nch):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nch)))
    return out.reshape(shape)


def build_target_logits_np(draft_logits: np.ndarray, noise: np.ndarray, sigma: float = 0.5) -> np.ndarray:
    """Synthetic target logits [B, n+1, V] (harness, not method): the draft logits
    plus sigma * noise at the n draft positions, the noise itself at the bonus."""
    z = np.asarray(draft_logits, dtype=np.float32)
    t = np.array(noise, dtype=np.float32, copy=True)
    t[:, :-1] *= np.float32(sigma)
    t[:, :-1] += z
    return t


def build_target_np(draft: np.ndarray, match: np.ndarray, r: np.ndarray,
                    bonus: np.ndarray, V: int) -> np.ndarray:
    """Synthetic target tokens [B, n+1] from drafts [B, n] (harness, not method)."""
    d = draft.astype(np.int64)
    t = np.where(match, d, (d + r.astype(np.int64)) % V)
    return np.concatenate([t, bonus.astype(np.int64)[:, None]], axis=1).astype(np.int32)


class Inputs:
    """Lazily generated, seeded inputs of one workload.

    All floating tensors come back as C-contiguous float32 numpy arrays whose
    values are exactly representable in the workload's storage type.
    """

    def __init__(self, cfg: Config, base_seed: int = BASE_SEED):
        self.cfg = cfg
        self.base = base_seed
        self.bf16 = cfg.dtype == "bf16"

    # -- helpers -----------------------------------------------------------
    def _key(self, tid: int) -> tuple:
        return (self.base, self.cfg.cid, tid)

    def _rng(self, tid: int) -> np.random.Generator:
        return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(self._key(tid)) + [0])))

    def _w(self, tid: int, shape) -> np.ndarray:
        return _normal(self._key(tid), shape, self.cfg.w_std, 0.0, self.bf16)

    def _gain(self, tid: int, n: int) -> np.ndarray:
        c = self.cfg
        if c.gain_std == 0.0:
            return np.ones(n, dtype=np.float32)
        return _normal(self._key(tid), (n,), c.gain_std, 1.0, self.bf16)

    # -- context -------------------------------------------------------------
    def ctx_states(self) -> list:
        """n_tgt arrays [sum(ctx), D] ~ N(0,1): the tapped target hidden states."""
        c = self.cfg
        return [_normal(self._key(T_CTX + k), (c.n_ctx_total, c.D), 1.0, 0.0, self.bf16)
                for k in range(c.n_tgt)]

    def append_states(self, it: int) -> list:
        """n_tgt arrays [B*append_rows, D] for drafting iteration ``it``."""
        c = self.cfg
        a = _normal(self._key(T_APPEND + it), (c.n_tgt, c.B * c.append_rows, c.D), 1.0, 0.0, self.bf16)
        return [np.ascontiguousarray(a[k]) for k in range(c.n_tgt)]

    # -- weights -------------------------------------------------------------
    def w_c(self) -> np.ndarray:
        c = self.cfg
        return self._w(T_WC, (c.D, c.n_tgt * c.D))

    def g_c(self) -> np.ndarray:
        return self._gain(T_GC, self.cfg.D)

    def w_qkv(self, l: int) -> np.ndarray:
        c = self.cfg
        return self._w(T_LAYER + 10 * l + 0, ((c.Hq + 2 * c.Hkv) * c.d, c.D))

    def w_o(self, l: int) -> np.ndarray:
        c = self.cfg
        return self._w(T_LAYER + 10 * l + 1, (c.D, c.Hq * c.d))

    def w_gateup(self, l: int) -> np.ndarray:
        c = self.cfg
        return self._w(T_LAYER + 10 * l + 2, (2 * c.F, c.D))

    def w_down(self, l: int) -> np.ndarray:
        c = self.cfg
        return self._w(T_LAYER + 10 * l + 3, (c.D, c.F))

    def g_attn(self, l: int) -> np.ndarray:
        return self._gain(T_LAYER + 10 * l + 4, self.cfg.D)

    def g_ffn(self, l: int) -> np.ndarray:
        return self._gain(T_LAYER + 10 * l + 5, self.cfg.D)

    def g_final(self) -> np.ndarray:
        return self._gain(T_GFINAL, self.cfg.D)

    def embed(self) -> np.ndarray:
        """Tied embedding / LM-head table [V, D]."""
        c = self.cfg
        return self._w(T_EMBED, (c.V, c.D))

    # -- tokens ----------------------------------------------------------------
    def anchors(self) -> np.ndarray:
        c = self.cfg
        return self._rng(T_ANCHOR).integers(0, c.V - 1, size=c.B).astype(np.int32)

    def block_tokens(self, gamma: int, anchors=None) -> np.ndarray:
        """[B, gamma] int32: anchor at row 0, mask id elsewhere."""
        c = self.cfg
        a = self.anchors() if anchors is None else np.asarray(anchors, dtype=np.int32)
        t = np.full((c.B, gamma), c.mask_id, dtype=np.int32)
        t[:, 0] = a
        return t

    def embed_override(self, gamma: int) -> np.ndarray:
        """[B, gamma, D] ~ N(0,1) distinct block rows (used instead of embeddings)."""
        c = self.cfg
        return _normal(self._key(T_OVERRIDE + gamma), (c.B, gamma, c.D), 1.0, 0.0, False)

    def verify_draws(self, it: int, gamma: int):
        """(match [B,n] bool, r [B,n] int, bonus [B] int) for iteration ``it``."""
        c = self.cfg
        n = gamma - 1
        rng = self._rng(T_MATCH + 1000 * gamma + it)
        u = rng.random((c.B, n))
        match = u < c.match_probs(gamma)[None, :]
        r = rng.integers(1, c.V, size=(c.B, n))
        bonus = rng.integers(0, c.V, size=c.B)
        return match, r, bonus

    # -- sampled decoding ------------------------------------------------------
    def _skey(self, gamma: int, it: int, kind: int) -> tuple:
        return self._key(T_SAMPLE + 100 * gamma + 10 * it + kind)

    def sample_uniforms(self, it: int, gamma: int):
        """(draws [B, n, V], accept [B, n], emit [B, V]) float32 uniforms in (0, 1)."""
        c = self.cfg
        n = gamma - 1
        return (_uniform_open(self._skey(gamma, it, 0), (c.B, n, c.V)),
                _uniform_open(self._skey(gamma, it, 1), (c.B, n)),
                _uniform_open(self._skey(gamma, it, 2), (c.B, c.V)))

    def target_noise(self, it: int, gamma: int) -> np.ndarray:
        """[B, n+1, V] float32 ~ N(0, 1) for synthetic target logits."""
        c = self.cfg
        return _normal(self._skey(gamma, it, 3), (c.B, gamma, c.V), 1.0, 0.0, False)

    def synthetic_logits(self, it: int, gamma: int, std: float) -> np.ndarray:
        """[B, n, V] float32 ~ N(0, std^2): stand-in draft logits for verify-only tests."""
        c = self.cfg
        return _normal(self._skey(gamma, it, 4), (c.B, gamma - 1, c.V), std, 0.0, False)

    def random_ids(self, it: int, gamma: int) -> np.ndarray:
        """[B, n] int32 ~ U{0..V-1}: stand-in drafts for verify-only tests."""
        c = self.cfg
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(self._skey(gamma, it, 5)) + [0])))
        return rng.integers(0, c.V, size=(c.B, gamma - 1)).astype(np.int32)

    def final_states(self, gamma: int) -> np.ndarray:
        """[B, gamma, D] float32 ~ N(0, 1): stand-in h_final rows (unit RMS on
        average, like the drafter's final RMSNorm output) for LM-head tests."""
        c = self.cfg
        return _normal(self._skey(gamma, 0, 6), (c.B, gamma, c.D), 1.0, 0.0, False)
