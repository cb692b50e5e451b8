"""PyTorch plumbing around the C ABI: device weights, KV cache and workspace.

PyTorch only allocates device memory and provides the stream; every step of the
hot path runs in libdflash's HIP kernels through ``binding``.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import binding as B


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def dims_of(cfg) -> B.Dims:
    return B.Dims(D=cfg.D, L=cfg.L, Hq=cfg.Hq, Hkv=cfg.Hkv, head_dim=cfg.d, F=cfg.F, V=cfg.V,
                  n_tgt_layers=cfg.n_tgt, mask_id=cfg.V - 1, rms_eps=cfg.eps,
                  dtype=B.BF16 if cfg.dtype == "bf16" else B.F32,
                  cache_dtype=B.BF16 if cfg.cache_dtype == "bf16" else B.F32)


def tap_layers(L_t: int, n: int = 5) -> list:
    """0-based indices of the target layers whose hidden states the drafter
    fuses: n layers spread evenly from the target's second layer to its
    third-from-last ("DFlash: Block Diffusion for Flash Speculative Decoding
    논문 정리", section "실험 설정", settings table; "ICML'26 | DFlash", section
    3.1), a fractional position rounded half up (integer arithmetic)."""
    if n < 2:
        return [1]
    span = L_t - 4
    return [1 + (2 * k * span + (n - 1)) // (2 * (n - 1)) for k in range(n)]


def torch_dtype(cfg):
    """Weight / target-state type."""
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def cache_torch_dtype(cfg):
    """Type of H_t and the KV cache."""
    return torch.bfloat16 if cfg.cache_dtype == "bf16" else torch.float32


def upload(arr: np.ndarray, cfg, device="cuda") -> torch.Tensor:
    """fp32 numpy (values exact in the storage type) -> device tensor of the storage type."""
    t = torch.from_numpy(np.ascontiguousarray(arr)).to(device)
    return t.to(torch_dtype(cfg)) if cfg.dtype == "bf16" else t


def k_frag_perm(d: int) -> np.ndarray:
    """For a bf16 cache's 32-key K block: perm[i * d + c] = position of (key i,
    dimension c) in the stored block (the attention's score-fragment order:
    fragment ((i % 8) // 4) * (d // 32) + c // 32 of 512 elements, lane
    16 ((c % 32) // 8) + 4 (i // 8) + i % 4 of it, 8 dimensions per lane)."""
    i = np.arange(32)[:, None]
    c = np.arange(d)[None, :]
    f = ((i % 8) // 4) * (d // 32) + c // 32
    lane = 16 * ((c % 32) // 8) + 4 * (i // 8) + i % 4
    return (f * 512 + lane * 8 + c % 8).reshape(-1)


class DeviceCache:
    """KV cache.  fp32: keys [L][B][Hkv][cap][d], values transposed
    [L][B][Hkv][d][cap].  bf16: per block of 32 keys, keys [L][B][Hkv][cap/32][32*d]
    in the attention's fragment order (k_frag_perm) and values
    [L][B][Hkv][cap/32][d][32].  Also the host lengths the library plans from,
    and their device mirror."""

    def __init__(self, cfg, B_: int, cap: int, device="cuda"):
        dt = cache_torch_dtype(cfg)
        self.blocked = cfg.cache_dtype == "bf16"
        self.L, self.Hkv, self.d = cfg.L, cfg.Hkv, cfg.d
        if self.blocked:
            self.k = torch.zeros(cfg.L, B_, cfg.Hkv, cap // 32, 32 * cfg.d, dtype=dt, device=device)
            self.v = torch.zeros(cfg.L, B_, cfg.Hkv, cap // 32, cfg.d, 32, dtype=dt, device=device)
            self._perm = torch.from_numpy(k_frag_perm(cfg.d)).to(device)
        else:
            self.k = torch.zeros(cfg.L, B_, cfg.Hkv, cap, cfg.d, dtype=dt, device=device)
            self.v = torch.zeros(cfg.L, B_, cfg.Hkv, cfg.d, cap, dtype=dt, device=device)
        self.len_dev = torch.zeros(B_, dtype=torch.int32, device=device)
        self.lens = (ctypes.c_int32 * B_)()
        self.B, self.cap = B_, cap
        self.struct = B.KVCache(k=self.k.data_ptr(), v=self.v.data_ptr(), B=B_, cap=cap,
                                len=ctypes.cast(self.lens, ctypes.POINTER(ctypes.c_int32)),
                                len_dev=self.len_dev.data_ptr())

    def len_list(self):
        return [int(self.lens[b]) for b in range(self.B)]

    def set_lens(self, lens, mirror: bool = True):
        """Set the host lengths (what the library plans from) and, unless
        ``mirror`` is False, copy them to the device mirror (a host-to-device
        copy on the stream; an inject call rewrites the mirror itself)."""
        for b, n in enumerate(lens):
            self.lens[b] = int(n)
        if mirror:
            self.len_dev.copy_(torch.tensor(self.len_list(), dtype=torch.int32))

    # ---- the layout lives here only (tests and measurements)
    def _kt(self, b: int, lo: int, hi: int) -> torch.Tensor:
        """Keys of rows [lo, hi) of sequence b as [L][Hkv][hi - lo][d] (a view
        for an fp32 cache, a copy of the covering blocks for a bf16 one)."""
        if not self.blocked:
            return self.k[:, b, :, lo:hi]
        b0, b1 = lo // 32, (hi + 31) // 32
        blk = self.k[:, b, :, b0:b1]                       # [L][Hkv][nb][32 d] stored order
        rows = blk[..., self._perm].reshape(self.L, self.Hkv, (b1 - b0) * 32, self.d)
        return rows[:, :, lo - 32 * b0:hi - 32 * b0]

    def _put_k(self, b: int, lo: int, kt: torch.Tensor):
        """Write keys [L][Hkv][n][d] into rows [lo, lo + n) of sequence b."""
        n = kt.shape[2]
        if not self.blocked:
            self.k[:, b, :, lo:lo + n] = kt
            return
        b0, b1 = lo // 32, (lo + n + 31) // 32
        full = self._kt(b, 32 * b0, 32 * b1).clone()
        full[:, :, lo - 32 * b0:lo - 32 * b0 + n] = kt
        flat = full.reshape(self.L, self.Hkv, b1 - b0, 32 * self.d)
        stored = torch.empty_like(flat)
        stored[..., self._perm] = flat
        self.k[:, b, :, b0:b1] = stored

    def _vt(self, b: int, lo: int, hi: int) -> torch.Tensor:
        """Values of rows [lo, hi) of sequence b as V^T [L][Hkv][d][hi - lo] (a
        view for an fp32 cache, a copy of the covering blocks for a bf16 one)."""
        if not self.blocked:
            return self.v[:, b, :, :, lo:hi]
        b0, b1 = lo // 32, (hi + 31) // 32
        blk = self.v[:, b, :, b0:b1]                       # [L][Hkv][nb][d][32]
        vt = blk.permute(0, 1, 3, 2, 4).reshape(self.L, self.Hkv, self.d, (b1 - b0) * 32)
        return vt[..., lo - 32 * b0:hi - 32 * b0]

    def _put_vt(self, b: int, lo: int, vt: torch.Tensor):
        """Write V^T [L][Hkv][d][n] into rows [lo, lo + n) of sequence b."""
        n = vt.shape[-1]
        if not self.blocked:
            self.v[:, b, :, :, lo:lo + n] = vt
            return
        b0, b1 = lo // 32, (lo + n + 31) // 32
        full = self._vt(b, 32 * b0, 32 * b1).clone()
        full[..., lo - 32 * b0:lo - 32 * b0 + n] = vt
        self.v[:, b, :, b0:b1] = full.reshape(self.L, self.Hkv, self.d, b1 - b0, 32).permute(0, 1, 3, 2, 4)

    def rows(self, b: int, lo: int, hi: int):
        """Rows [lo, hi) of sequence b in every layer: (K, V) float64 numpy
        arrays [L][hi - lo][Hkv][d]."""
        k = self._kt(b, lo, hi).float().cpu().numpy().transpose(0, 2, 1, 3)
        v = self._vt(b, lo, hi).float().cpu().numpy().transpose(0, 3, 1, 2)
        return k.astype(np.float64), v.astype(np.float64)

    def put_rows(self, b: int, lo: int, k: np.ndarray, v: np.ndarray):
        """Write rows [lo, lo + n) of sequence b in every layer from (K, V)
        arrays [L][n][Hkv][d] (values exact in the cache type); lengths are
        not changed."""
        n = k.shape[1]
        kt = torch.from_numpy(np.ascontiguousarray(k.transpose(0, 2, 1, 3), dtype=np.float32))
        vt = torch.from_numpy(np.ascontiguousarray(v.transpose(0, 2, 3, 1), dtype=np.float32))
        self._put_k(b, lo, kt.to(self.k.device, self.k.dtype))
        self._put_vt(b, lo, vt.to(self.v.device, self.v.dtype))

    def fill_random(self, b: int, n: int, gen: torch.Generator):
        """Rows [0, n) of sequence b in every layer from N(0, 1) draws."""
        dev, dt = self.k.device, self.k.dtype
        self._put_k(b, 0, torch.randn(self.L, self.Hkv, n, self.d, generator=gen, device=dev).to(dt))
        self._put_vt(b, 0, torch.randn(self.L, self.Hkv, self.d, n, generator=gen, device=dev).to(dt))

    def snapshot(self, b: int, n: int):
        """A device copy of rows [0, n) of sequence b in every layer."""
        return self._kt(b, 0, n).clone(), self._vt(b, 0, n).clone()

    def same_rows(self, snap, b: int, n: int) -> bool:
        """Rows [0, n) of sequence b are bit-identical to ``snap``."""
        return torch.equal(self._kt(b, 0, n), snap[0]) and torch.equal(self._vt(b, 0, n), snap[1])


class DeviceDrafter:
    """Weights of one drafter on the device, and thin wrappers over the four calls."""

    def __init__(self, cfg, inputs, device="cuda", with_fusion=True):
        self.cfg, self.device = cfg, device
        self.dims = dims_of(cfg)
        L = cfg.L
        up = lambda a: upload(a, cfg, device)  # noqa: E731
        self.w_c = up(inputs.w_c()) if with_fusion else None
        self.g_c = up(inputs.g_c())
        dt = torch_dtype(cfg)
        self.w_qkv = torch.empty(L, (cfg.Hq + 2 * cfg.Hkv) * cfg.d, cfg.D, dtype=dt, device=device)
        self.w_o = torch.empty(L, cfg.D, cfg.Hq * cfg.d, dtype=dt, device=device)
        self.w_gateup = torch.empty(L, 2 * cfg.F, cfg.D, dtype=dt, device=device)
        self.w_down = torch.empty(L, cfg.D, cfg.F, dtype=dt, device=device)
        self.g_attn = torch.empty(L, cfg.D, dtype=dt, device=device)
        self.g_ffn = torch.empty(L, cfg.D, dtype=dt, device=device)
        for l in range(L):
            self.w_qkv[l].copy_(up(inputs.w_qkv(l)))
            self.w_o[l].copy_(up(inputs.w_o(l)))
            self.w_gateup[l].copy_(up(inputs.w_gateup(l)))
            self.w_down[l].copy_(up(inputs.w_down(l)))
            self.g_attn[l].copy_(up(inputs.g_attn(l)))
            self.g_ffn[l].copy_(up(inputs.g_ffn(l)))
        self.g_final = up(inputs.g_final())
        self.embed = up(inputs.embed())
        ptr = lambda t: 0 if t is None else t.data_ptr()  # noqa: E731
        self.weights = B.Weights(w_c=ptr(self.w_c), g_c=ptr(self.g_c), w_qkv=ptr(self.w_qkv), w_o=ptr(self.w_o),
                                 w_gateup=ptr(self.w_gateup), w_down=ptr(self.w_down), g_attn=ptr(self.g_attn),
                                 g_ffn=ptr(self.g_ffn), g_final=ptr(self.g_final), embed=ptr(self.embed),
                                 lm_head=ptr(self.embed))
        self.ws = None
        self.ws_bytes = 0

    @classmethod
    def random_init(cls, cfg, seed: int, device="cuda"):
        """Weights drawn on the device from a seeded generator (matrices
        N(0, cfg.w_std), unit gains, tied embedding / LM head), for measurements
        whose weights need not match the host-side seeded inputs."""
        self = cls.__new__(cls)
        self.cfg, self.device = cfg, device
        self.dims = dims_of(cfg)
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)
        dt = torch_dtype(cfg)

        def mat(*shape):
            return (torch.randn(*shape, generator=gen, device=device) * cfg.w_std).to(dt)

        L = cfg.L
        self.w_c = mat(cfg.D, cfg.n_tgt * cfg.D)
        self.g_c = torch.ones(cfg.D, dtype=dt, device=device)
        self.w_qkv = mat(L, (cfg.Hq + 2 * cfg.Hkv) * cfg.d, cfg.D)
        self.w_o = mat(L, cfg.D, cfg.Hq * cfg.d)
        self.w_gateup = mat(L, 2 * cfg.F, cfg.D)
        self.w_down = mat(L, cfg.D, cfg.F)
        self.g_attn = torch.ones(L, cfg.D, dtype=dt, device=device)
        self.g_ffn = torch.ones(L, cfg.D, dtype=dt, device=device)
        self.g_final = torch.ones(cfg.D, dtype=dt, device=device)
        self.embed = mat(cfg.V, cfg.D)
        p = lambda t: t.data_ptr()  # noqa: E731
        self.weights = B.Weights(w_c=p(self.w_c), g_c=p(self.g_c), w_qkv=p(self.w_qkv), w_o=p(self.w_o),
                                 w_gateup=p(self.w_gateup), w_down=p(self.w_down), g_attn=p(self.g_attn),
                                 g_ffn=p(self.g_ffn), g_final=p(self.g_final), embed=p(self.embed),
                                 lm_head=p(self.embed))
        self.ws = None
        self.ws_bytes = 0
        return self

    def with_cache_dtype(self, cache_dtype: str) -> "DeviceDrafter":
        """The same device weights with H_t and the KV cache in another type
        (its own workspace)."""
        import copy
        import dataclasses
        o = copy.copy(self)
        o.cfg = dataclasses.replace(self.cfg, cache_dtype=cache_dtype)
        o.dims = dims_of(o.cfg)
        o.ws, o.ws_bytes = None, 0
        return o

    # ---- memory
    def cache(self, B_: int, cap: int) -> DeviceCache:
        return DeviceCache(self.cfg, B_, cap, self.device)

    def ensure_workspace(self, B_: int, gamma: int, max_rows: int):
        need = B.workspace_size(self.dims, B_, gamma, max_rows)
        if need > self.ws_bytes:
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)
            self.ws_bytes = need
        return self.ws

    def context_buffer(self, T: int) -> torch.Tensor:
        """An H_t buffer [T, D] of the cache type."""
        return torch.empty(max(T, 1), self.cfg.D, dtype=cache_torch_dtype(self.cfg), device=self.device)

    # ---- the four calls
    def fuse(self, h_tgt, T: int, H_t: torch.Tensor):
        ld = h_tgt[0].stride(0)
        B.fuse_context(self.dims, self.weights, [h.data_ptr() for h in h_tgt], ld, T, H_t.data_ptr(),
                       self.ws.data_ptr() if self.ws is not None else 0, self.ws_bytes, _stream())

    def inject(self, H_t: torch.Tensor, rows_per_seq, cache: DeviceCache):
        B.inject_kv(self.dims, self.weights, H_t.data_ptr(), list(rows_per_seq), cache.struct,
                    self.ws.data_ptr() if self.ws is not None else 0, self.ws_bytes, _stream())

    def draft(self, cache: DeviceCache, tokens, override, gamma: int, h_final: torch.Tensor):
        B.draft_forward(self.dims, self.weights, cache.struct, 0 if tokens is None else tokens.data_ptr(),
                        0 if override is None else override.data_ptr(), gamma, h_final.data_ptr(),
                        self.ws.data_ptr(), self.ws_bytes, _stream())

    def argmax_accept(self, flags, h_final, B_, gamma, draft, target=None, tau=None, nxt=None, logits=None,
                      gap=None):
        p = lambda t: 0 if t is None else t.data_ptr()  # noqa: E731
        B.argmax_accept(self.dims, self.weights, flags, p(h_final), B_, gamma, p(draft), p(target), p(tau),
                        p(nxt), p(logits), p(gap), p(self.ws), self.ws_bytes, _stream())

    # ---- sampled drafting and verification (temperature T > 0)
    def sample_drafts(self, h_final, B_, gamma, temperature, uniforms, draft, logits, lse=None):
        p = lambda t: 0 if t is None else t.data_ptr()  # noqa: E731
        B.sample_drafts(self.dims, self.weights, p(h_final), B_, gamma, temperature, p(uniforms), p(draft),
                        p(logits), p(lse), p(self.ws), self.ws_bytes, _stream())

    def sample_accept(self, B_, gamma, temperature, draft, draft_logits, target_logits, accept_u, resid_u, tau,
                      nxt, draft_lse=None):
        p = lambda t: 0 if t is None else t.data_ptr()  # noqa: E731
        B.sample_accept(self.dims, B_, gamma, temperature, p(draft), p(draft_logits), p(draft_lse),
                        p(target_logits), p(accept_u), p(resid_u), p(tau), p(nxt), p(self.ws), self.ws_bytes,
                        _stream())

    # ---- the target's verify pass (this object holding a target's weights)
    def target_verify(self, cache: DeviceCache, tokens, gamma: int, tap_layers, taps, target_tokens, gap=None):
        p = lambda t: 0 if t is None else t.data_ptr()  # noqa: E731
        B.target_verify(self.dims, self.weights, cache.struct, p(tokens), gamma, list(tap_layers),
                        [t.data_ptr() for t in taps], p(target_tokens), p(gap), p(self.ws), self.ws_bytes, _stream())

    # ---- blocks with a length per sequence
    def draft_ragged(self, cache: DeviceCache, tokens, override, gammas, h_final: torch.Tensor):
        B.draft_forward_ragged(self.dims, self.weights, cache.struct, 0 if tokens is None else tokens.data_ptr(),
                               0 if override is None else override.data_ptr(), list(gammas), h_final.data_ptr(),
                               self.ws.data_ptr(), self.ws_bytes, _stream())

    def argmax_accept_ragged(self, flags, h_final, gammas, draft, target=None, tau=None, nxt=None, logits=None,
                             gap=None):
        p = lambda t: 0 if t is None else t.data_ptr()  # noqa: E731
        B.argmax_accept_ragged(self.dims, self.weights, flags, p(h_final), list(gammas), p(draft), p(target), p(tau),
                               p(nxt), p(logits), p(gap), p(self.ws), self.ws_bytes, _stream())

    # ---- many anchored blocks at once (training-style mask)
    def draft_blocks(self, cache: DeviceCache, block_seq, anchors, gamma, tokens, override, h_final: torch.Tensor):
        B.draft_forward_blocks(self.dims, self.weights, cache.struct, list(block_seq), list(anchors), gamma,
                               0 if tokens is None else tokens.data_ptr(),
                               0 if override is None else override.data_ptr(), h_final.data_ptr(),
                               self.ws.data_ptr(), self.ws_bytes, _stream())

