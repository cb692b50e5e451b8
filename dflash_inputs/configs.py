"""Workload shapes for the DFlash drafter hot path.

The five workloads follow the drafter shapes the DFlash pages discuss: a tiny
fp32 drafter, a Qwen3-8B-shaped 5-layer drafter at a 2048-token context (the
pages' 2048-token generation and memory table), a 32K-token long context, a
ragged batch of 16 sequences, and an 8-layer drafter swept over block sizes
8/16/32 ("DFlash: Block Diffusion for Flash Speculative Decoding 논문 정리",
sections "실험 설정" and "Ablation Study"; the 5-layer / 16-token drafter of
"ICML'26 | DFlash：用 Diffusion 模型干掉 AR Drafter", section 2).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

BASE_SEED = 20261202


@dataclass(frozen=True)
class Config:
    name: str
    cid: int                 # seed namespace for this workload
    dtype: str               # "f32" or "bf16": weights and target states
    D: int
    L: int
    Hq: int
    Hkv: int
    d: int                   # head dim
    F: int                   # SwiGLU hidden size
    V: int                   # vocabulary (tied embedding / LM head)
    B: int
    ctx: tuple               # context length per sequence
    gammas: tuple            # block lengths (query rows: 1 anchor + gamma-1 masks)
    iters: int = 8           # drafting iterations per run
    append_rows: int = 16    # target rows appended per sequence per iteration
    n_tgt: int = 5           # tapped target layers
    eps: float = 1e-6
    match: str = "const"     # "const": p=0.8 per position; "linear": 0.9 -> 0.5
    w_std: float = 0.02
    gain_std: float = 0.0    # 0: unit gains (benchmark); >0: 1 + N(0, gain_std)
    cache_dtype: str = "f32"  # H_t and the KV cache: "f32" (default) or "bf16"

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def gamma(self) -> int:
        return self.gammas[0]

    @property
    def mask_id(self) -> int:
        return self.V - 1

    @property
    def n_ctx_total(self) -> int:
        return int(sum(self.ctx))

    def match_probs(self, gamma: int) -> np.ndarray:
        """Per-position probability that draft j equals the target's token."""
        n = gamma - 1
        if self.match == "const":
            return np.full(n, 0.8)
        j = np.arange(n, dtype=np.float64)
        return 0.9 - 0.4 * j / max(n - 1, 1)


def _ragged_lens(cid: int, B: int, lo: int, hi: int) -> tuple:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, cid, 9001])))
    return tuple(int(x) for x in rng.integers(lo, hi + 1, size=B))


_QWEN = dict(D=4096, Hq=32, Hkv=8, d=128, F=12288, V=151936)

# The five workloads, named by what they are (cid seeds their inputs).
TINY_F32 = Config(name="tiny_f32", cid=1, dtype="f32", D=256, L=1, Hq=4, Hkv=4, d=64, F=768,
                  V=1024, B=1, ctx=(128,), gammas=(16,))
QWEN3_8B_N2048 = Config(name="qwen3_8b_shape_n2048", cid=2, dtype="bf16", L=5, B=1, ctx=(2048,),
                        gammas=(16,), **_QWEN)
LONG_CTX_N32768 = Config(name="long_ctx_n32768", cid=3, dtype="bf16", L=5, B=1, ctx=(32768,),
                         gammas=(16,), **_QWEN)
BATCH16_RAGGED = Config(name="batch16_ragged", cid=4, dtype="bf16", L=5, B=16,
                        ctx=_ragged_lens(4, 16, 1024, 4096), gammas=(16,), **_QWEN)
DEEP8_B4_N8192 = Config(name="deep8_b4_n8192", cid=5, dtype="bf16", L=8, B=4, ctx=(8192,) * 4,
                        gammas=(8, 16, 32), match="linear", **_QWEN)

WORKLOADS = {c.name: c for c in (TINY_F32, QWEN3_8B_N2048, LONG_CTX_N32768, BATCH16_RAGGED, DEEP8_B4_N8192)}


def shrink(cfg: Config, **kw) -> Config:
    """A copy of ``cfg`` with some fields replaced (used for small parity shapes)."""
    return dataclasses.replace(cfg, **kw)
