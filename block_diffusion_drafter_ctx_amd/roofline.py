"""Algorithmic work of each hot-path stage and MI355X peak figures.

"Algorithmic" bytes are what the method must move at least once: weights
streamed once per call, storage-type inputs read once, outputs written once,
context K/V read once per layer.  No padding, re-reads or split-K partials are
counted; those are implementation overheads the roofline fraction exposes.

The per-stage formulas follow the pages' cost discussion: the context feature
is computed once and reused ("DFlash: Block Diffusion for Flash Speculative
Decoding 논문 정리", section "KV Injection 메커니즘", memory table), and one
drafting pass costs one forward whatever the block size (same page, section
"Preliminaries", eq. (3)).
"""
from __future__ import annotations

# MI355X (gfx950) published peaks
HBM_PEAK_GBS = 8000.0            # HBM3E, GB/s
MFMA_BF16_TFLOPS = 2500.0        # dense bf16 MFMA
FP32_VECTOR_TFLOPS = 157.3
N_CU = 256
CLOCK_GHZ = 2.4


def elem_bytes(dtype: str) -> int:
    return {"bf16": 2, "f32": 4}[dtype]


# ---------------------------------------------------------------- (a) fusion
def fuse_bytes(T: int, D: int, n_tgt: int = 5, es: int = 2, cs: int = None) -> int:
    """n_tgt source states [T, D] + W_c [D, n_tgt*D] (weight type, es bytes) +
    H_t [T, D] (cache type, cs bytes)."""
    cs = es if cs is None else cs
    return (n_tgt * T * D + n_tgt * D * D) * es + T * D * cs


def fuse_flops(T: int, D: int, n_tgt: int = 5) -> int:
    return 2 * T * n_tgt * D * D


def w_c_bytes(D: int, n_tgt: int = 5, es: int = 2) -> int:
    return n_tgt * D * D * es


def fusion_input_bytes(T: int, D: int, n_tgt: int = 5, es: int = 2) -> int:
    return n_tgt * T * D * es


def fusion_output_bytes(T: int, D: int, es: int = 2) -> int:
    return T * D * es


# ------------------------------------------------------------- (b) injection
def inject_bytes(T: int, D: int, L: int, Hkv: int, d: int, es: int = 2, cs: int = None) -> int:
    """H_t [T, D] and the K/V rows written to the cache (cache type, cs bytes) +
    every layer's W_K, W_V (weight type, es bytes)."""
    cs = es if cs is None else cs
    kv = 2 * L * Hkv * d
    return kv * D * es + (T * D + T * kv) * cs


def inject_flops(T: int, D: int, L: int, Hkv: int, d: int) -> int:
    return 2 * T * D * 2 * L * Hkv * d


# ----------------------------------------------------------- (c) draft forward
def layer_weight_elems(D: int, Hq: int, Hkv: int, d: int, F: int) -> int:
    return (Hq + 2 * Hkv) * d * D + D * Hq * d + 2 * F * D + D * F + 2 * D


def draft_forward_bytes(D, L, Hq, Hkv, d, F, V, B, gamma, ctx_lens, es=2, cs=None) -> int:
    """All drafter weights once and the LM head once (weight type), each layer's
    context + block K/V once (cache type), and the fp32 activations in/out (block
    embedding rows and h_final)."""
    cs = es if cs is None else cs
    w = L * layer_weight_elems(D, Hq, Hkv, d, F) + D
    kv = L * sum(n + gamma for n in ctx_lens) * 2 * Hkv * d
    lm = V * D
    act = B * gamma * D * 4 * 2
    return (w + lm) * es + kv * cs + act


def draft_forward_bytes_ragged(D, L, Hq, Hkv, d, F, V, gammas, ctx_lens, es=2, cs=None) -> int:
    """``draft_forward_bytes`` for blocks of gammas[b] rows: each sequence's
    context + block K/V once per layer, the weights and the LM head once."""
    cs = es if cs is None else cs
    w = L * layer_weight_elems(D, Hq, Hkv, d, F) + D
    kv = L * sum(n + g for n, g in zip(ctx_lens, gammas)) * 2 * Hkv * d
    act = sum(gammas) * D * 4 * 2
    return (w + V * D) * es + kv * cs + act


def draft_forward_flops(D, L, Hq, Hkv, d, F, V, B, gamma, ctx_lens) -> int:
    M = B * gamma
    proj = 2 * M * L * ((Hq + 2 * Hkv) * d * D + D * Hq * d + 2 * F * D + D * F)
    att = L * sum(4 * Hq * gamma * (n + gamma) * d for n in ctx_lens)
    lm = 2 * B * (gamma - 1) * V * D
    return proj + att + lm


def lm_head_bytes(V: int, D: int, rows: int, es: int = 2) -> int:
    """LM-head GEMM + argmax: the [V, D] table once, fp32 rows in, ids out."""
    return V * D * es + rows * D * 4 + rows * 4


def lm_head_flops(V: int, D: int, rows: int) -> int:
    return 2 * rows * V * D


def lm_head_sample_bytes(V: int, D: int, rows: int, es: int = 2) -> int:
    """LM head with the sampling epilogue: the [V, D] table once and the fp32 rows
    in, one uniform read and one fp32 logit written per (row, token), ids and
    log-normalisers out."""
    return V * D * es + rows * D * 4 + 2 * rows * V * 4 + rows * 8


def row_stats_bytes(rows: int, V: int) -> int:
    """One read of each fp32 logits row (the log-sum-exp pass of the verify)."""
    return rows * V * 4


def verify_bytes(B: int, n: int, V: int, lse_given: bool = True) -> int:
    """Lossless verification of B sampled blocks of n drafts: every target row
    once (n + 1 per sequence), the draft rows once when their log-normalisers are
    not given, per sequence the residual's draft row and the emitting uniforms
    once, and the per-draft ids, uniforms, log-normalisers and gathered logits."""
    rows = B * (n + 1) + (0 if lse_given else B * n)
    return rows * V * 4 + B * 2 * V * 4 + B * n * 5 * 4 + B * 8


def attention_bytes(L: int, Hkv: int, d: int, gamma: int, ctx_lens, es: int = 2) -> int:
    return L * sum(n + gamma for n in ctx_lens) * 2 * Hkv * d * es


def accept_bytes(B: int, n: int) -> int:
    return B * (2 * n + 1) * 4 + B * 8


def gemm_bytes(N: int, K: int, M: int, es: int = 2, a_bytes: int = 4, out_bytes: int = 4) -> int:
    """Weight stream [N, K] once, the M activation rows in, the M output rows out."""
    return N * K * es + M * K * a_bytes + M * N * out_bytes
