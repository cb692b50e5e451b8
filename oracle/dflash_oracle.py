"""Plain, slow CPU oracle of the DFlash drafter hot path (float64 numpy).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
cpu_baseline leg may import this module.  It shares no code with the HIP path.

Every function writes a definition out in the order the pages state it, with a
numpy matmul as the only library primitive.  Storage tensors (the fused context
feature H_t and every key/value row that lands in the drafter's KV cache) are
rounded once to the workload's storage type ("bf16": round to nearest even;
"f32": IEEE single); everything else stays float64.

Sources (page titles as published):
  [JP]  "DFlash: Block Diffusion for Flash Speculative Decoding 논문 정리"
        (juhoplayground)
  [GL]  "DFlash 블록 확산 디코딩: 투기적 디코딩의 드래프트 비용을 상수로 만드는 법"
        (gillilab)
  [MG]  "ICML'26 | DFlash：用 Diffusion 模型干掉 AR Drafter，投机解码提速 6×"
        (marsggbo)

Readings taken where the pages are silent (each is also listed in the design
notes): pre-norm residual drafter layers with a final RMSNorm before the shared
LM head; no positional encoding, no bias; GQA with contiguous head groups and a
1/sqrt(d) softmax scale; the block is gamma query rows (anchor at row 0, mask
tokens after it) whose own K/V rows are stored in the cache like context rows.

Parity pins live in tests/test_oracle_pins.py; every function below is pinned.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------
def to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits, ties to
    even) and return them as float64."""
    x = np.asarray(x, dtype=F64)
    m, e = np.frexp(x)                   # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def store(x, storage: str) -> np.ndarray:
    """Value of ``x`` after it is written to a tensor of the storage type
    ("f64": kept as computed, for callers that round it themselves)."""
    if storage == "bf16":
        return to_bf16(x)
    if storage == "f32":
        return np.asarray(x, dtype=np.float32).astype(F64)
    if storage == "f64":
        return np.asarray(x, dtype=F64)
    raise ValueError(storage)


# ---------------------------------------------------------------------------
# elementwise pieces
# ---------------------------------------------------------------------------
def rmsnorm(x, g, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: g * x / sqrt(mean(x^2) + eps)
    ([MG] section 3.1 applies it to the fused projection)."""
    x = np.asarray(x, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(g, dtype=F64) * (x / np.sqrt(ms + eps))


def silu(x) -> np.ndarray:
    """SiLU(x) = x / (1 + exp(-x)), the gate of the SwiGLU FFN."""
    x = np.asarray(x, dtype=F64)
    return x / (1.0 + np.exp(-x))


# ---------------------------------------------------------------------------
# (a) context fusion
# ---------------------------------------------------------------------------
def fuse_context(h_tgt, w_c, g_c, eps: float, storage: str) -> np.ndarray:
    """H_t = RMSNorm(W_c [H(l1); ...; H(l5)]).

    [JP] section "KV Injection 메커니즘" (the fusion equation): the tapped target
    states are concatenated along the feature axis, shallowest first, projected
    by the bias-free W_c (D x 5D) and RMS-normalised; [MG] section 3.1 describes
    the same extractor as a bias-free 5D-to-D linear map followed by RMSNorm.
    h_tgt: list of [T, D]; w_c: [D, n*D] laid out [out, in]; returns [T, D].
    """
    x = np.concatenate([np.asarray(h, dtype=F64) for h in h_tgt], axis=1)
    u = x @ np.asarray(w_c, dtype=F64).T
    return store(rmsnorm(u, g_c, eps), storage)


# ---------------------------------------------------------------------------
# (b) KV injection
# ---------------------------------------------------------------------------
def split_qkv(w_qkv, Hq: int, Hkv: int, d: int):
    """Rows of a packed [Q; K; V] projection matrix."""
    w = np.asarray(w_qkv)
    return w[: Hq * d], w[Hq * d:(Hq + Hkv) * d], w[(Hq + Hkv) * d:(Hq + 2 * Hkv) * d]


def inject_kv(H_t, w_qkv, Hq: int, Hkv: int, d: int, storage: str):
    """Context key/value rows of one drafter layer: K = W_K H_t, V = W_V H_t.

    [JP] section "KV Injection 메커니즘": the target feature enters every layer
    only through that layer's K and V projections (no Q, O, FFN or norm);
    [MG] section 3.2 projects the context feature with the layer's own key and
    value maps.  Returns ([T, Hkv, d], [T, Hkv, d]).
    """
    _, wk, wv = split_qkv(w_qkv, Hq, Hkv, d)
    h = np.asarray(H_t, dtype=F64)
    k = store(h @ np.asarray(wk, dtype=F64).T, storage)
    v = store(h @ np.asarray(wv, dtype=F64).T, storage)
    T = h.shape[0]
    return k.reshape(T, Hkv, d), v.reshape(T, Hkv, d)


class OracleCache:
    """The drafter's per-layer KV cache of injected context rows.

    [JP] section "방법론 / 추론 구조" and [GL] section "KV 주입": the injected K/V
    are kept in the drafter's KV cache and reused across drafting iterations.
    k[l][b] / v[l][b] are [len_b, Hkv, d] float64 arrays.
    """

    def __init__(self, L: int, B: int, Hkv: int, d: int):
        self.k = [[np.zeros((0, Hkv, d)) for _ in range(B)] for _ in range(L)]
        self.v = [[np.zeros((0, Hkv, d)) for _ in range(B)] for _ in range(L)]

    def lens(self):
        return [self.k[0][b].shape[0] for b in range(len(self.k[0]))]

    def append(self, l: int, b: int, k, v):
        self.k[l][b] = np.concatenate([self.k[l][b], k], axis=0)
        self.v[l][b] = np.concatenate([self.v[l][b], v], axis=0)

    def sequence(self, b: int) -> "OracleCache":
        """A one-sequence cache holding sequence b's rows (shared, not copied)."""
        return self.prefix(b, self.k[0][b].shape[0])

    def prefix(self, b: int, n: int) -> "OracleCache":
        """A one-sequence cache holding the first n rows of sequence b."""
        one = OracleCache.__new__(OracleCache)
        one.k = [[self.k[l][b][:n]] for l in range(len(self.k))]
        one.v = [[self.v[l][b][:n]] for l in range(len(self.v))]
        return one


# ---------------------------------------------------------------------------
# (c) draft forward
# ---------------------------------------------------------------------------
def attention(q, k, v) -> np.ndarray:
    """Softmax attention of every query row over every key row, no mask.

    [JP] "KV Injection 메커니즘": queries come from the draft block only, keys and
    values are [context ; block] joined along the sequence; [MG] section 3.2:
    scaled dot-product attention over that join, bidirectional inside the block.
    q: [R, Hq, d]; k, v: [n, Hkv, d].  Query head h reads KV head h // (Hq/Hkv).
    Returns [R, Hq, d].
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    R, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.empty((R, Hq, d))
    for h in range(Hq):
        j = h // G
        s = (q[:, h, :] @ k[:, j, :].T) / np.sqrt(d)          # [R, n]
        s = s - np.max(s, axis=1, keepdims=True)
        p = np.exp(s)
        p = p / np.sum(p, axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, j, :]
    return out


def draft_forward(dims, layers, g_final, cache: OracleCache, gamma: int,
                  embed=None, tokens=None, override=None, storage: str = "bf16"):
    """One forward pass of the drafter over a block of ``gamma`` rows per sequence.

    [JP] "추론 구조": the block (the clean anchor from the last verify, then mask
    tokens; "학습 방법" puts the anchor at block position 0) is decoded in a single
    forward pass with bidirectional attention; "KV Injection 메커니즘": in layer i,
    Q = W_Q H_d and K, V = [W_K H_t ; W_K H_d] / [W_V H_t ; W_V H_d].
    [MG] section 3.3 runs the embedded block through every layer with the
    injected context.  Each layer is read as a pre-norm residual block:
        a = RMSNorm(h; g_attn); h += Attn(a) W_O^T
        f = RMSNorm(h; g_ffn);  h += (SiLU(f W_gate^T) * (f W_up^T)) W_down^T
    and a final RMSNorm(h; g_final) feeds the shared LM head.

    dims: object with D, Hq, Hkv, d, F, eps.  layers: list of dicts with w_qkv,
    w_o, w_gateup ([gate; up] rows), w_down, g_attn, g_ffn.  The block rows come
    from embed[tokens] ([B, gamma] ids) or from ``override`` ([B, gamma, D]).
    Returns (h_final [B, gamma, D] float64, block K/V per layer).
    """
    D, Hq, Hkv, d, F, eps = dims.D, dims.Hq, dims.Hkv, dims.d, dims.F, dims.eps
    if override is not None:
        h = np.asarray(override, dtype=F64).copy()
    else:
        h = np.asarray(embed)[np.asarray(tokens)].astype(F64)
    B = h.shape[0]
    assert h.shape == (B, gamma, D)
    block_kv = []
    for l, w in enumerate(layers):
        a = rmsnorm(h, w["g_attn"], eps)                                  # [B, g, D]
        qkv = a @ np.asarray(w["w_qkv"], dtype=F64).T                     # [B, g, (Hq+2Hkv)d]
        q = qkv[..., : Hq * d].reshape(B, gamma, Hq, d)
        kb = store(qkv[..., Hq * d:(Hq + Hkv) * d], storage).reshape(B, gamma, Hkv, d)
        vb = store(qkv[..., (Hq + Hkv) * d:], storage).reshape(B, gamma, Hkv, d)
        block_kv.append((kb, vb))
        o = np.empty((B, gamma, Hq * d))
        for b in range(B):
            keys = np.concatenate([cache.k[l][b], kb[b]], axis=0)
            vals = np.concatenate([cache.v[l][b], vb[b]], axis=0)
            o[b] = attention(q[b], keys, vals).reshape(gamma, Hq * d)
        h = h + o @ np.asarray(w["w_o"], dtype=F64).T
        f = rmsnorm(h, w["g_ffn"], eps)
        gu = f @ np.asarray(w["w_gateup"], dtype=F64).T
        s = silu(gu[..., :F]) * gu[..., F:]
        h = h + s @ np.asarray(w["w_down"], dtype=F64).T
    return rmsnorm(h, g_final, eps), block_kv


def draft_forward_ragged(dims, layers, g_final, cache: OracleCache, gammas, embed=None, tokens=None,
                         override=None, storage: str = "bf16"):
    """One drafting pass over sequences whose blocks have lengths of their own.

    [JP] "Ablation Study": a drafter trained with large blocks keeps its
    acceptance with smaller inference blocks, which allows the block size to be
    chosen per sequence at inference time ("한계와 주의사항" leaves that
    scheduling open).  Sequences never interact in the drafter: each block
    attends to its own context and its own rows only.  So the pass over a batch
    with block lengths gammas[b] is, for every sequence, the one-sequence pass
    of ``draft_forward`` over its own block.
    tokens: list of [gammas[b]] id arrays (or override: list of [gammas[b], D]).
    Returns (list of h_final [gammas[b], D], list of per-layer block K/V).
    """
    outs, kvs = [], []
    for b, g in enumerate(gammas):
        tok = None if tokens is None else np.asarray(tokens[b])[None]
        ov = None if override is None else np.asarray(override[b])[None]
        hf, kv = draft_forward(dims, layers, g_final, cache.sequence(b), int(g), embed=embed, tokens=tok,
                               override=ov, storage=storage)
        outs.append(hf[0])
        kvs.append([(k[0], v[0]) for k, v in kv])
    return outs, kvs


def draft_forward_blocks(dims, layers, g_final, cache: OracleCache, blocks, gamma: int, embed=None, tokens=None,
                         override=None, storage: str = "bf16"):
    """The drafter over many anchored blocks at once, as in training.

    [JP] "학습 방법" (sparse attention mask): the blocks, each anchored at a
    sampled position of a sequence, are processed together; a block's rows
    attend to each other in both directions and to their sequence's injected
    context features, and never to another block ([MG] describes a causal
    mask across blocks instead; the reading here follows [JP]).  A block
    anchored at position a sees the context features of positions [0, a): the
    anchor is the block's first row, as at inference, where it is the token
    right after the verified context.  Each block is therefore the one-sequence
    pass of ``draft_forward`` over that context prefix.
    blocks: list of (sequence index, anchor position a), a <= the sequence's
    cache length.  tokens: [nblk, gamma] ids (or override: [nblk, gamma, D]).
    Returns (h_final [nblk, gamma, D], per block the per-layer block K/V).
    """
    outs, kvs = [], []
    for k, (sq, a) in enumerate(blocks):
        tok = None if tokens is None else np.asarray(tokens[k])[None]
        ov = None if override is None else np.asarray(override[k])[None]
        hf, kv = draft_forward(dims, layers, g_final, cache.prefix(int(sq), int(a)), gamma, embed=embed,
                               tokens=tok, override=ov, storage=storage)
        outs.append(hf[0])
        kvs.append([(kk[0], vv[0]) for kk, vv in kv])
    return np.stack(outs), kvs


# ---------------------------------------------------------------------------
# (d) LM head, argmax and greedy acceptance
# ---------------------------------------------------------------------------
def lm_head_argmax(h_final, lm_head):
    """Logits of the mask rows and their argmax.

    [MG] section 3.3: the LM head is applied to the block rows after the anchor
    (the anchor's own output is not a draft), and each draft token is the argmax; [JP] "학습 방법": the LM head is the target's,
    shared and frozen.  Ties go to the lowest token id.
    Returns (draft [B, gamma-1] int32, top-2 gap [B, gamma-1], logits [B, gamma-1, V]).
    """
    z = np.asarray(h_final, dtype=F64)[:, 1:, :]
    logits = z @ np.asarray(lm_head, dtype=F64).T
    draft = np.argmax(logits, axis=-1).astype(np.int32)     # first maximum
    top2 = -np.partition(-logits, 1, axis=-1)[..., :2]
    gap = top2[..., 0] - top2[..., 1]
    return draft, gap, logits


def accept(draft, target):
    """Greedy acceptance length and the next anchor.

    [JP] "Preliminaries": tau counts the accepted drafts plus the target's bonus
    token, 1 <= tau <= (drafts) + 1; [GL] "투기적 디코딩에 확산 모델을 끼워 넣다":
    accepted tokens are kept and the ones after the first rejection dropped.
    draft: [B, n]; target: [B, n+1] (the target's token at each draft position,
    then the bonus).  tau = (length of the matching prefix) + 1 and the next
    anchor is the target's token right after that prefix.
    """
    draft = np.asarray(draft)
    target = np.asarray(target)
    B, n = draft.shape
    tau = np.zeros(B, dtype=np.int32)
    nxt = np.zeros(B, dtype=np.int32)
    for b in range(B):
        m = 0
        while m < n and int(draft[b, m]) == int(target[b, m]):
            m += 1
        tau[b] = m + 1
        nxt[b] = target[b, m]
    return tau, nxt


# ---------------------------------------------------------------------------
# sampled drafting and lossless verification at temperature T > 0
# ---------------------------------------------------------------------------
def log_softmax_t(logits, T: float) -> np.ndarray:
    """log softmax(logits / T) over the last axis (max-shifted)."""
    x = np.asarray(logits, dtype=F64) / float(T)
    mx = np.max(x, axis=-1, keepdims=True)
    return x - (mx + np.log(np.sum(np.exp(x - mx), axis=-1, keepdims=True)))


def logsumexp_t(logits, T: float) -> np.ndarray:
    """log sum_v exp(logits_v / T) over the last axis."""
    x = np.asarray(logits, dtype=F64) / float(T)
    mx = np.max(x, axis=-1)
    return mx + np.log(np.sum(np.exp(x - mx[..., None]), axis=-1))


def gumbel_pick(logw, u):
    """One categorical draw from weights proportional to exp(logw) along the
    last axis, using one uniform u_v in (0, 1) per category: the Gumbel-max
    rule picks argmax_v (logw_v - log(-log u_v)).  Entries with logw = -inf
    have weight 0.  Ties go to the lowest index.
    Returns (index, best key minus second-best key)."""
    key = np.asarray(logw, dtype=F64) - np.log(-np.log(np.asarray(u, dtype=F64)))
    idx = np.argmax(key, axis=-1)
    if key.shape[-1] < 2:
        return idx.astype(np.int32), np.full(idx.shape, np.inf)
    top = -np.partition(-key, 1, axis=-1)[..., :2]
    return idx.astype(np.int32), top[..., 0] - top[..., 1]


def sample_drafts(h_final, lm_head, T: float, u):
    """Draft tokens sampled from the drafter's temperature-T distribution.

    [JP] "주요 결과" reports DFlash at temperature 1 (sampling) next to greedy
    decoding, and "학습 방법" has the drafter predict all block positions after
    the anchor in parallel: each mask row i = 1..gamma-1 gets its own logits
    z = lm_head . h_final[b][i] and its draft token is one draw from
    q = softmax(z / T), made here with the Gumbel-max rule and the caller's
    uniforms u[b][i-1][:] (one per vocabulary entry).
    Returns (draft [B, n] int32, logits z [B, n, V], log sum exp(z / T) [B, n],
    key gap [B, n]: the winning perturbed key minus the runner-up).
    """
    z = np.asarray(h_final, dtype=F64)[:, 1:, :] @ np.asarray(lm_head, dtype=F64).T
    draft, gap = gumbel_pick(z / float(T), u)
    return draft, z, logsumexp_t(z, T), gap


def sample_accept(draft, draft_logits, target_logits, T: float, accept_u, resid_u):
    """Lossless verification of a sampled block (speculative sampling).

    [GL] "비용 구조의 차이가 만드는 성능 격차": DFlash's speedup is lossless, since
    the rejection/acceptance sampling of speculative decoding makes every output
    token follow the target model's own distribution.  The rule written out here
    is the standard one with that property.  With q_j = softmax(draft_logits[j] / T)
    and p_j = softmax(target_logits[j] / T):
      * for j = 0, 1, ... in order, draft j is accepted when
        accept_u[j] < p_j(d_j) / q_j(d_j); the first j that fails is m (m = n when
        every draft is accepted);
      * m < n: the emitted token is a draw from max(0, p_m - q_m) (normalised);
        should that residual have no positive entry, the draw is from p_m;
      * m = n: the emitted token is the bonus, a draw from p_n;
    both draws use the Gumbel-max rule with the uniforms resid_u[b][:].
    tau = m + 1 tokens are committed: d_0..d_{m-1} and the emitted token, which
    is also the next block's anchor.
    draft [B, n]; draft_logits [B, n, V]; target_logits [B, n+1, V];
    accept_u [B, n]; resid_u [B, V].
    Returns (tau [B], next_anchor [B], info) where info holds, per sequence,
    "m", "log_ratio" [B, n] (log p_j(d_j) - log q_j(d_j)), "resid_empty" and
    "key_gap" (margin of the final draw).
    """
    draft = np.asarray(draft)
    B, n = draft.shape
    lq = log_softmax_t(draft_logits, T)                    # [B, n, V]
    lp = log_softmax_t(target_logits, T)                   # [B, n+1, V]
    bi = np.arange(B)[:, None]
    ji = np.arange(n)[None, :]
    log_ratio = lp[:, :n][bi, ji, draft] - lq[bi, ji, draft]
    accepted = np.asarray(accept_u, dtype=F64) < np.exp(log_ratio)
    tau = np.zeros(B, dtype=np.int32)
    nxt = np.zeros(B, dtype=np.int32)
    m_all = np.zeros(B, dtype=np.int32)
    empty = np.zeros(B, dtype=bool)
    key_gap = np.zeros(B)
    for b in range(B):
        m = 0
        while m < n and accepted[b, m]:
            m += 1
        if m < n:
            r = np.maximum(0.0, np.exp(lp[b, m]) - np.exp(lq[b, m]))
            empty[b] = not np.any(r > 0.0)
            with np.errstate(divide="ignore"):
                logw = lp[b, m] if empty[b] else np.log(r)
        else:
            logw = lp[b, n]
        tok, gap = gumbel_pick(logw, resid_u[b])
        m_all[b], tau[b], nxt[b], key_gap[b] = m, m + 1, tok, gap
    return tau, nxt, dict(m=m_all, log_ratio=log_ratio, resid_empty=empty, key_gap=key_gap)


def lm_head_argmax_ragged(h_final, lm_head):
    """``lm_head_argmax`` per sequence of a ragged batch: h_final is a list of
    [gamma_b, D] blocks; returns lists of drafts [gamma_b - 1], gaps, logits."""
    out = [lm_head_argmax(np.asarray(h)[None], lm_head) for h in h_final]
    return [d[0] for d, _, _ in out], [g[0] for _, g, _ in out], [z[0] for _, _, z in out]


def accept_ragged(drafts, targets):
    """``accept`` per sequence of a ragged batch: drafts[b] has n_b entries and
    targets[b] has n_b + 1 (the target's token at each draft position, then its
    bonus).  Returns (tau [B], next_anchor [B])."""
    res = [accept(np.asarray(d)[None], np.asarray(t)[None]) for d, t in zip(drafts, targets)]
    return (np.array([int(t[0]) for t, _ in res], dtype=np.int32),
            np.array([int(x[0]) for _, x in res], dtype=np.int32))



# ---------------------------------------------------------------------------
# the target side: tapped layers and the parallel verify forward
# ---------------------------------------------------------------------------
def tap_layers(L_t: int, n: int = 5):
    """0-based indices of the n target layers whose hidden states are fused.

    [JP] "실험 설정" (settings table, row on the target hidden features) and
    [MG] section 3.1: five layers spread uniformly from the target's second
    layer to its third-from-last.  Index k (k = 0..n-1) is
    1 + k (L_t - 4) / (n - 1), rounded half up (the pages do not say how a
    fractional position is rounded).
    """
    if n == 1:
        return [1]
    first, last = 1, L_t - 3
    return [first + int(np.floor(k * (last - first) / (n - 1) + 0.5)) for k in range(n)]


def attention_causal(q, k, v, n_ctx: int) -> np.ndarray:
    """Softmax attention of the block rows over [context ; block] with a causal
    mask inside the block: block row i sees the n_ctx context rows and block
    rows 0..i (an autoregressive target reads each position's past only).
    q: [R, Hq, d]; k, v: [n_ctx + R, Hkv, d].  Query head h reads KV head
    h // (Hq/Hkv), scale 1/sqrt(d).  Returns [R, Hq, d]."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    R, Hq, d = q.shape
    G = Hq // k.shape[1]
    out = np.empty((R, Hq, d))
    for h in range(Hq):
        kv_head = h // G
        for i in range(R):
            seen = n_ctx + i + 1
            sc = (k[:seen, kv_head, :] @ q[i, h, :]) / np.sqrt(d)
            w = np.exp(sc - np.max(sc))
            out[i, h, :] = (w / np.sum(w)) @ v[:seen, kv_head, :]
    return out


def target_verify(dims, layers, g_final, embed, lm_head, cache: OracleCache, tokens, taps,
                  storage: str = "bf16", tap_storage: str = "bf16"):
    """The target model's parallel verify forward over one block per sequence.

    [JP] "방법론 / 추론 구조", last step: the target checks the whole drafted
    block in one parallel pass; [GL] "투기적 디코딩에 확산 모델을 끼워 넣다": the
    target verifies the proposed tokens in parallel and keeps the accepted
    ones.  The block is the anchor (the last verified token's successor) and
    the n drafts.  The synthetic target has the drafter's layer form
    (pre-norm residual layers, no positional encoding, no bias) with causal
    attention over its own KV cache of the verified context; the row of block
    position j predicts the token after it, so its argmax is the target's
    token at draft position j (j < n) and the last row's is the bonus.
    Alongside, the residual stream after each tapped layer is kept: the hidden
    states the drafter fuses for the verified tokens ([JP] "추론 구조": hidden
    states of a fixed set of uniformly chosen layers, read while the target
    runs).

    tokens [B, gamma] ids; cache: the target's K/V of the context rows;
    taps: 0-based layer indices.  Returns a dict with "tokens" [B, gamma]
    (argmax, lowest id on ties), "gap" [B, gamma] (top-2 gap), "logits",
    "taps" (per tapped layer [B, gamma, D], stored in tap_storage) and
    "block_kv" (per layer the block's K/V rows, stored in the cache type).
    """
    D, Hq, Hkv, d, F, eps = dims.D, dims.Hq, dims.Hkv, dims.d, dims.F, dims.eps
    tok = np.asarray(tokens)
    x = np.asarray(embed)[tok].astype(F64)
    B, gamma = tok.shape
    kept = {}
    rows_kv = []
    for l, w in enumerate(layers):
        xa = rmsnorm(x, w["g_attn"], eps)
        proj = xa @ np.asarray(w["w_qkv"], dtype=F64).T
        qt = proj[..., : Hq * d].reshape(B, gamma, Hq, d)
        kt = store(proj[..., Hq * d:(Hq + Hkv) * d], storage).reshape(B, gamma, Hkv, d)
        vt = store(proj[..., (Hq + Hkv) * d:], storage).reshape(B, gamma, Hkv, d)
        rows_kv.append((kt, vt))
        att = np.empty((B, gamma, Hq * d))
        for b in range(B):
            n_ctx = cache.k[l][b].shape[0]
            att[b] = attention_causal(qt[b], np.concatenate([cache.k[l][b], kt[b]], axis=0),
                                      np.concatenate([cache.v[l][b], vt[b]], axis=0), n_ctx).reshape(gamma, Hq * d)
        x = x + att @ np.asarray(w["w_o"], dtype=F64).T
        xf = rmsnorm(x, w["g_ffn"], eps)
        up = xf @ np.asarray(w["w_gateup"], dtype=F64).T
        x = x + (silu(up[..., :F]) * up[..., F:]) @ np.asarray(w["w_down"], dtype=F64).T
        if l in taps:
            kept[l] = store(x, tap_storage)
    logits = rmsnorm(x, g_final, eps) @ np.asarray(lm_head, dtype=F64).T
    best = np.argmax(logits, axis=-1).astype(np.int32)
    two = -np.partition(-logits, 1, axis=-1)[..., :2]
    return dict(tokens=best, gap=two[..., 0] - two[..., 1], logits=logits, taps=[kept[l] for l in taps],
                block_kv=rows_kv)
