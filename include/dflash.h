/*
 * dflash.h - C ABI of the MI355X (gfx950) DFlash drafter hot path.
 *
 * Four calls cover the data-parallel path of a block-diffusion drafter with
 * target-context KV injection:
 *   dflash_fuse_context   (a) H_t = RMSNorm(W_c [H(l1); ...; H(l5)])
 *   dflash_inject_kv      (b) K/V = W_K H_t, W_V H_t for every drafter layer,
 *                             appended to that layer's KV cache
 *   dflash_draft_forward  (c) one forward over a gamma-row block (anchor + mask
 *                             rows), bidirectional over [context ; block]
 *   dflash_argmax_accept  (d) LM-head argmax of the mask rows and greedy
 *                             acceptance length against the target's tokens
 * with variants for blocks whose length differs per sequence:
 *   dflash_draft_forward_ragged, dflash_argmax_accept_ragged
 * and the drafter over many anchored blocks at once (the training-style mask):
 *   dflash_draft_forward_blocks
 * the target model's side of an iteration (its causal verify pass over the
 * block, with the hidden states of the tapped layers):
 *   dflash_target_verify
 * and, for decoding at a temperature T > 0, the sampled counterpart of (d):
 *   dflash_sample_drafts  draft tokens drawn from softmax(logits / T)
 *   dflash_sample_accept  lossless acceptance of a sampled block against the
 *                         target's temperature-T distributions
 *
 * Sources (page titles as published):
 *   [JP] "DFlash: Block Diffusion for Flash Speculative Decoding 논문 정리"
 *   [GL] "DFlash 블록 확산 디코딩: 투기적 디코딩의 드래프트 비용을 상수로 만드는 법"
 *   [MG] "ICML'26 | DFlash：用 Diffusion 模型干掉 AR Drafter，投机解码提速 6×"
 *
 * Conventions for every call
 *   - All tensor pointers are DEVICE pointers unless marked "host".  The caller
 *     allocates and owns every buffer (weights, cache, workspace, outputs); the
 *     library never allocates device memory and keeps no state between calls
 *     except a per-thread error string and a per-device architecture check.
 *   - Matrices are row-major and laid out [out, in] (a linear map y = W x stores
 *     W as [rows = outputs][cols = inputs]).
 *   - "weight type" is dims->dtype (DFLASH_BF16 or DFLASH_F32): weights and the
 *     tapped target states use it.  "cache type" is dims->cache_dtype: the fused
 *     context feature H_t and the KV cache use it (with bf16 weights it may be
 *     bf16, halving cache traffic, or f32, which keeps the drafter's output within
 *     ~1e-5 of an exact evaluation; with f32 weights it must be f32).  The
 *     residual stream, h_final and logits are always float32.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and the
 *     call returns without synchronising the host.
 *   - Errors: arguments, shapes, capacities and workspace size are checked on the
 *     host before anything is enqueued; on any error the call returns a negative
 *     status, enqueues nothing and leaves every output untouched (a HIP launch
 *     failure, DFLASH_ERR_HIP, is the only error raised after enqueueing began).
 *     dflash_last_error() returns the message.  No C++ exception crosses the ABI.
 *   - Calls on one stream are ordered; calls that write the same cache or
 *     workspace from different streams race.
 */
#ifndef DFLASH_H_
#define DFLASH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH_MAX_BATCH 64      /* sequences per call */
#define DFLASH_MAX_TGT_LAYERS 8  /* tapped target layers fused by W_c */
#define DFLASH_MIN_GAMMA 2
#define DFLASH_MAX_GAMMA 33      /* 1 anchor + 32 mask rows */

typedef enum {
  DFLASH_OK = 0,
  DFLASH_ERR_INVALID_ARG = -1,  /* null pointer, bad shape or flag */
  DFLASH_ERR_UNSUPPORTED = -2,  /* device is not gfx950, or a shape outside the kernels' range */
  DFLASH_ERR_CAPACITY = -3,     /* KV cache rows would exceed cap */
  DFLASH_ERR_WORKSPACE = -4,    /* workspace missing or smaller than required */
  DFLASH_ERR_HIP = -5           /* a HIP runtime call or kernel launch failed */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* Drafter shape.  Hq query heads share Hkv KV heads in contiguous groups of
 * G = Hq / Hkv (query head h reads KV head h / G).  Constraints checked by every
 * call: D % 64 == 0, F % 64 == 0, head_dim in {64, 128}, Hq % Hkv == 0,
 * 1 <= n_tgt_layers <= 8, 0 <= mask_id < V, V >= 2, rms_eps > 0, L >= 1,
 * dtype and cache_dtype in {DFLASH_F32, DFLASH_BF16}, and cache_dtype ==
 * DFLASH_F32 when dtype == DFLASH_F32. */
typedef struct {
  int32_t D;            /* hidden size of target and drafter */
  int32_t L;            /* drafter layers */
  int32_t Hq, Hkv;      /* query / key-value heads */
  int32_t head_dim;     /* d */
  int32_t F;            /* SwiGLU hidden size */
  int32_t V;            /* vocabulary of the shared embedding / LM head */
  int32_t n_tgt_layers; /* tapped target layers (5 in the pages) */
  int32_t mask_id;      /* token id of the mask rows */
  float rms_eps;        /* RMSNorm epsilon */
  int32_t dtype;        /* dflash_dtype: weights and target states */
  int32_t cache_dtype;  /* dflash_dtype: H_t and the KV cache */
} dflash_dims;

/* Non-owning device pointers to the drafter's weights, all in the weight type.
 * Only the fields a call uses must be set (see each call). */
typedef struct {
  const void* w_c;      /* [D][n_tgt_layers*D]  fusion projection W_c ([JP] "KV Injection 메커니즘") */
  const void* g_c;      /* [D]  gain of the fusion RMSNorm */
  const void* w_qkv;    /* [L][(Hq+2*Hkv)*d][D]  per layer: W_Q rows, then W_K, then W_V */
  const void* w_o;      /* [L][D][Hq*d] */
  const void* w_gateup; /* [L][2*F][D]  per layer: F gate rows, then F up rows */
  const void* w_down;   /* [L][D][F] */
  const void* g_attn;   /* [L][D]  pre-attention RMSNorm gains */
  const void* g_ffn;    /* [L][D]  pre-FFN RMSNorm gains */
  const void* g_final;  /* [D]     final RMSNorm gain before the LM head */
  const void* embed;    /* [V][D]  shared token embedding ([JP] "학습 방법": shared with the target) */
  const void* lm_head;  /* [V][D]  shared LM head; may alias embed (tied) */
} dflash_weights;

/* The drafter's KV cache: injected context rows plus gamma scratch rows per
 * sequence ([JP] "추론 구조", [GL] "KV 주입": injected K/V are cached and reused
 * across drafting iterations).  Layouts, in the cache type:
 *   k, fp32 cache: [L][B][Hkv][cap][d]           row-major keys
 *   k, bf16 cache: [L][B][Hkv][cap/32][32*d]     per block of 32 keys, the block
 *                  in the order of the attention's score fragments: key i, dim c
 *                  of a block at 512*(((i%8)/4)*(d/32) + c/32)
 *                  + 8*(16*((c%32)/8) + 4*(i/8) + i%4) + c%8 (i = key % 32)
 *   v, fp32 cache: [L][B][Hkv][d][cap]           values transposed (key fastest)
 *   v, bf16 cache: [L][B][Hkv][cap/32][d][32]    values transposed per block of
 *                  32 keys
 * In a bf16 cache each block of K or V is contiguous (8 KB at d = 128) and
 * every kilobyte the attention loads into LDS is one run of whole lines.
 * len[b] (HOST array, caller-owned) is the number of valid context rows of
 * sequence b.  Rows [0, len[b]) are never written by draft_forward; inject_kv
 * writes rows [len[b], len[b]+T_b) and then adds T_b to len[b].  The host
 * array is authoritative: every launch shape (key ranges, row tables) is
 * planned from it on the host, so no kernel reads lengths from the device.
 * len_dev (nullable, DEVICE [B] int32, caller-owned, 4-byte aligned) is a
 * device mirror for device-side consumers: when non-NULL, inject_kv writes
 * the new lengths into it on the stream, with the same kernel that stores the
 * appended rows, so it holds len[b] once the stream reaches that point.  The
 * caller initialises it (e.g. with a copy of len) before the first call. */
typedef struct {
  void* k;
  void* v;
  int32_t B;     /* sequences, 1..DFLASH_MAX_BATCH */
  int32_t cap;   /* rows per (layer, sequence, head); a positive multiple of 32 (the
                    attention reads keys in aligned 32-row blocks).  With a bf16
                    cache cap * head_dim * 2 must stay below 2^32 (checked;
                    DFLASH_ERR_UNSUPPORTED otherwise) */
  int32_t* len;      /* host [B] */
  int32_t* len_dev;  /* nullable device [B]: mirror of len written by inject_kv */
} dflash_kv_cache;

/* Version string of the library. */
const char* dflash_version(void);

/* Message of the last non-OK status returned on this thread ("" if none). */
const char* dflash_last_error(void);

/* Bytes of workspace every call needs for up to B sequences, blocks of up to
 * `gamma` rows (the same length for all sequences, or lengths of their own up
 * to gamma in the _ragged calls) and fuse/inject calls of up to `max_rows`
 * rows in total.  Pure host computation; enqueues nothing. */
dflash_status dflash_workspace_size(const dflash_dims* dims, int32_t B, int32_t gamma,
                                    int32_t max_rows, size_t* bytes);

/* (a) Context fusion, [JP] "KV Injection 메커니즘" (fusion equation) and [MG]
 * section 3.1: H_t[t] = g_c * u / sqrt(mean(u^2) + eps) with
 * u = W_c [h_tgt[0][t]; ...; h_tgt[n-1][t]] (sources in order, shallowest first;
 * the concatenation is never materialised).
 *   h_tgt  HOST array of n_tgt_layers device pointers, each [T][ld] weight type
 *          (row t of source k starts at h_tgt[k] + t*ld, ld >= D)
 *   T      rows (0 is allowed and does nothing)
 *   H_t    out [T][D] cache type
 * Uses weights->w_c, weights->g_c. */
dflash_status dflash_fuse_context(const dflash_dims* dims, const dflash_weights* w,
                                  const void* const* h_tgt, int64_t ld, int32_t T,
                                  void* H_t, void* ws, size_t ws_bytes, void* stream);

/* (b) KV injection, [JP] "KV Injection 메커니즘" and [MG] section 3.2: for every
 * layer l, K = W_K^l H_t and V = W_V^l H_t (no norm, no bias, no position
 * encoding), appended to sequence b's cache at rows [len[b], len[b]+T_b).
 *   H_t           [sum_b T_b][D] cache type: the rows of sequence 0, then 1, ...
 *   rows_per_seq  HOST [cache->B] row counts T_b >= 0
 * Errors: DFLASH_ERR_CAPACITY if len[b] + T_b > cap for some b (checked before
 * any work).  On success cache->len[b] += T_b (host), the rows land when the
 * stream reaches the kernels, and so does the same update of cache->len_dev
 * when it is given.  Uses weights->w_qkv. */
dflash_status dflash_inject_kv(const dflash_dims* dims, const dflash_weights* w, const void* H_t,
                               const int32_t* rows_per_seq, dflash_kv_cache* cache, void* ws,
                               size_t ws_bytes, void* stream);

/* (c) One drafting forward pass over a block of `gamma` rows per sequence,
 * [JP] "추론 구조" / "KV Injection 메커니즘" and [MG] section 3.3:
 *   h = embed[block_tokens] (or embed_override); per layer:
 *   a = RMSNorm(h; g_attn); Q = a W_Q^T; the block's K/V rows (a W_K^T, a W_V^T,
 *   stored in the cache type) go to cache scratch rows [len[b], len[b]+gamma);
 *   every query row attends, unmasked, to all len[b] context rows and all gamma
 *   block rows (softmax scale 1/sqrt(d), query head h -> KV head h/G);
 *   h += O W_O^T; f = RMSNorm(h; g_ffn); h += (SiLU(f W_gate^T) * f W_up^T) W_down^T.
 *   h_final = RMSNorm(h; g_final).
 *   block_tokens    [B][gamma] int32 (anchor at row 0, mask_id after it)
 *   embed_override  nullable [B][gamma][D] float32 rows used instead of the
 *                   embedding lookup (block_tokens may then be NULL)
 *   h_final         out [B][gamma][D] float32
 * B = cache->B.  Errors: DFLASH_ERR_CAPACITY if len[b] + gamma > cap.
 * Cache rows below len[b] are read only; len is unchanged. */
dflash_status dflash_draft_forward(const dflash_dims* dims, const dflash_weights* w,
                                   const dflash_kv_cache* cache, const int32_t* block_tokens,
                                   const float* embed_override, int32_t gamma, float* h_final,
                                   void* ws, size_t ws_bytes, void* stream);

/* (c) without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  The same pass as dflash_draft_forward, on the same
 * kernels, with the workspace taken from a static device array of 96 MiB
 * inside the library (one per GPU, held until the process ends; the call
 * itself allocates nothing).  Passes whose workspace would exceed it are
 * refused with DFLASH_ERR_WORKSPACE before anything is enqueued (at the
 * Qwen3-8B drafter shape, up to four sequences of 16 block rows fit; one
 * sequence of 33 rows does not).
 * Nothing in the array needs to start at zero: every byte a kernel reads was
 * written earlier in the same call.  All calls on one GPU share the array, so
 * calls that overlap on that GPU (other streams, other threads) race; calls
 * ordered on one stream do not. */
dflash_status dflash_draft_forward_noalloc(const dflash_dims* dims, const dflash_weights* w,
                                           const dflash_kv_cache* cache, const int32_t* block_tokens,
                                           const float* embed_override, int32_t gamma, float* h_final,
                                           void* stream);

/* (c) with a block length per sequence ([JP] "Ablation Study": a drafter
 * trained with large blocks keeps its acceptance with smaller inference blocks,
 * which allows choosing the block size per sequence at inference time;
 * "한계와 주의사항" leaves that scheduling open).  The same pass as
 * dflash_draft_forward, where sequence b's block has gammas[b] rows; the
 * blocks are packed row after row (sequence b's rows start at
 * G_b = gammas[0] + ... + gammas[b-1]) and every block attends only to its
 * own context and its own rows.
 *   gammas          HOST [cache->B], each in [DFLASH_MIN_GAMMA, DFLASH_MAX_GAMMA]
 *   block_tokens    [sum gammas] int32 (each block: anchor, then mask ids)
 *   embed_override  nullable [sum gammas][D] float32
 *   h_final         out [sum gammas][D] float32
 * Errors: DFLASH_ERR_CAPACITY if len[b] + gammas[b] > cap.  Scratch rows
 * [len[b], len[b] + gammas[b]) of each sequence are written; len is unchanged.
 * A workspace sized by dflash_workspace_size(dims, B, max gammas, ..) suffices. */
dflash_status dflash_draft_forward_ragged(const dflash_dims* dims, const dflash_weights* w,
                                          const dflash_kv_cache* cache, const int32_t* block_tokens,
                                          const float* embed_override, const int32_t* gammas, float* h_final,
                                          void* ws, size_t ws_bytes, void* stream);

/* (c) over many blocks anchored inside the cached context at once, as in
 * training ([JP] "학습 방법", sparse attention mask: every block attends to its
 * own rows in both directions and to its sequence's injected context, never
 * to another block).  Block k is anchored at position anchors[k] of sequence
 * block_seq[k]: its gamma rows (the anchor token, then mask rows) see that
 * sequence's context rows [0, anchors[k]) and its own rows only.
 *   block_seq, anchors  HOST [nblk]; 0 <= anchors[k] <= len[block_seq[k]]
 *   nblk                1 .. DFLASH_MAX_BATCH blocks per call
 *   block_tokens        [nblk][gamma] int32 (or embed_override [nblk][gamma][D])
 *   h_final             out [nblk][gamma][D] float32
 * Each block's own K/V rows are written to scratch rows of its sequence past
 * the context, in slots that follow one another from L32 = len[s] rounded up
 * to a multiple of 32, in call order.  With bf16 weights, an fp32 cache and
 * 2 * (Hq / Hkv) * gamma <= 128, two consecutive blocks of the same sequence
 * form a pair (the attention reads each context tile once for both): a pair
 * takes a slot of 2*gamma rows rounded up
 * to a multiple of 32, its first block rows [P, P + gamma) and its second
 * [P + gamma, P + 2*gamma); any other block takes a slot of gamma rows rounded
 * up likewise, its rows [P, P + gamma).  Errors: DFLASH_ERR_CAPACITY if a
 * sequence's slots end past cap (never more rows than L32 + (blocks of s) *
 * (gamma rounded up to 32)).  Context rows and len are not changed.
 * A workspace sized by dflash_workspace_size(dims, nblk, gamma, ..) suffices. */
dflash_status dflash_draft_forward_blocks(const dflash_dims* dims, const dflash_weights* w,
                                          const dflash_kv_cache* cache, const int32_t* block_seq,
                                          const int32_t* anchors, int32_t nblk, int32_t gamma,
                                          const int32_t* block_tokens, const float* embed_override, float* h_final,
                                          void* ws, size_t ws_bytes, void* stream);

#define DFLASH_ARGMAX 1u
#define DFLASH_ACCEPT 2u

/* (d) LM head + argmax and greedy acceptance.
 * DFLASH_ARGMAX ([MG] section 3.3; [JP] "학습 방법": shared LM head): for block
 *   rows i = 1..gamma-1 of each sequence, logits = lm_head . h_final[b][i] and
 *   draft[b][i-1] = argmax (lowest token id on ties).
 * DFLASH_ACCEPT ([JP] "Preliminaries": 1 <= tau <= drafts + 1): m = length of the
 *   longest prefix with draft[b][j] == target[b][j]; tau[b] = m + 1;
 *   next_anchor[b] = target[b][m].
 *   h_final      [B][gamma][D] float32 (ARGMAX)
 *   draft        [B][gamma-1] int32: written by ARGMAX, read by ACCEPT
 *   target       [B][gamma] int32: the target's token at each draft position,
 *                then its bonus token (ACCEPT)
 *   tau, next_anchor  out [B] int32 (ACCEPT)
 *   logits_dbg   nullable out [B][gamma-1][V] float32 (ARGMAX)
 *   top2_gap     nullable out [B][gamma-1] float32: best minus second-best logit
 * flags: a non-empty subset of DFLASH_ARGMAX | DFLASH_ACCEPT.  Uses weights->lm_head. */
dflash_status dflash_argmax_accept(const dflash_dims* dims, const dflash_weights* w, uint32_t flags,
                                   const float* h_final, int32_t B, int32_t gamma, int32_t* draft,
                                   const int32_t* target, int32_t* tau, int32_t* next_anchor,
                                   float* logits_dbg, float* top2_gap, void* ws, size_t ws_bytes,
                                   void* stream);

/* (d) for blocks packed as dflash_draft_forward_ragged writes them: sequence b
 * has n_b = gammas[b] - 1 drafts.
 *   h_final      [sum gammas][D] float32 (ARGMAX)
 *   gammas       HOST [B]
 *   draft        [sum n_b] int32, sequence b's at n_0 + ... + n_{b-1}: written by
 *                ARGMAX, read by ACCEPT
 *   target       [sum gammas] int32: sequence b's n_b + 1 target tokens (at each
 *                draft position, then the bonus) at gammas[0] + ... + gammas[b-1]
 *   tau, next_anchor  out [B] int32 (ACCEPT)
 *   logits_dbg   nullable out [sum n_b][V] float32; top2_gap nullable [sum n_b]
 * Same rules as dflash_argmax_accept per sequence.  The mask rows are gathered
 * into the workspace before the LM head. */
dflash_status dflash_argmax_accept_ragged(const dflash_dims* dims, const dflash_weights* w, uint32_t flags,
                                          const float* h_final, int32_t B, const int32_t* gammas, int32_t* draft,
                                          const int32_t* target, int32_t* tau, int32_t* next_anchor,
                                          float* logits_dbg, float* top2_gap, void* ws, size_t ws_bytes,
                                          void* stream);

/* The target side of a drafting iteration, on a target model of the
 * drafter's layer form (dims->L target layers; pre-norm residual layers, no
 * position encoding, no bias) with causal attention.  [JP] "방법론 / 추론
 * 구조", last step: the target verifies the drafted block in one parallel
 * pass; [JP] "실험 설정" (settings table) and [MG] section 3.1: the drafter
 * fuses the hidden states of 5 target layers spread uniformly from the
 * second to the third-from-last.
 * For each sequence b the block is block_tokens[b] = (anchor, d_0 .. d_{n-1}),
 * n = gamma - 1.  Block row i attends to the target's cached context rows
 * [0, len[b]) and to block rows 0..i; its K/V rows go to the target cache's
 * scratch rows [len[b], len[b] + i] (len is not changed: after acceptance the
 * caller keeps the first tau[b] rows by adding tau[b] to len[b]).
 *   target_tokens[b][i] = argmax of lm_head . RMSNorm(h_i; g_final) (lowest id
 *   on ties): the target's token at draft position i (i < n), then its bonus
 *   (i = n) -- the `target` input of dflash_argmax_accept(DFLASH_ACCEPT).
 *   taps[k] receives the residual stream after layer tap_layers[k] for every
 *   block row, [B * gamma][D] in the weight type: the rows [b * gamma,
 *   b * gamma + tau[b]) are the target states of the newly verified tokens,
 *   the input of dflash_fuse_context (n_tgt_layers = dims->n_tgt_layers).
 *   dims         the target's shape (n_tgt_layers taps, mask_id unused)
 *   w            target weights: w_qkv, w_o, w_gateup, w_down, g_attn, g_ffn,
 *                g_final, embed, lm_head (w_c, g_c unused)
 *   cache        the target's own KV cache (same layout as the drafter's)
 *   block_tokens [B][gamma] int32 device, gamma in [1, DFLASH_MAX_GAMMA]
 *   tap_layers   HOST [n_tgt_layers], increasing, each in [0, L)
 *   taps         HOST array of n_tgt_layers device pointers
 *   target_tokens out [B][gamma] int32; top2_gap nullable out [B][gamma] float32
 * Errors: DFLASH_ERR_CAPACITY if len[b] + gamma > cap.  Workspace:
 * dflash_workspace_size(dims, B, gamma, ..). */
dflash_status dflash_target_verify(const dflash_dims* dims, const dflash_weights* w, const dflash_kv_cache* cache,
                                   const int32_t* block_tokens, int32_t gamma, const int32_t* tap_layers,
                                   void* const* taps, int32_t* target_tokens, float* top2_gap, void* ws,
                                   size_t ws_bytes, void* stream);

/* Sampled drafting at temperature T ([JP] "주요 결과": DFlash decodes at
 * temperature 1 as well as greedily; [JP] "학습 방법": all block positions after
 * the anchor are predicted in one parallel pass).  For block rows i = 1..gamma-1
 * of each sequence: z = lm_head . h_final[b][i] (the logits of
 * dflash_argmax_accept), and draft[b][i-1] is one draw from q = softmax(z / T)
 * made with the Gumbel-max rule: the token v maximising
 * z_v / T - log(-log uniforms[b][i-1][v]) (lowest id on ties).
 *   h_final      [B][gamma][D] float32
 *   temperature  T > 0, finite, with a finite 1/T (the kernels use 1/T in fp32)
 *   uniforms     [B][gamma-1][V] float32, every value strictly inside (0, 1)
 *                (a 0 never wins, a 1 always wins)
 *   draft        out [B][gamma-1] int32
 *   logits       out [B][gamma-1][V] float32: z (needed by dflash_sample_accept)
 *   lse          nullable out [B][gamma-1] float32: log sum_v exp(z_v / T)
 * Uses weights->lm_head.  Workspace: dflash_workspace_size. */
dflash_status dflash_sample_drafts(const dflash_dims* dims, const dflash_weights* w, const float* h_final,
                                   int32_t B, int32_t gamma, float temperature, const float* uniforms,
                                   int32_t* draft, float* logits, float* lse, void* ws, size_t ws_bytes,
                                   void* stream);

/* Lossless acceptance of a sampled block ([GL] "비용 구조의 차이가 만드는 성능
 * 격차": through rejection/acceptance sampling the emitted tokens follow the
 * target model's own distribution).  With n = gamma-1, q_j = softmax(draft_logits
 * [b][j] / T) and p_j = softmax(target_logits[b][j] / T):
 *   draft j is accepted when accept_u[b][j] < p_j(d_j) / q_j(d_j), in order
 *   j = 0, 1, ...; the first j that fails is m (m = n if none fails);
 *   m < n: the emitted token is a draw from max(0, p_m - q_m) (normalised), or
 *          from p_m when that residual has no positive entry (rounding only);
 *   m = n: the emitted token is the bonus, a draw from p_n;
 *   both draws use the Gumbel-max rule with resid_u[b][:] (as in
 *   dflash_sample_drafts).  tau[b] = m + 1 tokens are committed: d_0..d_{m-1}
 *   and the emitted token, returned as next_anchor[b].
 *   draft          [B][n] int32 (ids outside [0, V) are clamped)
 *   draft_logits   [B][n][V] float32 (the logits output of dflash_sample_drafts)
 *   draft_lse      nullable [B][n] float32: log sum exp(draft_logits / T) as
 *                  written by dflash_sample_drafts; NULL = computed here
 *   target_logits  [B][n+1][V] float32: the target's logits at each draft
 *                  position, then at the bonus position
 *   accept_u       [B][n] float32 uniforms in [0, 1]
 *   resid_u        [B][V] float32 uniforms strictly inside (0, 1)
 *   tau, next_anchor  out [B] int32
 * Workspace: dflash_workspace_size. */
dflash_status dflash_sample_accept(const dflash_dims* dims, int32_t B, int32_t gamma, float temperature,
                                   const int32_t* draft, const float* draft_logits, const float* draft_lse,
                                   const float* target_logits, const float* accept_u, const float* resid_u,
                                   int32_t* tau, int32_t* next_anchor, void* ws, size_t ws_bytes, void* stream);

/* Kernel roles the profiling hook can bracket. */
typedef enum {
  DFLASH_PROF_NONE = 0,
  DFLASH_PROF_LM_HEAD = 1,   /* LM-head weight stream of dflash_argmax_accept / dflash_sample_drafts */
  DFLASH_PROF_QKV = 2,       /* per-layer Q/K/V projection */
  DFLASH_PROF_O = 3,         /* per-layer output projection */
  DFLASH_PROF_GATEUP = 4,    /* per-layer gate/up projection */
  DFLASH_PROF_DOWN = 5,      /* per-layer down projection */
  DFLASH_PROF_FUSE = 6,      /* W_c projection of dflash_fuse_context */
  DFLASH_PROF_INJECT = 7,    /* W_K/W_V projection of dflash_inject_kv */
  DFLASH_PROF_ATTENTION = 8, /* injected-context attention (without its combine step) */
  DFLASH_PROF_ROW_STATS = 9, /* row log-sum-exp pass of dflash_sample_accept (and of dflash_sample_drafts
                                when the LM head runs split-K) */
  DFLASH_PROF_VERIFY = 10    /* first-rejection and emitted-token kernels of dflash_sample_accept
                                (two launches, bracketed together) */
} dflash_prof_role;

/* Profiling hook (measurement only; not needed to run the path).  From now on,
 * on the calling thread, the i-th kernel launch of `role` records start[i] and
 * stop[i] (hipEvent_t, created with timing enabled) as part of its own dispatch
 * (hipExtLaunchKernelGGL), so that the interval is that kernel's run, for
 * i < n; later launches of the role record nothing.  DFLASH_PROF_VERIFY
 * brackets its two launches with events recorded on the stream before the
 * first and after the second.  The caller owns the
 * events and must keep the arrays alive until it calls this again.  role ==
 * DFLASH_PROF_NONE (or n == 0) turns the hook off.  Returns the number of
 * launches recorded since the previous call in *recorded (nullable).
 * Allocates nothing; errors: DFLASH_ERR_INVALID_ARG for an unknown role or
 * n > 0 with NULL arrays. */
dflash_status dflash_profile_events(int32_t role, void* const* start, void* const* stop, int32_t n,
                                    int32_t* recorded);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H_ */
