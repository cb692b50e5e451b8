// Host-side launchers of the gfx950 kernels (internal to libdflash).  Each
// launcher enqueues on `st` and returns hipGetLastError() of its launches; the
// argument structs are passed to the kernels by value.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dflash {

constexpr int kMaxSrc = 8;
constexpr int kMaxSeq = 64;

// ------------------------------------------------------- profiling events
// A start / stop event pair that the next launch made through launch_k records
// as part of its own dispatch (hipExtLaunchKernelGGL): the timestamps bracket
// the kernel itself and add no packets to the stream.  The library's profiling
// hook sets it right before the launch of a bracketed role; the launch
// consumes it.  Per thread.
struct PendingEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
PendingEvents& pending_events();

template <typename K, typename... Args>
inline void launch_k(K kernel, dim3 grid, dim3 block, size_t shm, hipStream_t st, Args... args) {
  PendingEvents& pe = pending_events();
  if (pe.start != nullptr) {
    const PendingEvents e = pe;
    pe = PendingEvents{};
    hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(shm), st, e.start, e.stop, 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shm, st, args...);
  }
}

// ------------------------------------------------------- launch attributes
// Raise kernel fn's dynamic-LDS limit to at least `bytes` on the current
// device.  Function attributes are per device; the first launch on each
// device sets it, later ones find it in a table (thread-safe).
hipError_t ensure_dyn_lds(const void* fn, int bytes);
// The dynamic LDS kernel fn may use beside its static LDS (rounded down to
// KB, 0 if under 1 KB or the limit cannot be raised), set as its limit on the
// current device the first time it is asked for there (thread-safe).
int dyn_lds_room(const void* fn, int lds_bytes);

// ------------------------------------------------------------------- GEMMs
// C[m][n] = sum_k A[m][k] * W[n][k] over a K range, written as split-K partials
// part[s][m][n] (fp32).
//   A row m, column k: src[k / a_cols] + (m / a_rg) * a_gs + (m % a_rg) * a_ld + k % a_cols
//   W row n: w + ((n / w_rg) * w_gs + w_off + n % w_rg) * w_ld
struct GemmArgs {
  const void* a_src[kMaxSrc];
  int32_t a_cols;
  int32_t a_rg;
  int64_t a_ld, a_gs;
  const void* w;
  int64_t w_ld, w_gs, w_off;
  int32_t w_rg;
  int32_t M, N, K;
  int32_t chunks_per_split;   // 32-wide k steps per split (MFMA path)
  int32_t S, ntiles, mtiles;  // work decomposition (MFMA path; set by the launcher)
  float* part;                // [S][M][N]
  const void* a_lo;           // A_BF16_HILO: the lo plane, laid out like a_src[0] (the hi plane)
  const float* su;            // LM-head sampling epilogue: uniforms [M][N] in (0, 1)
  float inv_t;                // LM-head sampling epilogue: 1 / temperature
  int32_t stage_tiles;        // LM-head sampling epilogue: logits tiles held in LDS per workgroup (set by the launcher)
  int32_t rchunks;            // register-K: 16-row chunks of A, one workgroup each (set by the launcher)
  int32_t xcd_tiles;          // tiled kernel: 1-D launch in XCD-grouped tile order (set by the launcher)
};

// exact bf16 A; fp32 A split hi/lo on the fly; or A given as pre-split bf16
// hi (a_src[0]) and lo (a_lo) planes of an fp32 matrix (tiled kernel only)
enum GemmAKind { A_BF16 = 0, A_F32_SPLIT = 1, A_BF16_HILO = 2 };

struct GemmPlan {
  int MT = 16, mtiles = 1, ntiles = 1, nchunks = 1, cps = 1, S = 1, waves = 8, grid = 1;
  bool tiled = false;   // LDS-tiled kernel for many activation rows
  bool rk = false;      // register-K kernel (16-row chunks, tall weight)
  int ks = 8;           // register-K: k steps per wave
  int mr = 1;           // register-K: 16-row chunks (the launch has mr * grid workgroups)
  int tn = 0;           // tiled: weight rows per tile (with MT, the tile shape)
  size_t part_floats = 0;
};

// wide = 16-wave workgroups with a 128 KB activation slice (fewer K splits for
// very tall weights such as the LM head); otherwise 8 waves and 64 KB.
GemmPlan plan_gemm_mfma(int M, int N, int K, GemmAKind ak, bool wide);
// Many activation rows: LDS-tiled MFMA kernel (K % 64 == 0), 128 activation rows
// per tile against 128 (fp32 A split on the fly) or 256 (bf16 A, or pre-split
// hi/lo planes) weight rows.
GemmPlan plan_gemm_tiled(int M, int N, int K, GemmAKind ak);
// The plan the library uses for an M x N x K product (register-K for few rows
// and suitable shapes, tiled from 33 rows when K % 64 == 0, streaming
// otherwise).
GemmPlan plan_gemm(int M, int N, int K, GemmAKind ak, bool wide);
hipError_t launch_gemm_mfma(const GemmArgs& a, GemmAKind ak, const GemmPlan& p, hipStream_t st);

// The LM head on the tiled kernel (plan from plan_gemm(.., A_BF16_HILO, ..) with
// a single K split; a addresses the hi / lo planes): writes the top-2 of every
// row within each n-tile to top2 [p.ntiles][M][3] (value, index bits,
// runner-up) and, when logits != nullptr, the logits [M][N].
hipError_t launch_gemm_tiled_top2(const GemmArgs& a, const GemmPlan& p, float* top2, float* logits, hipStream_t st);

// Register-K kernel for up to rk_max_rows(tall) activation rows (fp32 split
// hi/lo, or exact bf16 with ak = A_BF16) against a bf16 weight, 16 rows per
// workgroup; plan.rk is false when the shape does not qualify.  top2 = true
// asks for the LM-head epilogue (a single K split).
constexpr int kRkMaxGrid = 1024;   // bound on register-K unit groups (top-2 workspace rows)
constexpr int kRkMaxRows = 128;    // largest row count the register-K form may be set to take
constexpr int kRkMaxRowsTall = 32; // default for the tall forms (a single K split); the short form takes 16
int rk_max_rows(bool tall);
GemmPlan plan_gemm_rk(int M, int N, int K, bool top2);
// top2 == nullptr: store part[s][m][n].  Otherwise write the per-workgroup top-2
// of every row to top2 [p.grid][M][3] (value, index bits, runner-up) and, when
// logits != nullptr, the logits [M][N].
hipError_t launch_gemm_rk(const GemmArgs& a, const GemmPlan& p, float* top2, float* logits, hipStream_t st,
                          GemmAKind ak = A_F32_SPLIT);
// LM head with the temperature-sampling epilogue (plan from plan_gemm_rk(.., true)):
// stores logits [M][N] and writes each workgroup's per-row SampleStat (key over
// x + G(a.su), x = logit * a.inv_t) to stats [p.grid][M].
hipError_t launch_gemm_rk_sample(const GemmArgs& a, const GemmPlan& p, float4* stats, float* logits,
                                 hipStream_t st);
// FFN gate/up with SwiGLU fused: W is the stacked [gate (F rows); up (F rows)]
// weight, a.N = F; writes s_out[m][f] = silu(gate) * up.  plan.rk is false when
// the shape does not qualify (the caller then runs the GEMM and swiglu apart).
GemmPlan plan_gemm_rk_swiglu(int M, int F, int K);
hipError_t launch_gemm_rk_swiglu(const GemmArgs& a, const GemmPlan& p, float* s_out, hipStream_t st);

// Sum the split-K partials of logits [S][M][N] per 512-column tile, optionally
// store the logits, and write each (tile, row) top-2 to top2 [ntiles][M][3].
hipError_t launch_reduce_top2(const float* part, int S, int M, int N, float* logits, float* top2,
                              int* ntiles_out, hipStream_t st);

// fp32 storage path: plain FMA GEMM, single split; writes part[0][m][n].
hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t st);

// hi[m][k] = bf16(x[m][k]), lo[m][k] = bf16(x - hi) for an fp32 [M][K] matrix
// whose row m starts at x + (m / rg) * gs + (m % rg) * ld (elements; rg = INT_MAX
// for plain rows of stride ld); hi and lo are dense [M][K].
hipError_t launch_split_hilo(const float* x, int64_t ld, int M, int K, uint16_t* hi, uint16_t* lo, hipStream_t st,
                             int rg = 0x7fffffff, int64_t gs = 0);

// ------------------------------------------------------------ epilogues
// Per-sequence row table: rows [row_off[b], row_off[b+1]) of a GEMM output belong
// to sequence b and land at cache rows pos0[b] + (row - row_off[b]).
struct SeqRows {
  int32_t B;
  int32_t row_off[kMaxSeq + 1];
  int32_t pos0[kMaxSeq];
  int32_t seq[kMaxSeq];   // scatter: cache sequence of group b
};

struct ScatterArgs {
  const float* part;   // [S][M][N]
  int32_t S, M, N;
  int32_t nq;          // columns [0, nq) are query columns -> q_out[m][n]
  float* q_out;
  void* kc;            // cache K base of layer `layer0`: [L][B][Hkv][cap][d] (fp32), per 32-key block in fragment order (bf16)
  void* vc;            // cache V base: [L][B][Hkv][d][cap] (fp32), [L][B][Hkv][cap/32][d][32] (bf16)
  int32_t layer0, B, Hkv, d, cap;
  SeqRows rows;
  int32_t* len_dev;               // nullable: the cache's device length mirror ...
  int32_t len_new[kMaxSeq];       // ... set to these values (B of them) by the launch
};

hipError_t launch_scatter_kv(const ScatterArgs& a, bool bf16_cache, hipStream_t st);

// H_t[t] = store(g * u / sqrt(mean(u^2)+eps)), u = sum_s part[s][t]; g in the weight type,
// H_t in the cache type
hipError_t launch_ctx_norm(const float* part, int S, int T, int D, const void* g, float eps,
                           void* out, bool bf16_weights, bool bf16_cache, hipStream_t st);

// bf16 hi / lo planes [M][K] (row-major) of an fp32 matrix, x ~= hi + lo: the
// A operand of the tiled GEMM.  A producer given planes (hi != nullptr) writes
// them in place of its fp32 rows, with the split the GEMM's own split pass
// would apply to those rows.
struct HiLo {
  uint16_t* hi = nullptr;
  uint16_t* lo = nullptr;
};

// h[m] += sum_s part[s][m]; a[m] = g * h / sqrt(mean(h^2)+eps)   (part may be null;
// a as planes when pl.hi is set).  tap (nullable): the updated h also stored
// there, [M][D] in the weight type (a tapped hidden state of a target layer).
hipError_t launch_residual_norm(const float* part, int S, int M, int D, float* h, const void* g,
                                float eps, float* a_out, bool bf16, hipStream_t st, HiLo pl = HiLo{},
                                void* tap = nullptr);

// s[m][f] = silu(sum_s part[s][m][f]) * sum_s part[s][m][F+f]   (s as planes when pl.hi is set)
hipError_t launch_swiglu(const float* part, int S, int M, int F, float* s_out, hipStream_t st, HiLo pl = HiLo{});

// h[m] = embed[tok[m]] or override[m]; a[m] = RMSNorm(h[m]; g)   (ids clamped to [0, V);
// a as planes when pl.hi is set)
hipError_t launch_embed_norm(const int32_t* tok, const float* ov, const void* embed, int V, int M, int D,
                             const void* g, float eps, float* h, float* a, bool bf16, hipStream_t st,
                             HiLo pl = HiLo{});

// top-2 partials [ntiles][M] -> draft[m], gap[m]
hipError_t launch_argmax_final(const float* top2, int ntiles, int M, int32_t* draft, float* gap,
                               hipStream_t st);
// rows of logits [M][V] -> draft[m], gap[m]
hipError_t launch_argmax_rows(const float* logits, int M, int V, int32_t* draft, float* gap,
                              hipStream_t st);

hipError_t launch_accept(const int32_t* draft, const int32_t* target, int B, int n, int32_t* tau,
                         int32_t* next_anchor, hipStream_t st);

// dst row m of sequence b (t.row_off[b] <= m < t.row_off[b+1]) = src row
// t.pos0[b] + m - t.row_off[b]; rows of D floats (D % 4 == 0, 16-byte aligned)
hipError_t launch_gather_rows(const float* src, float* dst, int D, const SeqRows& t, hipStream_t st);
// greedy acceptance with n_b = t.row_off[b+1] - t.row_off[b] drafts at
// draft + t.row_off[b] and n_b + 1 targets at target + t.pos0[b] (n_b <= 63)
hipError_t launch_accept_ragged(const int32_t* draft, const int32_t* target, const SeqRows& t, int32_t* tau,
                                int32_t* next_anchor, hipStream_t st);

// ------------------------------------------------------------ sampling
constexpr int kSampleChunk = 4096;   // columns per row-statistics workgroup (at least)
constexpr int kSpecMaxChunks = 64;   // row-statistics pieces per row, at most
constexpr int kSpecMaxN = 32;        // drafts per block, at most
constexpr int kSpecDrawChunk = 1024; // columns per workgroup of the emitted-token draw

// Row-statistics pass.  Rows [0, rows1) read src + r*N, summing S split-K
// partials split_stride apart; rows [rows1, rows) read src2 + (r - rows1)*N.
// Per (row, chunk of `chunk` columns) it writes stats[chunk][row]: the
// log-sum-exp state of x = value * inv_t and, when su is given (rows of src
// only, su [rows1][N]), the best Gumbel key x + G(su).  logits_out (nullable)
// receives the summed src rows.
struct RowStatArgs {
  const float* src;
  int64_t split_stride;
  int32_t S;
  const float* src2;
  int32_t rows1, rows, N, chunk;
  int32_t vec;             // 1: N % 4 == 0 and every row 16-byte aligned
  float* logits_out;
  const float* su;
  float inv_t;
  float4* stats;
};

// Columns per row-statistics chunk for `rows` rows of a vocabulary of V (a
// multiple of kSampleChunk; at most kSpecMaxChunks chunks per row; never
// smaller for fewer rows, so a layout sized for many rows bounds fewer).
constexpr int kStatTargetGroups = 2048;
int sample_chunk(int V, int rows);
hipError_t launch_row_stats(const RowStatArgs& a, hipStream_t st);
// merge stats [nparts][M] per row: draft[m] = best key's index, lse[m] (nullable)
// = log sum exp(x)
hipError_t launch_sample_final(const float4* stats, int nparts, int M, int32_t* draft, float* lse, hipStream_t st);

// Lossless verification of a sampled block (spec_verify + spec_final kernels).
struct SpecArgs {
  const int32_t* draft;    // [B][n]
  const float* zq;         // draft logits [B][n][V]
  const float* zp;         // target logits [B][n+1][V]
  const float* lse_q;      // nullable [B][n]: log sum exp(zq / T) of the draft rows
  const float* accept_u;   // [B][n]
  const float* resid_u;    // [B][V]
  const float4* stats;     // row statistics [nchunk][rows]: target row j of sequence b at
                           // b*(n+1)+j, then (lse_q null) draft rows at B*(n+1)+b*n+j
  int32_t B, n, V, nchunk, rows, vec;
  int32_t ndraw;           // ceil(V / kSpecDrawChunk): workgroups per sequence of the draw
  float inv_t;
  float4* part;            // scratch [B][ndraw]
  int32_t* m_out;          // scratch [B]
  int32_t* tau;            // out [B]
  int32_t* next_anchor;    // out [B]
};
hipError_t launch_spec_verify(const SpecArgs& a, hipStream_t st);

// ------------------------------------------------------------ attention
struct AttnArgs {
  const float* q;        // [M][Hq*d], M = qrow0[B] block rows (sequence b's at qrow0[b] ..)
  const void* kc;        // layer base [B][Hkv][cap][d] (fp32), [B][Hkv][cap/32][32*d] in fragment order (bf16)
  const void* vc;        // layer base [B][Hkv][d][cap] (fp32), [B][Hkv][cap/32][d][32] (bf16)
  float* part_o;         // [items][Rpad][d]
  float* part_ml;        // [items][Rpad][2]
  float* o_out;          // [B*gamma][Hq*d]
  uint16_t* o_hi;        // when set: o_out written as bf16 hi / lo planes instead (same layout)
  uint16_t* o_lo;
  int32_t B, Hq, Hkv, d, cap;
  int32_t R, Rpad;       // query rows per (b, kv head): the largest G*gam[b], padded to 16
  int32_t gam[kMaxSeq];       // block rows of sequence b
  int32_t qrow0[kMaxSeq + 1]; // first block row of sequence b in q / o_out (qrow0[B] = M)
  int32_t kvseq[kMaxSeq];     // cache sequence whose K/V block b reads
  int32_t half[kMaxSeq];      // block rows of group b's first block (gam[b] unless two blocks share the group)
  int32_t ctx1[kMaxSeq];      // anchored blocks: context keys of the first block's rows
  int32_t ctx2[kMaxSeq];      // anchored blocks: context keys of the second block's rows
  int32_t blk0[kMaxSeq];      // -1: the block's rows follow the context (keys [0, nkeys[b]));
                              // else its own rows [blk0, blk0 + gam) are a separate key item
                              // after the context keys [0, nkeys[b]) (blk0 % 32 == 0)
  int32_t causal;        // 1: block row i sees keys [0, nkeys[b] - gam[b] + i] only (blocks that
                         // follow their context; an autoregressive target's verify pass)
  int32_t split_keys;    // keys per work item (multiple of 32)
  int32_t items;
  float scale_log2;      // log2(e) / sqrt(d)
  int32_t nkeys[kMaxSeq];     // len_b + gamma
  int32_t nsplit[kMaxSeq];
  int32_t item_off[kMaxSeq + 1];
};

struct AttnPlan {
  int split_keys = 32, items = 0, Rpad = 16, row_groups = 1;
  int nsplit[kMaxSeq] = {0};
  int item_off[kMaxSeq + 1] = {0};
  size_t part_floats = 0;
};

// apart (nullable): apart[b] != 0 when block b's own rows are stored apart
// from its context (one more key item per (b, kv head))
AttnPlan plan_attention(int B, const int32_t* nkeys, int Hkv, int R, int d, const int32_t* apart = nullptr);
size_t attention_part_bound(int B, int Hkv, int R, int d);
// The main attention kernel is launched through launch_k (pending profiling
// events bracket it, not its combine step).
hipError_t launch_attention(const AttnArgs& a, const AttnPlan& p, bool bf16_weights, bool bf16_cache,
                            hipStream_t st);

}  // namespace dflash
