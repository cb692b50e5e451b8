// C-ABI entry points of libdflash: argument validation, workspace planning and
// the launch sequence of each hot-path stage.  Everything that can be checked
// on the host is checked before the first HIP call, so a rejected call enqueues
// nothing and touches no output.
#include "../../include/dflash.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "launch.h"

using namespace dflash;

namespace {

thread_local std::string g_err;

dflash_status fail(dflash_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

dflash_status ok() {
  g_err.clear();
  return DFLASH_OK;
}

#define DF_REQUIRE(cond, st, ...)           \
  do {                                      \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

// A launch bracketed by the profiling hook: the hook's bookkeeping ends
// whether or not the launch failed.
#define DF_HIP_PROF(expr, slot)         \
  do {                                  \
    const hipError_t ep_ = (expr);      \
    prof_end((slot), s);                \
    DF_HIP(ep_);                        \
  } while (0)

#define DF_HIP(expr)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(DFLASH_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr size_t kAlign = 256;
constexpr int kRowBlock = 4096;   // rows per fuse / inject GEMM pass

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(const dflash_dims* d) { return d->dtype == DFLASH_BF16 ? 2 : 4; }          // weight type
size_t csize(const dflash_dims* d) { return d->cache_dtype == DFLASH_BF16 ? 2 : 4; }    // cache type

dflash_status check_dims(const dflash_dims* d) {
  DF_REQUIRE(d != nullptr, DFLASH_ERR_INVALID_ARG, "dims is NULL");
  DF_REQUIRE(d->dtype == DFLASH_F32 || d->dtype == DFLASH_BF16, DFLASH_ERR_INVALID_ARG,
             "dtype %d is neither DFLASH_F32 nor DFLASH_BF16", d->dtype);
  DF_REQUIRE(d->cache_dtype == DFLASH_F32 || d->cache_dtype == DFLASH_BF16, DFLASH_ERR_INVALID_ARG,
             "cache_dtype %d is neither DFLASH_F32 nor DFLASH_BF16", d->cache_dtype);
  DF_REQUIRE(!(d->dtype == DFLASH_F32 && d->cache_dtype == DFLASH_BF16), DFLASH_ERR_INVALID_ARG,
             "fp32 weights need an fp32 cache (cache_dtype DFLASH_F32)");
  DF_REQUIRE(d->D >= 64 && d->D % 64 == 0 && d->D <= 16384, DFLASH_ERR_INVALID_ARG,
             "D=%d must be a multiple of 64 in [64, 16384]", d->D);
  DF_REQUIRE(d->F >= 64 && d->F % 64 == 0, DFLASH_ERR_INVALID_ARG, "F=%d must be a positive multiple of 64", d->F);
  DF_REQUIRE(d->L >= 1, DFLASH_ERR_INVALID_ARG, "L=%d must be >= 1", d->L);
  DF_REQUIRE(d->head_dim == 64 || d->head_dim == 128, DFLASH_ERR_INVALID_ARG, "head_dim=%d must be 64 or 128",
             d->head_dim);
  DF_REQUIRE(d->Hq >= 1 && d->Hkv >= 1 && d->Hq % d->Hkv == 0, DFLASH_ERR_INVALID_ARG,
             "Hq=%d must be a positive multiple of Hkv=%d", d->Hq, d->Hkv);
  DF_REQUIRE(d->n_tgt_layers >= 1 && d->n_tgt_layers <= DFLASH_MAX_TGT_LAYERS, DFLASH_ERR_INVALID_ARG,
             "n_tgt_layers=%d must be in [1, %d]", d->n_tgt_layers, DFLASH_MAX_TGT_LAYERS);
  DF_REQUIRE(d->V >= 2, DFLASH_ERR_INVALID_ARG, "V=%d must be >= 2", d->V);
  DF_REQUIRE(d->mask_id >= 0 && d->mask_id < d->V, DFLASH_ERR_INVALID_ARG, "mask_id=%d outside [0, V)", d->mask_id);
  DF_REQUIRE(std::isfinite(d->rms_eps) && d->rms_eps > 0.f, DFLASH_ERR_INVALID_ARG, "rms_eps must be > 0");
  const int64_t kvcols = static_cast<int64_t>(2) * d->L * d->Hkv * d->head_dim;
  DF_REQUIRE(kvcols < INT_MAX && static_cast<int64_t>(d->Hq + 2 * d->Hkv) * d->head_dim < INT_MAX,
             DFLASH_ERR_INVALID_ARG, "head counts too large");
  return DFLASH_OK;
}

dflash_status check_gamma(int gamma) {
  DF_REQUIRE(gamma >= DFLASH_MIN_GAMMA && gamma <= DFLASH_MAX_GAMMA, DFLASH_ERR_INVALID_ARG,
             "gamma=%d outside [%d, %d]", gamma, DFLASH_MIN_GAMMA, DFLASH_MAX_GAMMA);
  return DFLASH_OK;
}

dflash_status check_cache(const dflash_kv_cache* c) {
  DF_REQUIRE(c != nullptr, DFLASH_ERR_INVALID_ARG, "cache is NULL");
  DF_REQUIRE(c->B >= 1 && c->B <= DFLASH_MAX_BATCH, DFLASH_ERR_INVALID_ARG, "cache->B=%d outside [1, %d]", c->B,
             DFLASH_MAX_BATCH);
  DF_REQUIRE(c->k != nullptr && c->v != nullptr && c->len != nullptr, DFLASH_ERR_INVALID_ARG,
             "cache k, v and len must be non-NULL");
  DF_REQUIRE(aligned16(c->k) && aligned16(c->v), DFLASH_ERR_INVALID_ARG, "cache k/v must be 16-byte aligned");
  DF_REQUIRE(c->cap >= 32 && c->cap % 32 == 0, DFLASH_ERR_INVALID_ARG, "cache->cap=%d must be a positive multiple of 32",
             c->cap);
  DF_REQUIRE((reinterpret_cast<uintptr_t>(c->len_dev) & 3u) == 0, DFLASH_ERR_INVALID_ARG,
             "cache->len_dev must be 4-byte aligned");
  for (int b = 0; b < c->B; ++b)
    DF_REQUIRE(c->len[b] >= 0 && c->len[b] <= c->cap, DFLASH_ERR_INVALID_ARG, "cache->len[%d]=%d outside [0, cap]",
               b, c->len[b]);
  return DFLASH_OK;
}

// Shape limits of the attention kernels for a cache (checked before any launch).
dflash_status check_attention_cache(const dflash_dims* d, const dflash_kv_cache* c) {
  // the bf16-cache kernel addresses one head's K or V with 32-bit byte offsets
  DF_REQUIRE(d->cache_dtype != DFLASH_BF16 ||
                 static_cast<int64_t>(c->cap) * d->head_dim * 2 < (int64_t{1} << 32),
             DFLASH_ERR_UNSUPPORTED, "a bf16 cache needs cap * head_dim * 2 < 2^32 (cap=%d, head_dim=%d)", c->cap,
             d->head_dim);
  return DFLASH_OK;
}

dflash_status check_ptr(const void* p, const char* name) {
  DF_REQUIRE(p != nullptr, DFLASH_ERR_INVALID_ARG, "%s is NULL", name);
  DF_REQUIRE(aligned16(p), DFLASH_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  return DFLASH_OK;
}

dflash_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return DFLASH_OK;
  DF_REQUIRE(ws != nullptr, DFLASH_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  DF_REQUIRE(ws_bytes >= need, DFLASH_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  DF_REQUIRE((reinterpret_cast<uintptr_t>(ws) % kAlign) == 0, DFLASH_ERR_WORKSPACE,
             "workspace must be %zu-byte aligned", kAlign);
  return DFLASH_OK;
}

// gfx950 check, once per device.
dflash_status check_device() {
  static std::mutex mu;
  static int state[64] = {0};   // 0 unknown, 1 ok, -1 unsupported
  int dev = 0;
  DF_HIP(hipGetDevice(&dev));
  DF_REQUIRE(dev >= 0 && dev < 64, DFLASH_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (state[dev] == 0) {
    hipDeviceProp_t prop;
    DF_HIP(hipGetDeviceProperties(&prop, dev));
    state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    if (state[dev] < 0) return fail(DFLASH_ERR_UNSUPPORTED, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  }
  DF_REQUIRE(state[dev] == 1, DFLASH_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return DFLASH_OK;
}

// ----------------------------------------------------------- workspace plans
struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

size_t gemm_part_floats(const dflash_dims* d, int M, int N, int K, GemmAKind ak, bool wide = false) {
  if (M <= 0) return 0;
  if (d->dtype == DFLASH_F32) return static_cast<size_t>(M) * N;
  return plan_gemm(M, N, K, ak, wide).part_floats;
}

GemmAKind ctx_a_kind(const dflash_dims* d) { return d->cache_dtype == DFLASH_BF16 ? A_BF16 : A_F32_SPLIT; }

// fuse: partials of one row-block pass
size_t fuse_ws(const dflash_dims* d, int max_rows) {
  size_t best = 0;
  const int hi = max_rows < kRowBlock ? max_rows : kRowBlock;
  for (int M = 1; M <= hi; ++M) {
    const size_t f = gemm_part_floats(d, M, d->D, d->n_tgt_layers * d->D, A_BF16);
    if (f > best) best = f;
  }
  return best ? align_up(best * 4) : 0;
}

// Row passes of inject that take the tiled GEMM with an fp32 H_t split first
// into bf16 hi / lo planes (placed after the partial sums).
bool inject_splits(const dflash_dims* d, int M) {
  return d->dtype == DFLASH_BF16 && ctx_a_kind(d) == A_F32_SPLIT &&
         plan_gemm(M, 2 * d->L * d->Hkv * d->head_dim, d->D, A_F32_SPLIT, false).tiled;
}

GemmAKind inject_kind(const dflash_dims* d, int M) { return inject_splits(d, M) ? A_BF16_HILO : ctx_a_kind(d); }

size_t inject_ws(const dflash_dims* d, int max_rows) {
  size_t best = 0, planes = 0;
  const int N = 2 * d->L * d->Hkv * d->head_dim;
  const int hi = max_rows < kRowBlock ? max_rows : kRowBlock;
  for (int M = 1; M <= hi; ++M) {
    const size_t f = gemm_part_floats(d, M, N, d->D, inject_kind(d, M));
    if (f > best) best = f;
    if (inject_splits(d, M)) {
      const size_t pl = 2 * align_up(static_cast<size_t>(M) * d->D * 2);
      if (pl > planes) planes = pl;
    }
  }
  return best || planes ? align_up(best * 4) + planes : 0;
}

// An fp32-activation product against a bf16 weight.  When the tiled GEMM
// takes it (many rows), the activations are split once into bf16 hi / lo
// planes for the LDS-direct kernel; otherwise they are split on the fly.
struct ActPlan {
  GemmPlan p;
  GemmAKind kind;
};

ActPlan plan_act(int M, int N, int K, bool wide) {
  const GemmPlan p = plan_gemm(M, N, K, A_F32_SPLIT, wide);
  if (!p.tiled) return ActPlan{p, A_F32_SPLIT};
  return ActPlan{plan_gemm(M, N, K, A_BF16_HILO, wide), A_BF16_HILO};
}

size_t act_planes_bytes(const ActPlan& a, int M, int K) {
  return a.kind == A_BF16_HILO ? 2 * align_up(static_cast<size_t>(M) * K * 2) : 0;
}

// Where the hi / lo planes of an M x K activation block sit in `planes` (the
// lo plane after the hi plane, 256-byte aligned).
HiLo act_planes(const ActPlan& a, void* planes, int M, int K) {
  if (a.kind != A_BF16_HILO) return HiLo{};
  HiLo pl;
  pl.hi = static_cast<uint16_t*>(planes);
  pl.lo = reinterpret_cast<uint16_t*>(static_cast<char*>(planes) + align_up(static_cast<size_t>(M) * K * 2));
  return pl;
}

// Points g at the activation planes (splitting g's fp32 rows into them unless
// ready) when the plan takes them; otherwise leaves g as it is.
hipError_t prepare_act(GemmArgs& g, const ActPlan& a, void* planes, hipStream_t s, bool ready) {
  if (a.kind == A_BF16_HILO) {
    const HiLo pl = act_planes(a, planes, g.M, g.K);
    uint16_t* hi = pl.hi;
    uint16_t* lo = pl.lo;
    if (!ready) {
      const hipError_t e = launch_split_hilo(static_cast<const float*>(g.a_src[0]), g.a_ld, g.M, g.K, hi, lo, s,
                                             g.a_rg, g.a_gs);
      if (e != hipSuccess) return e;
    }
    for (int k = 0; k < kMaxSrc; ++k) g.a_src[k] = hi;
    g.a_lo = lo;
    g.a_cols = g.K;
    g.a_ld = g.K;
    g.a_rg = INT_MAX;
    g.a_gs = 0;
  }
  return hipSuccess;
}

// g addresses fp32 activations (any row mapping of one source); planes:
// act_planes_bytes of scratch.  ready: the producer of A has already written
// the planes (act_planes) in place of g's fp32 rows.
hipError_t launch_act_gemm(GemmArgs g, const ActPlan& a, void* planes, hipStream_t s, bool ready = false) {
  const hipError_t e = prepare_act(g, a, planes, s, ready);
  if (e != hipSuccess) return e;
  return launch_gemm_mfma(g, a.kind, a.p, s);
}

struct DraftWs {
  size_t h, a, q, o, s, part, att_o, att_ml, planes, total;
};

// M block rows in all (sum of the block lengths), the longest block gmax rows.
DraftWs draft_ws(const dflash_dims* d, int B, int M, int gmax) {
  const int hd = d->Hq * d->head_dim;
  const int nqkv = (d->Hq + 2 * d->Hkv) * d->head_dim;
  size_t part = 0, planes = 0;
  auto upd = [&](int N, int K) {
    if (d->dtype == DFLASH_F32) {
      part = static_cast<size_t>(M) * N > part ? static_cast<size_t>(M) * N : part;
      return;
    }
    const ActPlan ap = plan_act(M, N, K, false);
    part = ap.p.part_floats > part ? ap.p.part_floats : part;
    const size_t pl = act_planes_bytes(ap, M, K);
    planes = pl > planes ? pl : planes;
  };
  upd(nqkv, d->D);
  upd(d->D, hd);
  upd(2 * d->F, d->D);
  upd(d->D, d->F);
  const int R = (d->Hq / d->Hkv) * gmax;
  const size_t att = d->dtype == DFLASH_BF16 ? attention_part_bound(B, d->Hkv, R, d->head_dim) : 0;
  const size_t rpad_rows = att / (d->head_dim + 2);
  DraftWs w{};
  Carve c;
  w.h = c.take(static_cast<size_t>(M) * d->D * 4);
  w.a = c.take(static_cast<size_t>(M) * d->D * 4);
  w.q = c.take(static_cast<size_t>(M) * hd * 4);
  w.o = c.take(static_cast<size_t>(M) * hd * 4);
  w.s = c.take(static_cast<size_t>(M) * d->F * 4);
  w.part = c.take(part * 4);
  w.att_o = c.take(rpad_rows * d->head_dim * 4);
  w.att_ml = c.take(rpad_rows * 2 * 4);
  w.planes = c.take(planes);
  w.total = c.off;
  return w;
}

// The LM head of M rows (bf16 weights): the register-K kernel with the top-2
// epilogue (up to 32 rows); else the tiled kernel over hi / lo planes with one
// K split and the top-2 epilogue (D is a multiple of 64); else split-K
// partials and a reduce pass.  The single split can cost more whole-K rounds
// than the tiled planner's choice but writes no partials: on the 151936 x 4096
// head, 60 rows take 335 us (streaming kernel + reduce: 362 + 53 us) and 124
// rows 360 us (two splits + reduce: 351 + 30 us).
struct HeadPlan {
  bool rk = false, top2 = false;
  GemmPlan rkp;
  ActPlan ap;
};

HeadPlan lm_head_plan(const dflash_dims* d, int M) {
  HeadPlan h;
  h.rkp = plan_gemm_rk(M, d->V, d->D, true);
  if (h.rkp.rk) {
    h.rk = true;
    return h;
  }
  h.ap = plan_act(M, d->V, d->D, true);
  const char* knob = getenv("DFLASH_HEAD_TILED");   // 2: the plain GEMM plan (measurement)
  if (knob == nullptr || atoi(knob) != 2) {
    GemmPlan t = plan_gemm_tiled(M, d->V, d->D, A_BF16_HILO);
    t.cps = d->D / 64;                        // one split: every 64-wide k tile
    t.S = 1;
    t.part_floats = 0;
    h.ap = ActPlan{t, A_BF16_HILO};
  }
  h.top2 = h.ap.kind == A_BF16_HILO && h.ap.p.S == 1;
  return h;
}

// LM head: split-K partials [S][M][V], then per-128-column top-2 [ceil(V/128)][M][3]
struct ArgmaxWs {
  size_t part, top2, rows, planes, total;
};

// M mask rows (logits rows); `gathered` adds room for them as a dense [M][D]
// block (a ragged batch's mask rows are gathered before the LM head).
ArgmaxWs argmax_ws(const dflash_dims* d, int M, bool gathered = false) {
  ArgmaxWs w{};
  Carve c;
  if (gathered) w.rows = c.take(static_cast<size_t>(M) * d->D * 4);
  if (d->dtype == DFLASH_F32) {
    w.part = c.take(static_cast<size_t>(M) * d->V * 4);
  } else {
    const HeadPlan hp = lm_head_plan(d, M);
    size_t pf = hp.rk ? 0 : hp.ap.p.part_floats;
    const size_t pf_stream = plan_gemm_mfma(M, d->V, d->D, A_F32_SPLIT, true).part_floats;
    if (pf_stream > pf) pf = pf_stream;
    w.part = c.take(pf * 4);
    w.planes = c.take(hp.rk ? 0 : act_planes_bytes(hp.ap, M, d->D));
    // top-2 candidates: one row per 512-column reduce tile, 256-column tiled
    // GEMM tile, or register-K workgroup
    size_t t2 = static_cast<size_t>((d->V + 255) / 256);
    if (t2 < static_cast<size_t>(kRkMaxGrid)) t2 = kRkMaxGrid;
    if (!hp.rk && static_cast<size_t>(hp.ap.p.ntiles) > t2) t2 = hp.ap.p.ntiles;   // one per n-tile of the plan
    w.top2 = c.take(t2 * M * 3 * 4);
  }
  w.total = c.off;
  return w;
}

// Sampled drafting: the LM head's split-K partials (streaming kernel, bf16
// weights with more than 16 rows) and the per-row sampling statistics
// [pieces][M] (one piece per register-K workgroup or per column chunk).
struct SampleWs {
  size_t part, stats, planes, total;
};

SampleWs sample_ws(const dflash_dims* d, int B, int gamma) {
  const int M = B * (gamma - 1);
  SampleWs w{};
  Carve c;
  const int chunk = sample_chunk(d->V, M);
  const size_t nchunk = static_cast<size_t>((d->V + chunk - 1) / chunk);
  size_t pieces = nchunk;
  if (d->dtype == DFLASH_BF16) {
    const GemmPlan rk = plan_gemm_rk(M, d->V, d->D, true);
    if (rk.rk) {
      if (static_cast<size_t>(rk.grid) > pieces) pieces = rk.grid;
    } else {
      const ActPlan ap = plan_act(M, d->V, d->D, true);
      w.part = c.take(ap.p.part_floats * 4);
      w.planes = c.take(act_planes_bytes(ap, M, d->D));
    }
  }
  w.stats = c.take(pieces * M * sizeof(float4));
  w.total = c.off;
  return w;
}

// Sampled verification: row statistics of the target rows (and of the draft
// rows when their log-normalisers are not given), the per-chunk candidate
// draws and the first-rejection index.
struct AcceptWs {
  size_t stats, part, m, total;
  int chunk, nchunk, rows;
};

AcceptWs sample_accept_ws(const dflash_dims* d, int B, int gamma, bool lse_given) {
  const int n = gamma - 1;
  AcceptWs w{};
  w.chunk = sample_chunk(d->V, B * (n + 1) + (lse_given ? 0 : B * n));
  w.nchunk = (d->V + w.chunk - 1) / w.chunk;
  w.rows = B * (n + 1) + (lse_given ? 0 : B * n);
  Carve c;
  w.stats = c.take(static_cast<size_t>(w.nchunk) * w.rows * sizeof(float4));
  w.part = c.take(static_cast<size_t>(B) * ((d->V + kSpecDrawChunk - 1) / kSpecDrawChunk) * sizeof(float4));
  w.m = c.take(static_cast<size_t>(B) * 4);
  w.total = c.off;
  return w;
}

// The target's verify pass over B blocks of gamma rows: the drafting pass's
// workspace, then the final states [M][D] and the LM head's over all M rows.
struct VerifyWs {
  size_t hf, head, total;
  DraftWs draft;
  ArgmaxWs argmax;
};

VerifyWs verify_ws(const dflash_dims* d, int B, int gamma) {
  VerifyWs w{};
  const int M = B * gamma;
  w.draft = draft_ws(d, B, M, gamma);
  w.argmax = argmax_ws(d, M);
  Carve c;
  c.take(w.draft.total);
  w.hf = c.take(static_cast<size_t>(M) * d->D * 4);
  w.head = c.take(w.argmax.total);
  w.total = c.off;
  return w;
}

dflash_status check_temperature(float T) {
  DF_REQUIRE(std::isfinite(T) && T > 0.f && std::isfinite(1.0f / T), DFLASH_ERR_INVALID_ARG,
             "temperature=%g must be positive and finite (with a finite reciprocal)", static_cast<double>(T));
  return DFLASH_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// ---------------------------------------------------------- profiling hook
struct ProfHook {
  int role = DFLASH_PROF_NONE;
  void* const* start = nullptr;
  void* const* stop = nullptr;
  int n = 0, idx = 0;
};
thread_local ProfHook g_prof;

// If this launch matches the hook's role, hand its next event pair to the
// role's kernel launch (recorded as part of that kernel's dispatch, so the
// interval is the kernel's own run); returns the slot used.  The verify role
// brackets two launches and records its events on the stream instead.
int prof_begin(int role, hipStream_t s) {
  if (g_prof.role != role || g_prof.idx >= g_prof.n) return -1;
  const int i = g_prof.idx++;
  if (role == DFLASH_PROF_VERIFY) {
    if (hipEventRecord(static_cast<hipEvent_t>(g_prof.start[i]), s) != hipSuccess) return -1;
    return i;
  }
  pending_events() = PendingEvents{static_cast<hipEvent_t>(g_prof.start[i]), static_cast<hipEvent_t>(g_prof.stop[i])};
  return i;
}

void prof_end(int slot, hipStream_t s) {
  if (slot < 0) return;
  if (g_prof.role == DFLASH_PROF_VERIFY) {
    (void)hipEventRecord(static_cast<hipEvent_t>(g_prof.stop[slot]), s);
    return;
  }
  // a launch path that did not take the events (none should): record them
  // back to back so the pair is still complete
  PendingEvents& pe = pending_events();
  if (pe.start != nullptr) {
    (void)hipEventRecord(pe.start, s);
    (void)hipEventRecord(pe.stop, s);
    pe = PendingEvents{};
  }
}

}  // namespace

extern "C" {

const char* dflash_version(void) { return "dflash-mi355x 0.1.0 (gfx950)"; }

dflash_status dflash_profile_events(int32_t role, void* const* start, void* const* stop, int32_t n,
                                    int32_t* recorded) {
  DF_REQUIRE(role >= DFLASH_PROF_NONE && role <= DFLASH_PROF_VERIFY, DFLASH_ERR_INVALID_ARG,
             "unknown profiling role %d", role);
  DF_REQUIRE(n >= 0, DFLASH_ERR_INVALID_ARG, "n=%d < 0", n);
  DF_REQUIRE(role == DFLASH_PROF_NONE || n == 0 || (start != nullptr && stop != nullptr), DFLASH_ERR_INVALID_ARG,
             "event arrays are NULL");
  if (recorded != nullptr) *recorded = g_prof.idx;
  g_prof = ProfHook{};
  if (role != DFLASH_PROF_NONE && n > 0) {
    g_prof.role = role;
    g_prof.start = start;
    g_prof.stop = stop;
    g_prof.n = n;
  }
  return ok();
}

const char* dflash_last_error(void) { return g_err.c_str(); }

// Two anchored blocks of gamma rows may share a query group: bf16 weights, an
// fp32 cache (the attention kernel that masks each row to its own block) and
// both blocks' query rows within the 128 rows one attention workgroup takes.
static bool pairs_fit(const dflash_dims* d, int gamma) {
  return d->dtype == DFLASH_BF16 && d->cache_dtype == DFLASH_F32 && 2 * (d->Hq / d->Hkv) * gamma <= 128;
}

dflash_status dflash_workspace_size(const dflash_dims* dims, int32_t B, int32_t gamma, int32_t max_rows,
                                    size_t* bytes) {
  dflash_status st = check_dims(dims);
  if (st != DFLASH_OK) return st;
  if ((st = check_gamma(gamma)) != DFLASH_OK) return st;
  DF_REQUIRE(B >= 1 && B <= DFLASH_MAX_BATCH, DFLASH_ERR_INVALID_ARG, "B=%d outside [1, %d]", B, DFLASH_MAX_BATCH);
  DF_REQUIRE(max_rows >= 0, DFLASH_ERR_INVALID_ARG, "max_rows=%d < 0", max_rows);
  DF_REQUIRE(bytes != nullptr, DFLASH_ERR_INVALID_ARG, "bytes is NULL");
  // The kernels chosen (and so the scratch they need) depend on the row counts,
  // not monotonically: take the maximum over every row count that a call with
  // at most B sequences and blocks of at most gamma rows can have, uniform or
  // ragged (the attention bound grows with B and the longest block).
  size_t need = 0;
  auto upd = [&](size_t x) { need = x > need ? x : need; };
  for (int M = DFLASH_MIN_GAMMA; M <= B * gamma; ++M) {
    upd(draft_ws(dims, B, M, gamma).total);
    if (pairs_fit(dims, gamma)) upd(draft_ws(dims, B, M, 2 * gamma).total);   // anchored blocks two to a group
  }
  for (int M = 1; M <= B * (gamma - 1); ++M) upd(argmax_ws(dims, M, true).total);
  for (int g = 1; g <= gamma; ++g)
    for (int b = 1; b <= B; ++b) upd(verify_ws(dims, b, g).total);
  for (int b = 1; b <= B; ++b)
    for (int g = DFLASH_MIN_GAMMA; g <= gamma; ++g) {
      upd(sample_ws(dims, b, g).total);
      upd(sample_accept_ws(dims, b, g, false).total);
      upd(sample_accept_ws(dims, b, g, true).total);
    }
  const size_t f = fuse_ws(dims, max_rows), i = inject_ws(dims, max_rows);
  if (f > need) need = f;
  if (i > need) need = i;
  *bytes = need;
  return ok();
}

dflash_status dflash_fuse_context(const dflash_dims* dims, const dflash_weights* w, const void* const* h_tgt,
                                  int64_t ld, int32_t T, void* H_t, void* ws, size_t ws_bytes, void* stream) {
  dflash_status st = check_dims(dims);
  if (st != DFLASH_OK) return st;
  DF_REQUIRE(w != nullptr, DFLASH_ERR_INVALID_ARG, "weights is NULL");
  DF_REQUIRE(T >= 0, DFLASH_ERR_INVALID_ARG, "T=%d < 0", T);
  if (T == 0) return ok();
  if ((st = check_ptr(w->w_c, "w_c")) != DFLASH_OK) return st;
  if ((st = check_ptr(w->g_c, "g_c")) != DFLASH_OK) return st;
  if ((st = check_ptr(H_t, "H_t")) != DFLASH_OK) return st;
  DF_REQUIRE(h_tgt != nullptr, DFLASH_ERR_INVALID_ARG, "h_tgt is NULL");
  DF_REQUIRE(ld >= dims->D && (ld * static_cast<int64_t>(esize(dims))) % 16 == 0, DFLASH_ERR_INVALID_ARG,
             "ld=%lld must be >= D and keep rows 16-byte aligned", static_cast<long long>(ld));
  for (int k = 0; k < dims->n_tgt_layers; ++k)
    if ((st = check_ptr(h_tgt[k], "h_tgt[k]")) != DFLASH_OK) return st;
  const size_t need = fuse_ws(dims, T);
  if ((st = check_ws(ws, ws_bytes, need)) != DFLASH_OK) return st;
  if ((st = check_device()) != DFLASH_OK) return st;

  const bool bf = dims->dtype == DFLASH_BF16, cbf = dims->cache_dtype == DFLASH_BF16;
  const int D = dims->D, K = dims->n_tgt_layers * D;
  const size_t es = esize(dims), cs = csize(dims);
  float* part = static_cast<float*>(ws);
  hipStream_t s = as_stream(stream);
  for (int r0 = 0; r0 < T; r0 += kRowBlock) {
    const int M = T - r0 < kRowBlock ? T - r0 : kRowBlock;
    GemmArgs g{};
    for (int k = 0; k < dims->n_tgt_layers; ++k)
      g.a_src[k] = static_cast<const char*>(h_tgt[k]) + static_cast<int64_t>(r0) * ld * es;
    for (int k = dims->n_tgt_layers; k < kMaxSrc; ++k) g.a_src[k] = g.a_src[0];
    g.a_cols = D;
    g.a_rg = INT_MAX;
    g.a_ld = ld;
    g.a_gs = 0;
    g.w = w->w_c;
    g.w_ld = K;
    g.w_rg = INT_MAX;
    g.w_gs = 0;
    g.w_off = 0;
    g.M = M;
    g.N = D;
    g.K = K;
    g.part = part;
    int S = 1;
    if (bf) {
      const GemmPlan p = plan_gemm(M, D, K, A_BF16, false);
      S = p.S;
      const int ps = prof_begin(DFLASH_PROF_FUSE, s);
      DF_HIP_PROF(launch_gemm_mfma(g, A_BF16, p, s), ps);
    } else {
      DF_HIP(launch_gemm_f32(g, s));
    }
    DF_HIP(launch_ctx_norm(part, S, M, D, w->g_c, dims->rms_eps,
                           static_cast<char*>(H_t) + static_cast<int64_t>(r0) * D * cs, bf, cbf, s));
  }
  return ok();
}

dflash_status dflash_inject_kv(const dflash_dims* dims, const dflash_weights* w, const void* H_t,
                               const int32_t* rows_per_seq, dflash_kv_cache* cache, void* ws, size_t ws_bytes,
                               void* stream) {
  dflash_status st = check_dims(dims);
  if (st != DFLASH_OK) return st;
  DF_REQUIRE(w != nullptr, DFLASH_ERR_INVALID_ARG, "weights is NULL");
  if ((st = check_cache(cache)) != DFLASH_OK) return st;
  DF_REQUIRE(rows_per_seq != nullptr, DFLASH_ERR_INVALID_ARG, "rows_per_seq is NULL");
  int64_t total = 0;
  for (int b = 0; b < cache->B; ++b) {
    DF_REQUIRE(rows_per_seq[b] >= 0, DFLASH_ERR_INVALID_ARG, "rows_per_seq[%d]=%d < 0", b, rows_per_seq[b]);
    DF_REQUIRE(static_cast<int64_t>(cache->len[b]) + rows_per_seq[b] <= cache->cap, DFLASH_ERR_CAPACITY,
               "sequence %d: len %d + %d rows exceeds cap %d", b, cache->len[b], rows_per_seq[b], cache->cap);
    total += rows_per_seq[b];
  }
  DF_REQUIRE(total < INT_MAX, DFLASH_ERR_INVALID_ARG, "too many rows");
  if (total == 0) return ok();
  if ((st = check_ptr(w->w_qkv, "w_qkv")) != DFLASH_OK) return st;
  if ((st = check_ptr(H_t, "H_t")) != DFLASH_OK) return st;
  const size_t need = inject_ws(dims, static_cast<int>(total));
  if ((st = check_ws(ws, ws_bytes, need)) != DFLASH_OK) return st;
  if ((st = check_device()) != DFLASH_OK) return st;

  const bool bf = dims->dtype == DFLASH_BF16, cbf = dims->cache_dtype == DFLASH_BF16;
  const int D = dims->D, d = dims->head_dim, Hkv = dims->Hkv;
  const int N = 2 * dims->L * Hkv * d;
  const size_t cs = csize(dims);
  float* part = static_cast<float*>(ws);
  hipStream_t s = as_stream(stream);
  int row_off[kMaxSeq + 1];
  row_off[0] = 0;
  for (int b = 0; b < cache->B; ++b) row_off[b + 1] = row_off[b] + rows_per_seq[b];
  const int T = static_cast<int>(total);
  for (int r0 = 0; r0 < T; r0 += kRowBlock) {
    const int M = T - r0 < kRowBlock ? T - r0 : kRowBlock;
    GemmArgs g{};
    for (int k = 0; k < kMaxSrc; ++k) g.a_src[k] = static_cast<const char*>(H_t) + static_cast<int64_t>(r0) * D * cs;
    g.a_cols = D;
    g.a_rg = INT_MAX;
    g.a_ld = D;
    g.a_gs = 0;
    g.w = w->w_qkv;
    g.w_ld = D;
    g.w_rg = 2 * Hkv * d;
    g.w_gs = static_cast<int64_t>(dims->Hq + 2 * Hkv) * d;
    g.w_off = static_cast<int64_t>(dims->Hq) * d;
    g.M = M;
    g.N = N;
    g.K = D;
    g.part = part;
    int S = 1;
    if (bf) {
      // an fp32 H_t is split hi + lo against the bf16 weights like any fp32
      // activation: on the fly, or (many rows, tiled GEMM) once into two planes
      const GemmAKind kind = inject_kind(dims, M);
      const GemmPlan p = plan_gemm(M, N, D, kind, false);
      S = p.S;
      if (kind == A_BF16_HILO) {
        uint16_t* hi = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + align_up(p.part_floats * 4));
        uint16_t* lo = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(hi) + align_up(static_cast<size_t>(M) * D * 2));
        DF_HIP(launch_split_hilo(static_cast<const float*>(g.a_src[0]), D, M, D, hi, lo, s));
        for (int k = 0; k < kMaxSrc; ++k) g.a_src[k] = hi;
        g.a_lo = lo;
      }
      const int ps = prof_begin(DFLASH_PROF_INJECT, s);
      DF_HIP_PROF(launch_gemm_mfma(g, kind, p, s), ps);
    } else {
      DF_HIP(launch_gemm_f32(g, s));
    }
    ScatterArgs sa{};
    sa.part = part;
    sa.S = S;
    sa.M = M;
    sa.N = N;
    sa.nq = 0;
    sa.q_out = nullptr;
    sa.kc = cache->k;
    sa.vc = cache->v;
    sa.layer0 = 0;
    sa.B = cache->B;
    sa.Hkv = Hkv;
    sa.d = d;
    sa.cap = cache->cap;
    sa.rows.B = cache->B;
    for (int b = 0; b < cache->B; ++b) {
      const int lo = row_off[b] - r0, hi = row_off[b + 1] - r0;
      sa.rows.row_off[b] = lo < 0 ? 0 : (lo > M ? M : lo);
      sa.rows.pos0[b] = cache->len[b] + (r0 > row_off[b] ? r0 - row_off[b] : 0);
      sa.rows.seq[b] = b;
      (void)hi;
    }
    sa.rows.row_off[cache->B] = M;
    sa.len_dev = r0 + kRowBlock >= T ? cache->len_dev : nullptr;   // the last pass updates the mirror
    for (int b = 0; b < cache->B; ++b) sa.len_new[b] = cache->len[b] + rows_per_seq[b];
    DF_HIP(launch_scatter_kv(sa, cbf, s));
  }
  for (int b = 0; b < cache->B; ++b) cache->len[b] += rows_per_seq[b];
  return ok();
}

// Query groups of a drafting pass (validated by the caller).  Group b has
// gam[b] block rows (packed row after row), reads the K/V of cache sequence
// kvseq[b], sees that sequence's context rows [0, nctx[b]) and its own rows,
// and writes its own K/V to cache rows [pos0[b], pos0[b] + gam[b]).  At
// inference pos0 = nctx = len: the block follows the context.  Anchored blocks
// (apart) keep their rows in a scratch region past the context, read as a key
// item of their own.
// Two anchored blocks of one sequence can share a group (gam = both blocks'
// rows, the first block's half[b] rows first): their own rows then sit
// together from pos0[b], the first block sees context rows [0, nctx[b]) and
// the second [0, nctx2[b]), each only its own block rows.
struct QueryGroups {
  int n = 0;
  bool apart = false;
  int32_t gam[kMaxSeq], kvseq[kMaxSeq], nctx[kMaxSeq], pos0[kMaxSeq];
  int32_t half[kMaxSeq], nctx2[kMaxSeq];
};

// A pass run as the target model's verify forward: causal attention inside
// the block, and the residual stream after some layers stored (tapped).
struct TargetPass {
  int n_taps = 0;
  int32_t layer[DFLASH_MAX_TGT_LAYERS];
  void* out[DFLASH_MAX_TGT_LAYERS];   // [M][D] weight type each
};

static dflash_status draft_forward_impl(const dflash_dims* dims, const dflash_weights* w,
                                        const dflash_kv_cache* cache, const int32_t* block_tokens,
                                        const float* embed_override, const QueryGroups& qg, float* h_final,
                                        void* ws, size_t ws_bytes, void* stream,
                                        const TargetPass* tp = nullptr) {
  dflash_status st = DFLASH_OK;
  int M = 0, gmax = 0;
  int32_t qrow0[kMaxSeq + 1];
  for (int b = 0; b < qg.n; ++b) {
    qrow0[b] = M;
    M += qg.gam[b];
    gmax = qg.gam[b] > gmax ? qg.gam[b] : gmax;
  }
  qrow0[qg.n] = M;
  const char* names[] = {"w_qkv", "w_o", "w_gateup", "w_down", "g_attn", "g_ffn", "g_final"};
  const void* ptrs[] = {w->w_qkv, w->w_o, w->w_gateup, w->w_down, w->g_attn, w->g_ffn, w->g_final};
  for (int i = 0; i < 7; ++i)
    if ((st = check_ptr(ptrs[i], names[i])) != DFLASH_OK) return st;
  if (embed_override != nullptr) {
    if ((st = check_ptr(embed_override, "embed_override")) != DFLASH_OK) return st;
  } else {
    if ((st = check_ptr(w->embed, "embed")) != DFLASH_OK) return st;
    DF_REQUIRE(block_tokens != nullptr, DFLASH_ERR_INVALID_ARG, "block_tokens is NULL (and no embed_override)");
  }
  if ((st = check_ptr(h_final, "h_final")) != DFLASH_OK) return st;
  const int B = qg.n;   // query groups (sequences, or anchored blocks)
  if ((st = check_attention_cache(dims, cache)) != DFLASH_OK) return st;
  const DraftWs lay = draft_ws(dims, B, M, gmax);
  if ((st = check_ws(ws, ws_bytes, lay.total)) != DFLASH_OK) return st;
  if ((st = check_device()) != DFLASH_OK) return st;

  const bool bf = dims->dtype == DFLASH_BF16, cbf = dims->cache_dtype == DFLASH_BF16;
  const int D = dims->D, d = dims->head_dim, Hq = dims->Hq, Hkv = dims->Hkv, F = dims->F, L = dims->L;
  const int hd = Hq * d, nqkv = (Hq + 2 * Hkv) * d;
  const size_t es = esize(dims), cs = csize(dims);
  char* base = static_cast<char*>(ws);
  float* h = reinterpret_cast<float*>(base + lay.h);
  float* a = reinterpret_cast<float*>(base + lay.a);
  float* q = reinterpret_cast<float*>(base + lay.q);
  float* o = reinterpret_cast<float*>(base + lay.o);
  float* sw = reinterpret_cast<float*>(base + lay.s);
  float* part = reinterpret_cast<float*>(base + lay.part);
  hipStream_t s = as_stream(stream);
  auto wp = [&](const void* p, int64_t elems) { return static_cast<const char*>(p) + elems * es; };

  // Activation planes: when a GEMM takes the tiled kernel (many rows) its
  // producer (embedding / residual norm, attention combine, SwiGLU) writes the
  // bf16 hi / lo planes of its output directly, and the GEMM skips its split.
  const ActPlan ap_qkv = bf ? plan_act(M, nqkv, D, false) : ActPlan{};
  const ActPlan ap_o = bf ? plan_act(M, D, hd, false) : ActPlan{};
  const ActPlan ap_gu = bf ? plan_act(M, 2 * F, D, false) : ActPlan{};
  const ActPlan ap_dn = bf ? plan_act(M, D, F, false) : ActPlan{};
  void* planes = base + lay.planes;
  const HiLo pl_qkv = bf ? act_planes(ap_qkv, planes, M, D) : HiLo{};
  const HiLo pl_o = bf ? act_planes(ap_o, planes, M, hd) : HiLo{};
  const HiLo pl_gu = bf ? act_planes(ap_gu, planes, M, D) : HiLo{};
  const HiLo pl_dn = bf ? act_planes(ap_dn, planes, M, F) : HiLo{};

  // GEMM on fp32 activations (rows = block rows), returns the split count;
  // ready: A's planes were written by its producer.
  auto gemm = [&](const float* A, int K, const void* W, int N, int* S, int role, bool ready) -> hipError_t {
    GemmArgs g{};
    for (int k = 0; k < kMaxSrc; ++k) g.a_src[k] = A;
    g.a_cols = K;
    g.a_rg = INT_MAX;
    g.a_ld = K;
    g.a_gs = 0;
    g.w = W;
    g.w_ld = K;
    g.w_rg = INT_MAX;
    g.w_gs = 0;
    g.w_off = 0;
    g.M = M;
    g.N = N;
    g.K = K;
    g.part = part;
    if (!bf) {
      *S = 1;
      return launch_gemm_f32(g, s);
    }
    const ActPlan ap = plan_act(M, N, K, false);
    *S = ap.p.S;
    const int ps = prof_begin(role, s);
    const hipError_t e = launch_act_gemm(g, ap, planes, s, ready);
    prof_end(ps, s);
    return e;
  };

  int32_t nkeys[kMaxSeq], apart[kMaxSeq];
  for (int b = 0; b < B; ++b) {
    nkeys[b] = qg.apart ? std::max(qg.nctx[b], qg.nctx2[b]) : qg.nctx[b] + qg.gam[b];
    apart[b] = qg.apart ? 1 : 0;
  }
  const int R = (Hq / Hkv) * gmax;
  const AttnPlan ap = bf ? plan_attention(B, nkeys, Hkv, R, d, apart) : AttnPlan{};
  // one layer of the cache holds all cache->B sequences (B counts query groups)
  const size_t layer_elems = static_cast<size_t>(cache->B) * Hkv * cache->cap * d;

  const GemmPlan swiglu_rk = bf ? plan_gemm_rk_swiglu(M, F, D) : GemmPlan{};
  DF_HIP(launch_embed_norm(block_tokens, embed_override, w->embed, dims->V, M, D, w->g_attn, dims->rms_eps, h, a, bf, s,
                           pl_qkv));
  for (int l = 0; l < L; ++l) {
    int S = 1;
    DF_HIP(gemm(a, D, wp(w->w_qkv, static_cast<int64_t>(l) * nqkv * D), nqkv, &S, DFLASH_PROF_QKV,
                pl_qkv.hi != nullptr));
    ScatterArgs sa{};
    sa.part = part;
    sa.S = S;
    sa.M = M;
    sa.N = nqkv;
    sa.nq = hd;
    sa.q_out = q;
    sa.kc = cache->k;
    sa.vc = cache->v;
    sa.layer0 = l;
    sa.B = cache->B;
    sa.Hkv = Hkv;
    sa.d = d;
    sa.cap = cache->cap;
    sa.rows.B = B;
    for (int b = 0; b < B; ++b) {
      sa.rows.row_off[b] = qrow0[b];
      sa.rows.pos0[b] = qg.pos0[b];
      sa.rows.seq[b] = qg.kvseq[b];
    }
    sa.rows.row_off[B] = M;
    DF_HIP(launch_scatter_kv(sa, cbf, s));

    AttnArgs at{};
    at.q = q;
    at.kc = static_cast<const char*>(cache->k) + l * layer_elems * cs;
    at.vc = static_cast<const char*>(cache->v) + l * layer_elems * cs;
    at.part_o = reinterpret_cast<float*>(base + lay.att_o);
    at.part_ml = reinterpret_cast<float*>(base + lay.att_ml);
    at.o_out = o;
    at.o_hi = pl_o.hi;
    at.o_lo = pl_o.lo;
    at.B = B;
    at.Hq = Hq;
    at.Hkv = Hkv;
    at.d = d;
    at.cap = cache->cap;
    at.R = R;
    at.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(d)));
    at.causal = tp != nullptr ? 1 : 0;
    for (int b = 0; b < B; ++b) {
      at.nkeys[b] = nkeys[b];
      at.gam[b] = qg.gam[b];
      at.qrow0[b] = qrow0[b];
      at.kvseq[b] = qg.kvseq[b];
      at.blk0[b] = qg.apart ? qg.pos0[b] : -1;
      at.half[b] = qg.half[b];
      at.ctx1[b] = qg.apart ? qg.nctx[b] : nkeys[b];
      at.ctx2[b] = qg.apart ? qg.nctx2[b] : nkeys[b];
    }
    at.qrow0[B] = M;
    const int pa = prof_begin(DFLASH_PROF_ATTENTION, s);
    const hipError_t ea = launch_attention(at, ap, bf, cbf, s);
    prof_end(pa, s);
    DF_HIP(ea);

    DF_HIP(gemm(o, hd, wp(w->w_o, static_cast<int64_t>(l) * D * hd), D, &S, DFLASH_PROF_O, pl_o.hi != nullptr));
    DF_HIP(launch_residual_norm(part, S, M, D, h, wp(w->g_ffn, static_cast<int64_t>(l) * D), dims->rms_eps, a, bf, s,
                                swiglu_rk.rk ? HiLo{} : pl_gu));
    if (swiglu_rk.rk) {
      // gate/up GEMM with SwiGLU in its epilogue
      GemmArgs g{};
      for (int k = 0; k < kMaxSrc; ++k) g.a_src[k] = a;
      g.a_cols = D;
      g.a_rg = INT_MAX;
      g.a_ld = D;
      g.w = wp(w->w_gateup, static_cast<int64_t>(l) * 2 * F * D);
      g.w_ld = D;
      g.w_rg = INT_MAX;
      g.M = M;
      g.N = F;
      g.K = D;
      const int ps = prof_begin(DFLASH_PROF_GATEUP, s);
      const hipError_t e = launch_gemm_rk_swiglu(g, swiglu_rk, sw, s);
      prof_end(ps, s);
      DF_HIP(e);
    } else {
      DF_HIP(gemm(a, D, wp(w->w_gateup, static_cast<int64_t>(l) * 2 * F * D), 2 * F, &S, DFLASH_PROF_GATEUP,
                  pl_gu.hi != nullptr));
      DF_HIP(launch_swiglu(part, S, M, F, sw, s, pl_dn));
    }
    DF_HIP(gemm(sw, F, wp(w->w_down, static_cast<int64_t>(l) * D * F), D, &S, DFLASH_PROF_DOWN,
                pl_dn.hi != nullptr && !swiglu_rk.rk));
    const bool last = l + 1 == L;
    void* tap = nullptr;
    for (int k = 0; tp != nullptr && k < tp->n_taps; ++k)
      if (tp->layer[k] == l) tap = tp->out[k];
    DF_HIP(launch_residual_norm(part, S, M, D, h,
                                last ? w->g_final : wp(w->g_attn, static_cast<int64_t>(l + 1) * D),
                                dims->rms_eps, last ? h_final : a, bf, s, last ? HiLo{} : pl_qkv, tap));
  }
  return ok();
}

// Inference groups: sequence b's block of gammas[b] rows follows its context.
static dflash_status inference_groups(const dflash_dims* dims, const dflash_weights* w,
                                      const dflash_kv_cache* cache, const int32_t* gammas, QueryGroups* qg) {
  dflash_status st = check_dims(dims);
  if (st != DFLASH_OK) return st;
  DF_REQUIRE(w != nullptr, DFLASH_ERR_INVALID_ARG, "weights is NULL");
  if ((st = check_cache(cache)) != DFLASH_OK) return st;
  DF_REQUIRE(gammas != nullptr, DFLASH_ERR_INVALID_ARG, "gammas is NULL");
  qg->n = cache->B;
  qg->apart = false;
  for (int b = 0; b < cache->B; ++b) {
    if ((st = check_gamma(gammas[b])) != DFLASH_OK) return st;
    DF_REQUIRE(static_cast<int64_t>(cache->len[b]) + gammas[b] <= cache->cap, DFLASH_ERR_CAPACITY,
               "sequence %d: len %d + gamma %d exceeds cap %d", b, cache->len[b], gammas[b], cache->cap);
    qg->gam[b] = gammas[b];
    qg->half[b] = gammas[b];
    qg->kvseq[b] = b;
    qg->nctx[b] = qg->nctx2[b] = qg->pos0[b] = cache->len[b];
  }
  return DFLASH_OK;
}

dflash_status dflash_draft_forward(const dflash_dims* dims, const dflash_weights* w, const dflash_kv_cache* cache,
                                   const int32_t* block_tokens, const float* embed_override, int32_t gamma,
                                   float* h_final, void* ws, size_t ws_bytes, void* stream) {
  dflash_status st = check_gamma(gamma);
  if (st != DFLASH_OK) return st;
  if ((st = check_cache(cache)) != DFLASH_OK) return st;
  int32_t gammas[kMaxSeq];
  for (int b = 0; b < cache->B; ++b) gammas[b] = gamma;
  QueryGroups qg;
  if ((st = inference_groups(dims, w, cache, gammas, &qg)) != DFLASH_OK) return st;
  return draft_forward_impl(dims, w, cache, block_tokens, embed_override, qg, h_final, ws, ws_bytes, stream);
}

// ---------------------------------------------------- no-allocation variant
// dflash_draft_forward_noalloc keeps the pass's workspace in this static
// device array instead of a caller buffer: one copy per GPU, alive until the
// process ends.  Host code never uses the array's name as an address (on the
// host it only names the symbol): the device address comes from
// hipGetSymbolAddress, looked up once per device and kept in g_scratch.
constexpr size_t kScratchBytes = size_t{96} << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch[64] = {};

// The current device's address of `scratch` (looked up on first use there).
dflash_status scratch_address(void** out) {
  int dev = 0;
  DF_HIP(hipGetDevice(&dev));
  DF_REQUIRE(dev >= 0 && dev < 64, DFLASH_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    DF_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    DF_REQUIRE(p != nullptr && (reinterpret_cast<uintptr_t>(p) % kAlign) == 0, DFLASH_ERR_HIP,
               "scratch address %p is not %zu-byte aligned", p, kAlign);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return DFLASH_OK;
}
}  // namespace

dflash_status dflash_draft_forward_noalloc(const dflash_dims* dims, const dflash_weights* w,
                                           const dflash_kv_cache* cache, const int32_t* block_tokens,
                                           const float* embed_override, int32_t gamma, float* h_final,
                                           void* stream) {
  dflash_status st = check_gamma(gamma);
  if (st != DFLASH_OK) return st;
  if ((st = check_cache(cache)) != DFLASH_OK) return st;
  int32_t gammas[kMaxSeq];
  for (int b = 0; b < cache->B; ++b) gammas[b] = gamma;
  QueryGroups qg;
  if ((st = inference_groups(dims, w, cache, gammas, &qg)) != DFLASH_OK) return st;
  const size_t need = draft_ws(dims, cache->B, cache->B * gamma, gamma).total;
  DF_REQUIRE(need <= kScratchBytes, DFLASH_ERR_WORKSPACE,
             "this pass needs %zu bytes of scratch; the no-allocation call holds %zu (use dflash_draft_forward "
             "with a workspace)", need, kScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != DFLASH_OK) return st;
  return draft_forward_impl(dims, w, cache, block_tokens, embed_override, qg, h_final, ws, kScratchBytes, stream);
}

dflash_status dflash_draft_forward_ragged(const dflash_dims* dims, const dflash_weights* w,
                                          const dflash_kv_cache* cache, const int32_t* block_tokens,
                                          const float* embed_override, const int32_t* gammas, float* h_final,
                                          void* ws, size_t ws_bytes, void* stream) {
  QueryGroups qg;
  const dflash_status st = inference_groups(dims, w, cache, gammas, &qg);
  if (st != DFLASH_OK) return st;
  return draft_forward_impl(dims, w, cache, block_tokens, embed_override, qg, h_final, ws, ws_bytes, stream);
}

dflash_status dflash_draft_forward_blocks(const dflash_dims* dims, const dflash_weights* w,
                                          const dflash_kv_cache* cache, const int32_t* block_seq,
                                          const int32_t* anchors, int32_t nblk, int32_t gamma,
                                          const int32_t* block_tokens, const float* embed_override, float* h_final,
                                          void* ws, size_t ws_bytes, void* stream) {
  dflash_status st = check_dims(dims);
  if (st != DFLASH_OK) return st;
  DF_REQUIRE(w != nullptr, DFLASH_ERR_INVALID_ARG, "weights is NULL");
  if ((st = check_cache(cache)) != DFLASH_OK) return st;
  if ((st = check_gamma(gamma)) != DFLASH_OK) return st;
  DF_REQUIRE(nblk >= 1 && nblk <= DFLASH_MAX_BATCH, DFLASH_ERR_INVALID_ARG, "nblk=%d outside [1, %d]", nblk,
             DFLASH_MAX_BATCH);
  DF_REQUIRE(block_seq != nullptr && anchors != nullptr, DFLASH_ERR_INVALID_ARG, "block_seq / anchors is NULL");
  for (int k = 0; k < nblk; ++k) {
    const int sq = block_seq[k];
    DF_REQUIRE(sq >= 0 && sq < cache->B, DFLASH_ERR_INVALID_ARG, "block %d: sequence %d outside [0, %d)", k, sq,
               cache->B);
    DF_REQUIRE(anchors[k] >= 0 && anchors[k] <= cache->len[sq], DFLASH_ERR_INVALID_ARG,
               "block %d: anchor %d outside [0, len %d]", k, anchors[k], cache->len[sq]);
  }
  // Consecutive blocks of one sequence share a query group (bf16 weights, fp32
  // cache: the attention kernel that reads each key tile once for both), so
  // that each context tile is read once for two blocks.  A group's own rows
  // take one 32-row-aligned slot past the sequence's context: ceil32(rows)
  // rows, never more than the two blocks' separate slots.
  const char* knob = getenv("DFLASH_BLOCK_PAIRS");   // 2: one block per group (measurement)
  const bool pairs = pairs_fit(dims, gamma) && (knob == nullptr || atoi(knob) != 2);
  QueryGroups qg;
  qg.n = 0;
  qg.apart = true;
  int64_t next[kMaxSeq];   // next free scratch row per sequence
  for (int b = 0; b < cache->B; ++b) next[b] = (static_cast<int64_t>(cache->len[b]) + 31) / 32 * 32;
  for (int k = 0; k < nblk;) {
    const int sq = block_seq[k];
    const bool two = pairs && k + 1 < nblk && block_seq[k + 1] == sq;
    const int rows = two ? 2 * gamma : gamma;
    const int64_t pos = next[sq];
    const int64_t slot = (rows + 31) / 32 * 32;
    DF_REQUIRE(pos + slot <= cache->cap, DFLASH_ERR_CAPACITY,
               "block %d: scratch rows [%lld, %lld) of sequence %d exceed cap %d", k, static_cast<long long>(pos),
               static_cast<long long>(pos + slot), sq, cache->cap);
    next[sq] = pos + slot;
    const int g = qg.n++;
    qg.gam[g] = rows;
    qg.half[g] = gamma;
    qg.kvseq[g] = sq;
    qg.nctx[g] = anchors[k];
    qg.nctx2[g] = two ? anchors[k + 1] : anchors[k];
    qg.pos0[g] = static_cast<int32_t>(pos);
    k += two ? 2 : 1;
  }
  return draft_forward_impl(dims, w, cache, block_tokens, embed_override, qg, h_final, ws, ws_bytes, stream);
}

// LM head + argmax over Mr activation rows that g's A mapping addresses (K = D).
static dflash_status lm_head_argmax(const dflash_dims* dims, const dflash_weights* w, GemmArgs g, int Mr,
                                    int32_t* draft, float* logits_dbg, float* top2_gap, char* base,
                                    const ArgmaxWs& lay, void* ws, hipStream_t s) {
  const int D = dims->D;
  g.w = w->lm_head;
  g.w_ld = D;
  g.w_rg = INT_MAX;
  g.w_gs = 0;
  g.w_off = 0;
  g.M = Mr;
  g.N = dims->V;
  g.K = D;
  if (dims->dtype == DFLASH_BF16) {
    g.part = reinterpret_cast<float*>(base + lay.part);
    float* top2 = reinterpret_cast<float*>(base + lay.top2);
    const HeadPlan hp = lm_head_plan(dims, Mr);
    if (hp.rk) {
      // one pass over the LM head: logits reduced in-register, top-2 per workgroup
      const int ps = prof_begin(DFLASH_PROF_LM_HEAD, s);
      DF_HIP_PROF(launch_gemm_rk(g, hp.rkp, top2, logits_dbg, s), ps);
      DF_HIP(launch_argmax_final(top2, hp.rkp.grid, Mr, draft, top2_gap, s));
    } else {
      const ActPlan& ap = hp.ap;
      if (hp.top2) {
        // tiled, one K split: each workgroup reduces its tile to a top-2 per
        // row (no logits round trip unless they are asked for)
        DF_HIP(prepare_act(g, ap, base + lay.planes, s, false));
        const int ps = prof_begin(DFLASH_PROF_LM_HEAD, s);
        DF_HIP_PROF(launch_gemm_tiled_top2(g, ap.p, top2, logits_dbg, s), ps);
        DF_HIP(launch_argmax_final(top2, ap.p.ntiles, Mr, draft, top2_gap, s));
      } else {
        const int ps = prof_begin(DFLASH_PROF_LM_HEAD, s);
        DF_HIP_PROF(launch_act_gemm(g, ap, base + lay.planes, s), ps);
        int nt = 0;
        DF_HIP(launch_reduce_top2(g.part, ap.p.S, Mr, dims->V, logits_dbg, top2, &nt, s));
        DF_HIP(launch_argmax_final(top2, nt, Mr, draft, top2_gap, s));
      }
    }
  } else {
    float* lg = logits_dbg != nullptr ? logits_dbg : reinterpret_cast<float*>(base + lay.part);
    g.part = lg;
    DF_HIP(launch_gemm_f32(g, s));
    DF_HIP(launch_argmax_rows(lg, Mr, dims->V, draft, top2_gap, s));
  }
  return ok();
}

dflash_status dflash_argmax_accept(const dflash_dims* dims, const dflash_weights* w, uint32_t flags,
                                   const float* h_final, int32_t B, int32_t gamma, int32_t* draft,
                                   const int32_t* target, int32_t* tau, int32_t* next_anchor, float* logits_dbg,
                                   float* top2_gap, void* ws, size_t ws_bytes, void* stream) {
  dflash_status st = check_dims(dims);
  if (st != DFLASH_OK) return st;
  if ((st = check_gamma(gamma)) != DFLASH_OK) return st;
  DF_REQUIRE(flags != 0 && (flags & ~(DFLASH_ARGMAX | DFLASH_ACCEPT)) == 0, DFLASH_ERR_INVALID_ARG,
             "flags=0x%x must be a non-empty subset of ARGMAX|ACCEPT", flags);
  DF_REQUIRE(B >= 1 && B <= DFLASH_MAX_BATCH, DFLASH_ERR_INVALID_ARG, "B=%d outside [1, %d]", B, DFLASH_MAX_BATCH);
  DF_REQUIRE(draft != nullptr, DFLASH_ERR_INVALID_ARG, "draft is NULL");
  const int n = gamma - 1, Mr = B * n, D = dims->D;
  size_t need = 0;
  if (flags & DFLASH_ARGMAX) {
    DF_REQUIRE(w != nullptr, DFLASH_ERR_INVALID_ARG, "weights is NULL");
    if ((st = check_ptr(w->lm_head, "lm_head")) != DFLASH_OK) return st;
    if ((st = check_ptr(h_final, "h_final")) != DFLASH_OK) return st;
    if (logits_dbg != nullptr && (st = check_ptr(logits_dbg, "logits_dbg")) != DFLASH_OK) return st;
    need = argmax_ws(dims, Mr).total;
  }
  if (flags & DFLASH_ACCEPT) {
    DF_REQUIRE(target != nullptr && tau != nullptr && next_anchor != nullptr, DFLASH_ERR_INVALID_ARG,
               "target, tau and next_anchor must be non-NULL for ACCEPT");
  }
  if ((st = check_ws(ws, ws_bytes, need)) != DFLASH_OK) return st;
  if ((st = check_device()) != DFLASH_OK) return st;

  hipStream_t s = as_stream(stream);
  if (flags & DFLASH_ARGMAX) {
    GemmArgs g{};
    for (int k = 0; k < kMaxSrc; ++k) g.a_src[k] = h_final + D;   // block row 1 of sequence 0
    g.a_cols = D;
    g.a_rg = n;
    g.a_gs = static_cast<int64_t>(gamma) * D;
    g.a_ld = D;
    if ((st = lm_head_argmax(dims, w, g, Mr, draft, logits_dbg, top2_gap, static_cast<char*>(ws),
                             argmax_ws(dims, Mr), ws, s)) != DFLASH_OK)
      return st;
  }
  if (flags & DFLASH_ACCEPT) DF_HIP(launch_accept(draft, target, B, n, tau, next_anchor, s));
  return ok();
}

dflash_status dflash_argmax_accept_ragged(const dflash_dims* dims, const dflash_weights* w, uint32_t flags,
                                          const float* h_final, int32_t B, const int32_t* gammas, int32_t* draft,
                                          const int32_t* target, int32_t* tau, int32_t* next_anchor,
                                          float* logits_dbg, float* top2_gap, void* ws, size_t ws_bytes,
                                          void* stream) {
  dflash_status st = check_dims(dims);
  if (st != DFLASH_OK) return st;
  DF_REQUIRE(flags != 0 && (flags & ~(DFLASH_ARGMAX | DFLASH_ACCEPT)) == 0, DFLASH_ERR_INVALID_ARG,
             "flags=0x%x must be a non-empty subset of ARGMAX|ACCEPT", flags);
  DF_REQUIRE(B >= 1 && B <= DFLASH_MAX_BATCH, DFLASH_ERR_INVALID_ARG, "B=%d outside [1, %d]", B, DFLASH_MAX_BATCH);
  DF_REQUIRE(gammas != nullptr, DFLASH_ERR_INVALID_ARG, "gammas is NULL");
  DF_REQUIRE(draft != nullptr, DFLASH_ERR_INVALID_ARG, "draft is NULL");
  // block rows of sequence b start at qrow0[b]; its drafts at doff[b]
  SeqRows mask{}, acc{};
  mask.B = acc.B = B;
  int M = 0, Mr = 0;
  for (int b = 0; b < B; ++b) {
    if ((st = check_gamma(gammas[b])) != DFLASH_OK) return st;
    mask.row_off[b] = Mr;          // gathered mask rows [Mr, Mr + n_b) ...
    mask.pos0[b] = M + 1;          // ... come from block rows M + 1 ..
    acc.row_off[b] = Mr;           // drafts of sequence b
    acc.pos0[b] = M;               // its targets (n_b + 1 of them) line up with its block rows
    M += gammas[b];
    Mr += gammas[b] - 1;
  }
  mask.row_off[B] = acc.row_off[B] = Mr;
  const int D = dims->D;
  size_t need = 0;
  if (flags & DFLASH_ARGMAX) {
    DF_REQUIRE(w != nullptr, DFLASH_ERR_INVALID_ARG, "weights is NULL");
    if ((st = check_ptr(w->lm_head, "lm_head")) != DFLASH_OK) return st;
    if ((st = check_ptr(h_final, "h_final")) != DFLASH_OK) return st;
    if (logits_dbg != nullptr && (st = check_ptr(logits_dbg, "logits_dbg")) != DFLASH_OK) return st;
    need = argmax_ws(dims, Mr, true).total;
  }
  if (flags & DFLASH_ACCEPT) {
    DF_REQUIRE(target != nullptr && tau != nullptr && next_anchor != nullptr, DFLASH_ERR_INVALID_ARG,
               "target, tau and next_anchor must be non-NULL for ACCEPT");
  }
  if ((st = check_ws(ws, ws_bytes, need)) != DFLASH_OK) return st;
  if ((st = check_device()) != DFLASH_OK) return st;

  hipStream_t s = as_stream(stream);
  if (flags & DFLASH_ARGMAX) {
    const ArgmaxWs lay = argmax_ws(dims, Mr, true);
    char* base = static_cast<char*>(ws);
    float* rows = reinterpret_cast<float*>(base + lay.rows);
    DF_HIP(launch_gather_rows(h_final, rows, D, mask, s));
    GemmArgs g{};
    for (int k = 0; k < kMaxSrc; ++k) g.a_src[k] = rows;
    g.a_cols = D;
    g.a_rg = INT_MAX;
    g.a_gs = 0;
    g.a_ld = D;
    if ((st = lm_head_argmax(dims, w, g, Mr, draft, logits_dbg, top2_gap, base, lay, ws, s)) != DFLASH_OK) return st;
  }
  if (flags & DFLASH_ACCEPT) DF_HIP(launch_accept_ragged(draft, target, acc, tau, next_anchor, s));
  return ok();
}

dflash_status dflash_target_verify(const dflash_dims* dims, const dflash_weights* w, const dflash_kv_cache* cache,
                                   const int32_t* block_tokens, int32_t gamma, const int32_t* tap_layers,
                                   void* const* taps, int32_t* target_tokens, float* top2_gap, void* ws,
                                   size_t ws_bytes, void* stream) {
  dflash_status st = check_dims(dims);
  if (st != DFLASH_OK) return st;
  DF_REQUIRE(w != nullptr, DFLASH_ERR_INVALID_ARG, "weights is NULL");
  if ((st = check_cache(cache)) != DFLASH_OK) return st;
  DF_REQUIRE(gamma >= 1 && gamma <= DFLASH_MAX_GAMMA, DFLASH_ERR_INVALID_ARG, "gamma=%d outside [1, %d]", gamma,
             DFLASH_MAX_GAMMA);
  DF_REQUIRE(block_tokens != nullptr && target_tokens != nullptr, DFLASH_ERR_INVALID_ARG,
             "block_tokens and target_tokens must be non-NULL");
  if ((st = check_ptr(w->lm_head, "lm_head")) != DFLASH_OK) return st;
  if ((st = check_ptr(w->embed, "embed")) != DFLASH_OK) return st;
  const int nt = dims->n_tgt_layers;
  DF_REQUIRE(tap_layers != nullptr && taps != nullptr, DFLASH_ERR_INVALID_ARG, "tap_layers and taps must be non-NULL");
  TargetPass tp;
  tp.n_taps = nt;
  for (int k = 0; k < nt; ++k) {
    DF_REQUIRE(tap_layers[k] >= 0 && tap_layers[k] < dims->L, DFLASH_ERR_INVALID_ARG,
               "tap_layers[%d]=%d outside [0, L=%d)", k, tap_layers[k], dims->L);
    DF_REQUIRE(k == 0 || tap_layers[k] > tap_layers[k - 1], DFLASH_ERR_INVALID_ARG,
               "tap_layers must increase (tap_layers[%d]=%d after %d)", k, tap_layers[k], tap_layers[k - 1]);
    if ((st = check_ptr(taps[k], "taps[k]")) != DFLASH_OK) return st;
    tp.layer[k] = tap_layers[k];
    tp.out[k] = taps[k];
  }
  QueryGroups qg;
  qg.n = cache->B;
  qg.apart = false;
  for (int b = 0; b < cache->B; ++b) {
    DF_REQUIRE(static_cast<int64_t>(cache->len[b]) + gamma <= cache->cap, DFLASH_ERR_CAPACITY,
               "sequence %d: len %d + gamma %d exceeds cap %d", b, cache->len[b], gamma, cache->cap);
    qg.gam[b] = qg.half[b] = gamma;
    qg.kvseq[b] = b;
    qg.nctx[b] = qg.nctx2[b] = qg.pos0[b] = cache->len[b];
  }
  const int B = cache->B, M = B * gamma;
  const VerifyWs lay = verify_ws(dims, B, gamma);
  if ((st = check_ws(ws, ws_bytes, lay.total)) != DFLASH_OK) return st;
  char* base = static_cast<char*>(ws);
  float* hf = reinterpret_cast<float*>(base + lay.hf);
  // the pass itself checks the remaining weights and the device
  if ((st = draft_forward_impl(dims, w, cache, block_tokens, nullptr, qg, hf, ws, lay.draft.total, stream, &tp)) !=
      DFLASH_OK)
    return st;
  hipStream_t s = as_stream(stream);
  GemmArgs g{};
  for (int k = 0; k < kMaxSrc; ++k) g.a_src[k] = hf;   // every block row, the anchor's included
  g.a_cols = dims->D;
  g.a_rg = INT_MAX;
  g.a_gs = 0;
  g.a_ld = dims->D;
  return lm_head_argmax(dims, w, g, M, target_tokens, nullptr, top2_gap, base + lay.head, lay.argmax,
                        base + lay.head, s);
}

dflash_status dflash_sample_drafts(const dflash_dims* dims, const dflash_weights* w, const float* h_final,
                                   int32_t B, int32_t gamma, float temperature, const float* uniforms,
                                   int32_t* draft, float* logits, float* lse, void* ws, size_t ws_bytes,
                                   void* stream) {
  dflash_status st = check_dims(dims);
  if (st != DFLASH_OK) return st;
  if ((st = check_gamma(gamma)) != DFLASH_OK) return st;
  if ((st = check_temperature(temperature)) != DFLASH_OK) return st;
  DF_REQUIRE(B >= 1 && B <= DFLASH_MAX_BATCH, DFLASH_ERR_INVALID_ARG, "B=%d outside [1, %d]", B, DFLASH_MAX_BATCH);
  DF_REQUIRE(w != nullptr, DFLASH_ERR_INVALID_ARG, "weights is NULL");
  if ((st = check_ptr(w->lm_head, "lm_head")) != DFLASH_OK) return st;
  if ((st = check_ptr(h_final, "h_final")) != DFLASH_OK) return st;
  if ((st = check_ptr(uniforms, "uniforms")) != DFLASH_OK) return st;
  if ((st = check_ptr(logits, "logits")) != DFLASH_OK) return st;
  DF_REQUIRE(draft != nullptr, DFLASH_ERR_INVALID_ARG, "draft is NULL");
  const SampleWs lay = sample_ws(dims, B, gamma);
  if ((st = check_ws(ws, ws_bytes, lay.total)) != DFLASH_OK) return st;
  if ((st = check_device()) != DFLASH_OK) return st;

  hipStream_t s = as_stream(stream);
  const int n = gamma - 1, Mr = B * n, D = dims->D, V = dims->V;
  const float inv_t = 1.0f / temperature;
  char* base = static_cast<char*>(ws);
  float4* stats = reinterpret_cast<float4*>(base + lay.stats);
  GemmArgs g{};
  for (int k = 0; k < kMaxSrc; ++k) g.a_src[k] = h_final + D;   // block row 1 of sequence 0
  g.a_cols = D;
  g.a_rg = n;
  g.a_gs = static_cast<int64_t>(gamma) * D;
  g.a_ld = D;
  g.w = w->lm_head;
  g.w_ld = D;
  g.w_rg = INT_MAX;
  g.w_gs = 0;
  g.w_off = 0;
  g.M = Mr;
  g.N = V;
  g.K = D;
  g.su = uniforms;
  g.inv_t = inv_t;
  RowStatArgs r{};
  r.rows1 = r.rows = Mr;
  r.N = V;
  r.chunk = sample_chunk(V, Mr);
  r.vec = V % 4 == 0;
  r.su = uniforms;
  r.inv_t = inv_t;
  r.stats = stats;
  r.S = 1;
  const int nchunk = (V + r.chunk - 1) / r.chunk;
  if (dims->dtype == DFLASH_BF16) {
    const GemmPlan rk = plan_gemm_rk(Mr, V, D, true);
    if (rk.rk) {
      // one pass over the LM head: logits stored, sampling statistics per workgroup
      const int ps = prof_begin(DFLASH_PROF_LM_HEAD, s);
      DF_HIP_PROF(launch_gemm_rk_sample(g, rk, stats, logits, s), ps);
      DF_HIP(launch_sample_final(stats, rk.grid, Mr, draft, lse, s));
      return ok();
    }
    const ActPlan ap = plan_act(Mr, V, D, true);
    g.part = reinterpret_cast<float*>(base + lay.part);
    const int ps = prof_begin(DFLASH_PROF_LM_HEAD, s);
    DF_HIP_PROF(launch_act_gemm(g, ap, base + lay.planes, s), ps);
    r.src = g.part;
    r.S = ap.p.S;
    r.split_stride = static_cast<int64_t>(Mr) * V;
    r.logits_out = logits;
  } else {
    g.part = logits;
    DF_HIP(launch_gemm_f32(g, s));
    r.src = logits;
  }
  const int ps = prof_begin(DFLASH_PROF_ROW_STATS, s);
  DF_HIP_PROF(launch_row_stats(r, s), ps);
  DF_HIP(launch_sample_final(stats, nchunk, Mr, draft, lse, s));
  return ok();
}

dflash_status dflash_sample_accept(const dflash_dims* dims, int32_t B, int32_t gamma, float temperature,
                                   const int32_t* draft, const float* draft_logits, const float* draft_lse,
                                   const float* target_logits, const float* accept_u, const float* resid_u,
                                   int32_t* tau, int32_t* next_anchor, void* ws, size_t ws_bytes, void* stream) {
  dflash_status st = check_dims(dims);
  if (st != DFLASH_OK) return st;
  if ((st = check_gamma(gamma)) != DFLASH_OK) return st;
  if ((st = check_temperature(temperature)) != DFLASH_OK) return st;
  DF_REQUIRE(B >= 1 && B <= DFLASH_MAX_BATCH, DFLASH_ERR_INVALID_ARG, "B=%d outside [1, %d]", B, DFLASH_MAX_BATCH);
  if ((st = check_ptr(draft_logits, "draft_logits")) != DFLASH_OK) return st;
  if ((st = check_ptr(target_logits, "target_logits")) != DFLASH_OK) return st;
  if ((st = check_ptr(resid_u, "resid_u")) != DFLASH_OK) return st;
  DF_REQUIRE(draft != nullptr && accept_u != nullptr && tau != nullptr && next_anchor != nullptr,
             DFLASH_ERR_INVALID_ARG, "draft, accept_u, tau and next_anchor must be non-NULL");
  const AcceptWs lay = sample_accept_ws(dims, B, gamma, draft_lse != nullptr);
  if ((st = check_ws(ws, ws_bytes, lay.total)) != DFLASH_OK) return st;
  if ((st = check_device()) != DFLASH_OK) return st;

  hipStream_t s = as_stream(stream);
  const int n = gamma - 1, V = dims->V;
  const float inv_t = 1.0f / temperature;
  char* base = static_cast<char*>(ws);
  RowStatArgs r{};
  r.src = target_logits;
  r.S = 1;
  r.rows1 = B * (n + 1);
  r.src2 = draft_logits;
  r.rows = lay.rows;
  r.N = V;
  r.chunk = lay.chunk;
  r.vec = V % 4 == 0;
  r.inv_t = inv_t;
  r.stats = reinterpret_cast<float4*>(base + lay.stats);
  int ps = prof_begin(DFLASH_PROF_ROW_STATS, s);
  DF_HIP_PROF(launch_row_stats(r, s), ps);
  SpecArgs a{};
  a.draft = draft;
  a.zq = draft_logits;
  a.zp = target_logits;
  a.lse_q = draft_lse;
  a.accept_u = accept_u;
  a.resid_u = resid_u;
  a.stats = r.stats;
  a.B = B;
  a.n = n;
  a.V = V;
  a.nchunk = lay.nchunk;
  a.ndraw = (V + kSpecDrawChunk - 1) / kSpecDrawChunk;
  a.rows = lay.rows;
  a.vec = r.vec;
  a.inv_t = inv_t;
  a.part = reinterpret_cast<float4*>(base + lay.part);
  a.m_out = reinterpret_cast<int32_t*>(base + lay.m);
  a.tau = tau;
  a.next_anchor = next_anchor;
  ps = prof_begin(DFLASH_PROF_VERIFY, s);
  DF_HIP_PROF(launch_spec_verify(a, s), ps);
  return ok();
}

}  // extern "C"
