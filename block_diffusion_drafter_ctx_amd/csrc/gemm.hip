// The GEMMs of the drafter path: C[m][n] = sum_k A[m][k] W[n][k], W bf16
// [N][K] row-major, A fp32 (split into bf16 hi + lo, two MFMA products, which
// keeps ~16 significant bits against the exact bf16 weights) or exact bf16.
// Which kernel runs depends on the activation rows M (plan_gemm):
//   * register-K (gemm_rk_kernel), M <= 16 per workgroup: a workgroup keeps
//     its 16 rows' K range in registers and streams whole 16-row weight tiles;
//     tall weights (LM head, gate/up) take the whole K per workgroup with the
//     top-2, sampling or SwiGLU epilogue, up to 32 rows in 16-row chunks on
//     XCD-adjacent workgroups; short weights (QKV, O, down, appends) split K
//     in 1024-wide ranges (1536 where that evens out the workgroups' share);
//   * streaming (gemm_stream_kernel), 17-32 rows and shapes the others do not
//     take: each wave streams a 16-row strip of W against an activation slice
//     staged in LDS, with split-K partials;
//   * tiled (gemm_tile_lds_kernel), from 33 rows: hi / lo plane tiles of
//     256 x 128 (128 x 128, 128 x 64, 256 x 64, 256 x 32 for fewer rows) or
//     128 x 256 bf16 tiles, fed by global-to-LDS loads, launched in
//     XCD-grouped tile order, with split-K partials or, for the LM head, a
//     per-tile top-2 epilogue;
//   * gemm_f32_kernel for fp32 weights (tiny configurations only).
// Split-K partials go to a [split][M][N] fp32 buffer that the consumer reduces
// in split order (deterministic, no float atomics).
#include "common.h"
#include "launch.h"

#include <stdlib.h>

#include <atomic>
#include <map>
#include <mutex>
#include <utility>

namespace dflash {
namespace {

constexpr int kStreamU = 8;          // weight k steps in flight per wave

template <typename T>
__device__ __forceinline__ const T* pick_src(const GemmArgs& g, int s) {
  // Select chain instead of a dynamic index into the kernel-argument array.
  const void* p = g.a_src[0];
#pragma unroll
  for (int i = 1; i < kMaxSrc; ++i) p = (s == i) ? g.a_src[i] : p;
  return static_cast<const T*>(p);
}

// Kernel arguments are read from memory by scalar loads.  Left alone, the
// compiler issues each batch where it is first needed, behind branches (and
// gridDim.x, an implicit argument, with them), and each dependent round is a
// memory latency before the first weight load goes out.  Naming every field a
// kernel uses in one empty asm statement before its first branch makes them
// arrive in one round.
__device__ __forceinline__ void fetch_args(const GemmArgs& g) {
  asm volatile("" ::"s"(g.a_src[0]), "s"(g.a_src[1]), "s"(g.a_src[2]), "s"(g.a_src[3]), "s"(g.a_src[4]),
               "s"(g.a_src[5]), "s"(g.a_src[6]), "s"(g.a_src[7]), "s"(g.a_cols), "s"(g.a_rg), "s"(g.a_ld),
               "s"(g.a_gs), "s"(g.w), "s"(g.w_ld), "s"(g.w_gs), "s"(g.w_off), "s"(g.w_rg), "s"(g.M), "s"(g.N),
               "s"(g.K), "s"(g.S), "s"(g.ntiles), "s"(g.part), "s"(g.stage_tiles), "s"(g.rchunks), "s"(gridDim.x));
}

// the tiled kernel's fields, in one statement too
__device__ __forceinline__ void fetch_args_tile(const GemmArgs& g) {
  asm volatile("" ::"s"(g.a_src[0]), "s"(g.a_src[1]), "s"(g.a_src[2]), "s"(g.a_src[3]), "s"(g.a_src[4]),
               "s"(g.a_src[5]), "s"(g.a_src[6]), "s"(g.a_src[7]), "s"(g.a_cols), "s"(g.a_rg), "s"(g.a_ld),
               "s"(g.a_gs), "s"(g.w), "s"(g.w_ld), "s"(g.w_gs), "s"(g.w_off), "s"(g.w_rg), "s"(g.M), "s"(g.N),
               "s"(g.K), "s"(g.S), "s"(g.ntiles), "s"(g.mtiles), "s"(g.chunks_per_split), "s"(g.xcd_tiles),
               "s"(g.part), "s"(g.a_lo));
}

// A source pointer chosen by a wave-uniform index.  A select among plain
// argument loads is turned back into one load at a computed offset (a
// dependent memory round trip); selecting among byte offsets from the first
// source keeps the values in registers and the pointer in the global space.
template <typename T>
__device__ __forceinline__ const T* pick_src_reg(const GemmArgs& g, int s) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(g.a_src[0]);
  uintptr_t off = 0;
#pragma unroll
  for (int k = 1; k < kMaxSrc; ++k) {
    const uintptr_t d = reinterpret_cast<uintptr_t>(g.a_src[k]) - b;
    off = s == k ? d : off;
  }
  return reinterpret_cast<const T*>(static_cast<const char*>(g.a_src[0]) + off);
}

__device__ __forceinline__ int64_t a_row_off(const GemmArgs& g, int r) {
  return static_cast<int64_t>(r / g.a_rg) * g.a_gs + static_cast<int64_t>(r % g.a_rg) * g.a_ld;
}

// Persistent workgroups of WAVES waves.  The work is a list of units
// (split, m-tile, n-tile) with unit u -> split u % S, then n-tile, then m-tile;
// workgroup i takes units i, i + P, i + 2P, ... (P = gridDim.x, a multiple of S,
// so a workgroup keeps one K range and stages its activation slice once).
// Wave w of a unit streams weight rows [tile*16*WAVES + 16w, +16) over the K
// range with U k-steps (U KB) of loads in flight, double buffered in registers;
// the stream continues across unit boundaries without a bubble.  After the
// activation slice is staged the loop has no barrier.
template <int MT, int AK, int WAVES, int KR>
__global__ __launch_bounds__(64 * WAVES) void gemm_stream_kernel(GemmArgs g) {
  constexpr int MTL = MT / 16;
  constexpr int HL = (AK == A_F32_SPLIT) ? 2 : 1;
  constexpr int NT = 64 * WAVES;
  constexpr int U = kStreamU;
  extern __shared__ uint4 lds[];              // [KR/32][MTL][HL][64]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = g.S, ntiles = g.ntiles;
  const int units = S * ntiles * g.mtiles;
  const int P = gridDim.x;
  const int cps = g.chunks_per_split;         // k steps per split
  int u = blockIdx.x;
  if (u >= units) return;

  // geometry of a unit for this lane
  auto nks_of = [&](int uu) { const int sp = uu % S; return min(g.K / 32 - sp * cps, cps); };
  auto wptr_of = [&](int uu) {
    const int sp = uu % S, rest = uu / S, tile = rest % ntiles;
    int n = tile * 16 * WAVES + wave * 16 + (lane & 15);
    n = min(n, g.N - 1);                       // rows past N are clamped; their results are dropped
    const int64_t wrow = static_cast<int64_t>(n / g.w_rg) * g.w_gs + g.w_off + n % g.w_rg;
    return static_cast<const uint16_t*>(g.w) + wrow * g.w_ld + sp * cps * 32 + 8 * (lane >> 4);
  };
  auto key_of = [&](int uu) { return (uu % S) + S * ((uu / S) / ntiles); };   // (split, m-tile)

  // stage the activation slice of unit uu: group q -> row q / kg8, k = k0 + 8 * (q % kg8)
  auto stage = [&](int uu) {
    const int sp = uu % S, mtile = (uu / S) / ntiles;
    const int m0 = mtile * MT, k0 = sp * cps * 32, kg8 = nks_of(uu) * 4;
    for (int q = tid; q < MT * kg8; q += NT) {
      const int m = q / kg8, kq = q - m * kg8;
      const int r = m0 + m;
      const int k = k0 + 8 * kq;
      const int slot = (((kq >> 2) * MTL + (m >> 4)) * HL) * 64 + (kq & 3) * 16 + (m & 15);
      const bool ok = r < g.M;
      const int s = k / g.a_cols, col = k - s * g.a_cols;
      if constexpr (AK == A_F32_SPLIT) {
        float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (ok) {
          const float* p = pick_src<float>(g, s) + a_row_off(g, r) + col;
          const float4 x0 = *reinterpret_cast<const float4*>(p), x1 = *reinterpret_cast<const float4*>(p + 4);
          x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w; x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
        }
        uint4 hi, lo;
        split8(x, hi, lo);
        lds[slot] = hi;
        lds[slot + 64] = lo;
      } else {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (ok) v = *reinterpret_cast<const uint4*>(pick_src<uint16_t>(g, s) + a_row_off(g, r) + col);
        lds[slot] = v;
      }
    }
  };

  uint4 wb0[U], wb1[U];
  auto load_w = [&](uint4 (&wb)[U], const uint16_t* wp, int nks, int grp) {
#pragma unroll
    for (int x = 0; x < U; ++x) {
      const int ks = grp * U + x;
      if (ks < nks) wb[x] = *reinterpret_cast<const uint4*>(wp + ks * 32);
    }
  };

  f32x4_t acc[MTL];
#pragma unroll
  for (int mt = 0; mt < MTL; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint4 (&wb)[U], int nks, int grp) {
#pragma unroll
    for (int x = 0; x < U; ++x) {
      const int ks = grp * U + x;
      if (ks < nks) {
#pragma unroll
        for (int mt = 0; mt < MTL; ++mt) {
          const uint4* bp = lds + ((ks * MTL + mt) * HL) * 64 + lane;
          acc[mt] = mfma16x16x32(wb[x], bp[0], acc[mt]);
          if constexpr (HL == 2) acc[mt] = mfma16x16x32(wb[x], bp[64], acc[mt]);
        }
      }
    }
  };

  auto flush = [&](int uu) {
    const int rest = uu / S, tile = rest % ntiles, mtile = rest / ntiles, sp = uu % S;
    const int nb = tile * 16 * WAVES + wave * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int mt = 0; mt < MTL; ++mt) {
      const int m = mtile * MT + mt * 16 + (lane & 15);
      if (m < g.M) {
        float* out = g.part + (static_cast<int64_t>(sp) * g.M + m) * g.N + nb;
        if (nb + 3 < g.N && (g.N & 3) == 0) {
          *reinterpret_cast<float4*>(out) = make_float4(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (nb + r < g.N) out[r] = acc[mt][r];
        }
      }
      acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };

  // ---- (unit, group) cursor: current cu/cg in buffer 0 or 1, next prefetched into the other
  int key = key_of(u);
  const uint16_t* wp = wptr_of(u);
  int nks = nks_of(u), ngrp = (nks + U - 1) / U, grp = 0;
  load_w(wb0, wp, nks, 0);                     // first weight group flies during staging
  stage(u);
  __syncthreads();

  // Advance to the next (unit, group); returns false when the list is done.  If
  // the next unit needs another activation slice the prefetch is skipped and
  // `restage` is set.
  auto next = [&](int& nu, int& ng, const uint16_t*& nwp, int& nnks, int& nngrp) {
    nu = u; ng = grp + 1; nwp = wp; nnks = nks; nngrp = ngrp;
    if (ng >= ngrp) {
      nu = u + P;
      ng = 0;
      if (nu < units) { nwp = wptr_of(nu); nnks = nks_of(nu); nngrp = (nnks + U - 1) / U; }
    }
    return nu < units;
  };

  for (;;) {
    // ---- step with wb0 current
    int nu, ng, nnks, nngrp;
    const uint16_t* nwp;
    bool more = next(nu, ng, nwp, nnks, nngrp);
    bool same = more && key_of(nu) == key;
    if (same) load_w(wb1, nwp, nnks, ng);
    compute(wb0, nks, grp);
    if (grp == ngrp - 1) flush(u);
    if (!more) break;
    if (!same) {
      __syncthreads();
      key = key_of(nu);
      load_w(wb1, nwp, nnks, ng);
      stage(nu);
      __syncthreads();
    }
    u = nu; grp = ng; wp = nwp; nks = nnks; ngrp = nngrp;
    // ---- step with wb1 current
    more = next(nu, ng, nwp, nnks, nngrp);
    same = more && key_of(nu) == key;
    if (same) load_w(wb0, nwp, nnks, ng);
    compute(wb1, nks, grp);
    if (grp == ngrp - 1) flush(u);
    if (!more) break;
    if (!same) {
      __syncthreads();
      key = key_of(nu);
      load_w(wb0, nwp, nnks, ng);
      stage(nu);
      __syncthreads();
    }
    u = nu; grp = ng; wp = nwp; nks = nnks; ngrp = nngrp;
  }
}

// ------------------------------------------------------------- register-K path
// One block of <= 16 activation rows (a 16-row chunk of a larger block, see
// rk_max_rows) against a tall weight (the LM head, the
// FFN gate/up projection; with eight waves, the short split-K form).  NW waves
// split the K range of a workgroup (wave w owns KS k-steps) and keep their
// activation fragments (hi + lo) in registers for the whole kernel, so a
// workgroup needs no split-K partner and no LDS slice: every output tile of
// 16 weight rows is one contiguous 16 x K block of W, streamed by all NW waves
// at once through a ring of KS loads per wave (the next tile's loads are
// issued as the current tile's MFMAs retire).  The NW per-wave partial tiles
// are summed through LDS
// in wave order (deterministic).  Epilogues: the [split][M][N] store; the LM
// head's running top-2 per row (plus the logits when asked for), merged per
// workgroup into top2[block][m] = (best value, its index, runner-up); the LM
// head's temperature-sampling statistics (logits stored, then per row the best
// Gumbel-perturbed key x + G(u) with x = logit / T, and the log-sum-exp state of
// x), merged per workgroup into stats[block][m]; or the
// FFN's SwiGLU, where a tile holds 8 gate rows and the 8 matching up rows of
// the stacked [gate; up] weight, so s = silu(gate) * up leaves the kernel
// directly (N = F outputs, 8 per tile).
constexpr int kRkWaves = 16;
constexpr int kRkShortWaves = 8;   // the short split-K form (see plan_gemm_rk_short)
constexpr int kLdsBytes = 160 * 1024;   // LDS per workgroup on gfx950
constexpr int kRkMinN = 16384;   // weight rows below which the split-K streaming kernel wins

enum RkEpilogue { RK_PART = 0, RK_TOP2 = 1, RK_SWIGLU = 2, RK_SAMPLE = 3 };

// Source of k index k (uniform): sources are a_cols wide, at most kMaxSrc of
// them; compares instead of a division.
__device__ __forceinline__ int src_of(int k, int a_cols) {
  int s = 0;
#pragma unroll
  for (int j = 1; j < kMaxSrc; ++j) s += k >= j * a_cols ? 1 : 0;
  return s;
}

template <int KS, int EP, int T, int AK = A_F32_SPLIT, int NW = kRkWaves>
__global__ __launch_bounds__(64 * NW) void gemm_rk_kernel(GemmArgs g, float* top2, float* logits) {
  fetch_args(g);
  constexpr bool TOP2 = EP == RK_TOP2;
  constexpr bool SAMPLE = EP == RK_SAMPLE;
  constexpr int TN = EP == RK_SWIGLU ? 8 : 16;   // outputs per tile
  static_assert(EP == RK_PART || T == 1, "fused epilogues stream one tile at a time");
  __shared__ float red[2][NW][T][256];
  __shared__ float tv1[4][16], tv2[4][16];
  __shared__ int ti1[4][16];
  __shared__ float4 sst[4][16];
  // Epilogues that write per tile (split-K partials, SwiGLU, sampled logits):
  // when the launch provides dynamic LDS for it, every output tile of this
  // workgroup stays in LDS ([slot][row][column], slot = (unit - u0) / P) and is
  // written out once, after the weight stream.  Small writes interleaved with
  // the read stream cost far more HBM time than their bytes.
  extern __shared__ __attribute__((aligned(16))) float lt_all[];
  constexpr int kOutCols = EP == RK_SWIGLU ? 8 : 16;   // output columns per tile
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = g.S;
  const int units = S * g.ntiles;
  // More than 16 activation rows: chunk c (rows 16c..16c+15) of unit group w
  // runs on its own workgroup, (w / 8) * 8C + 8c + w % 8 in launch order.
  // Workgroups 8 apart land on the same XCD and are dispatched together, so the
  // C chunks of a unit group stream the same weight tiles through one L2 at
  // about the same time.  The launcher makes P a multiple of 8 when C > 1.
  const int C = g.rchunks > 1 ? g.rchunks : 1;
  const int L = blockIdx.x;
  const int chunk = C > 1 ? (L >> 3) % C : 0;
  const int u0 = C > 1 ? (L / (8 * C)) * 8 + (L & 7) : L;   // unit group
  const int m0 = 16 * chunk;                  // first activation row of the chunk
  const int P = gridDim.x / C;
  if (u0 >= units) return;                    // uniform per workgroup
  const int sp = u0 % S;                      // P % S == 0: the split never changes
  const int kwave = sp * (32 * KS * NW) + wave * (32 * KS);
  const int kl = kwave + 8 * (lane >> 4);
  auto wrow = [&](int uu) {
    uu = uu < units ? uu : u0;                // past the last unit: re-read a valid one (result dropped)
    int n;
    if constexpr (EP == RK_SWIGLU) {
      // lanes 0-7: gate rows 8t.., lanes 8-15: up rows F + 8t.. (rows past F clamped, results dropped)
      n = min((uu / S) * 8 + (lane & 7), g.N - 1) + ((lane & 8) ? g.N : 0);
    } else {
      n = min((uu / S) * 16 + (lane & 15), g.N - 1);   // rows past N are clamped; their results are dropped
    }
    const int64_t r = static_cast<int64_t>(n / g.w_rg) * g.w_gs + g.w_off + n % g.w_rg;
    return static_cast<const uint16_t*>(g.w) + r * g.w_ld + kl;
  };
  // group q holds units u0 + P (T q + t), t < T; its weights stream through wb
  uint4 wb[T][KS];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const uint16_t* wp = wrow(u0 + P * t);
#pragma unroll
    for (int x = 0; x < KS; ++x) wb[t][x] = *reinterpret_cast<const uint4*>(wp + x * 32);
  }
  __builtin_amdgcn_sched_barrier(0);          // the first tiles' weights go out before the activation loads

  constexpr bool SPLIT = AK == A_F32_SPLIT;    // fp32 activations as bf16 hi + lo; else exact bf16
  uint4 bh[KS], bl[SPLIT ? KS : 1];
  const int a_m = m0 + (lane & 15) < g.M ? m0 + (lane & 15) : 0;
  // no division unless the activation rows are grouped
  const int64_t a_off = g.a_rg >= g.M ? static_cast<int64_t>(a_m) * g.a_ld : a_row_off(g, a_m);
  if constexpr (!SPLIT) {
    const int s = src_of(kwave, g.a_cols);
    const int m = m0 + (lane & 15);
    const bool ok = m < g.M;
    const uint16_t* p = pick_src_reg<uint16_t>(g, s) + a_off + (kl - s * g.a_cols);
#pragma unroll
    for (int x = 0; x < KS; ++x) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + x * 32);
      bh[x] = ok ? v : make_uint4(0, 0, 0, 0);
    }
  } else {
    // the host guarantees a_cols % (32 * KS) == 0: a wave's k range lies in one source
    const int s = src_of(kwave, g.a_cols);
    const int m = m0 + (lane & 15);
    const bool ok = m < g.M;
    const float* p = pick_src_reg<float>(g, s) + a_off + (kl - s * g.a_cols);
    float4 av[2 * KS];
#pragma unroll
    for (int x = 0; x < KS; ++x) {
      av[2 * x] = *reinterpret_cast<const float4*>(p + x * 32);
      av[2 * x + 1] = *reinterpret_cast<const float4*>(p + x * 32 + 4);
    }
    const float keep = ok ? 1.f : 0.f;
#pragma unroll
    for (int x = 0; x < KS; ++x) {
      float v[8] = {av[2 * x].x * keep,     av[2 * x].y * keep,     av[2 * x].z * keep,     av[2 * x].w * keep,
                    av[2 * x + 1].x * keep, av[2 * x + 1].y * keep, av[2 * x + 1].z * keep, av[2 * x + 1].w * keep};
      split8(v, bh[x], bl[x]);
    }
  }

  // reduction thread tid < 256 owns output (n = TN * tile + 4 * (ln / 16) + r, m = m0 + ln % 16), ln = tid / 4
  const int ln = tid >> 2;
  const int mo = ln & 15, no = 4 * (ln >> 4) + (tid & 3);
  const int mg = m0 + mo;                     // its activation row
  Top2 best{-INFINITY, 0x7fffffff, -INFINITY};
  SampleStat ss = sstat_empty();
  const bool staged = EP != RK_TOP2 && g.stage_tiles > 0;
  int buf = 0;
  for (int q = 0;; ++q) {
    const int ub = u0 + P * T * q;
    const bool more = ub + P * T < units;     // uniform per workgroup
    float su = 0.5f;                          // this thread's sampling uniform, fetched before the MFMAs
    if constexpr (SAMPLE) {
      const int n = (ub / S) * TN + no;
      if (tid < 256 && mg < g.M && n < g.N) su = g.su[static_cast<int64_t>(mg) * g.N + n];
    }
    f32x4_t acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (more) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint16_t* np = wrow(ub + P * T + P * t);
#pragma unroll
        for (int x = 0; x < KS; ++x) {
          acc[t] = mfma16x16x32(wb[t][x], bh[x], acc[t]);
          if constexpr (SPLIT) acc[t] = mfma16x16x32(wb[t][x], bl[x], acc[t]);
          wb[t][x] = *reinterpret_cast<const uint4*>(np + x * 32);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int x = 0; x < KS; ++x) {
          acc[t] = mfma16x16x32(wb[t][x], bh[x], acc[t]);
          if constexpr (SPLIT) acc[t] = mfma16x16x32(wb[t][x], bl[x], acc[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < T; ++t)
      *reinterpret_cast<float4*>(&red[buf][wave][t][lane * 4]) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    __syncthreads();
    if constexpr (EP == RK_SWIGLU) {
      // thread tid < 128 holds gate output j of row m at red index tid and the
      // matching up output at tid + 128 (weight row j + 8 of the tile)
      if (tid < 128) {
        float vg = 0.f, vu = 0.f;
#pragma unroll 4
        for (int w = 0; w < NW; ++w) {
          vg += red[buf][w][0][tid];
          vu += red[buf][w][0][tid + 128];
        }
        const int f = (ub / S) * TN + no;      // no < 8 for tid < 128
        if (mg < g.M && f < g.N) {
          const float sv = vg / (1.0f + expf(-vg)) * vu;
          if (staged) lt_all[q * 128 + mo * 8 + no] = sv;
          else g.part[static_cast<int64_t>(mg) * g.N + f] = sv;
        }
      }
    } else if (tid < 256) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int uu = ub + P * t;
        if (uu < units) {
          float v = 0.f;
#pragma unroll 4
          for (int w = 0; w < NW; ++w) v += red[buf][w][t][tid];
          const int n = (uu / S) * TN + no;
          if (mg < g.M && n < g.N) {
            if constexpr (TOP2) {
              if (logits != nullptr) logits[static_cast<int64_t>(mg) * g.N + n] = v;
              best = top2_push(best, v, n);
            } else if constexpr (SAMPLE) {
              if (staged) lt_all[q * 256 + mo * 16 + no] = v;
              else logits[static_cast<int64_t>(mg) * g.N + n] = v;
              const float x = v * g.inv_t;
              sstat_push_lse(ss, x);
              sstat_push_key(ss, x + gumbel_noise(su), n);
            } else if (staged) {
              lt_all[(q * T + t) * 256 + mo * 16 + no] = v;
            } else {
              g.part[(static_cast<int64_t>(sp) * g.M + mg) * g.N + n] = v;
            }
          }
        }
      }
    }
    buf ^= 1;
    if (!more) break;
  }

  if constexpr (TOP2) {
    // merge the 16 owners of each row: lanes 4m..4m+3 of waves 0..3
    if (tid < 256) {
      best = top2_merge(best, top2_shfl_xor(best, 1));
      best = top2_merge(best, top2_shfl_xor(best, 2));
      if ((lane & 3) == 0) {
        tv1[wave][lane >> 2] = best.v1;
        ti1[wave][lane >> 2] = best.i1;
        tv2[wave][lane >> 2] = best.v2;
      }
    }
    __syncthreads();
    if (tid < 16 && m0 + tid < g.M) {
      Top2 t{tv1[0][tid], ti1[0][tid], tv2[0][tid]};
#pragma unroll
      for (int w = 1; w < 4; ++w) t = top2_merge(t, Top2{tv1[w][tid], ti1[w][tid], tv2[w][tid]});
      float* o = top2 + (static_cast<int64_t>(u0) * g.M + m0 + tid) * 3;
      o[0] = t.v1;
      o[1] = __int_as_float(t.i1);
      o[2] = t.v2;
    }
  }
  if constexpr (SAMPLE) {
    // same owner layout as the top-2 merge
    if (tid < 256) {
      ss = sstat_merge(ss, sstat_shfl_xor(ss, 1));
      ss = sstat_merge(ss, sstat_shfl_xor(ss, 2));
      if ((lane & 3) == 0) sst[wave][lane >> 2] = sstat_pack(ss);
    }
    __syncthreads();
    if (tid < 16 && m0 + tid < g.M) {
      SampleStat t = sstat_unpack(sst[0][tid]);
#pragma unroll
      for (int w = 1; w < 4; ++w) t = sstat_merge(t, sstat_unpack(sst[w][tid]));
      reinterpret_cast<float4*>(top2)[static_cast<int64_t>(u0) * g.M + m0 + tid] = sstat_pack(t);
    }
  }
  if (staged) {
    if constexpr (!SAMPLE) __syncthreads();   // the last tile's epilogue is done
    // piece i: slot i / PPT, row (i % PPT) / (PPT / 16), four columns from 4 (i % (PPT / 16))
    constexpr int PPT = kOutCols * 16 / 4;     // float4 pieces per tile
    constexpr int PPR = kOutCols / 4;          // float4 pieces per row
    const int nslots = (units - u0 + P - 1) / P;
    float* out = SAMPLE ? logits : g.part + static_cast<int64_t>(sp) * g.M * g.N;
    for (int i = tid; i < nslots * PPT; i += 64 * NW) {
      const int slot = i / PPT, r = (i % PPT) / PPR, c4 = 4 * (i % PPR);
      const int n0 = ((u0 + P * slot) / S) * kOutCols;
      if (m0 + r < g.M) {
        float* dst = out + static_cast<int64_t>(m0 + r) * g.N + n0 + c4;
        const float* src = &lt_all[slot * (16 * kOutCols) + r * kOutCols + c4];
        if ((g.N & 3) == 0 && n0 + c4 + 3 < g.N) {
          *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(src);
        } else {
          for (int e = 0; e < 4; ++e)
            if (n0 + c4 + e < g.N) dst[e] = src[e];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ tiled path
// Many activation rows (context ingest, big batches): a classic LDS-tiled MFMA
// GEMM.  Workgroup tile 128 weight rows x 128 activation rows x 64 k; 4 waves
// in a 2 x 2 layout, each computing 64 x 64 with 16 MFMA accumulators.  Both
// operand tiles are staged in LDS in MFMA fragment order (conflict-free 16 B
// reads), double-buffered, with the next tile's global loads in flight while
// the current one is multiplied.  grid = (N / 128, M / 128, splits).
constexpr int kTileN = 128, kTileM = 128, kTileK = 64;
// LDS-direct kernel shapes (weight rows x activation rows): eight waves, two
// per SIMD, so one issues MFMAs while the other's load instructions are being
// accepted.  The first bf16 shape was 256 x 256 in waves of 64 x 128 with two
// 64 KB stages (kTileBf16, still selectable for measurement); hi/lo planes take
// 256 x 128 tiles in eight waves of 64 x 64 (a 256-row A tile's two planes
// would not leave room for two LDS stages)
struct TileShape { int tn, tm, wn, wm, ns; };
constexpr TileShape kTileBf16{256, 256, 64, 128, 2}, kTileHiLo{256, 128, 64, 64, 2};
// hi / lo planes of at most 64 activation rows: a 64-row tile (eight waves of
// 64 x 32) does half the MFMA work of the 128-row one, and its 48 KB stage (40
// KB at 32 rows) leaves room for three stages: two tiles in flight cover the
// HBM latency of the weight tiles, which one tile in flight does not (the
// 8-layer drafter at 4 x 16 block rows: 2126 -> 1976 us; bf16 A on 256 x 128
// tiles with three stages loses to 256 x 256 with two: ingest 585 -> 674 us)
constexpr TileShape kTileHiLo64{256, 64, 64, 32, 3}, kTileHiLo32{256, 32, 64, 16, 3};
// hi / lo planes of 65-256 activation rows against a drafter-sized weight: 128
// weight rows x 128 activation rows (eight waves of 64 x 32, three 48 KB
// stages).  Twice the n-tiles of the 256-row tile, so fewer K splits fill the
// CUs and fewer fp32 partials go through HBM: 16-sequence ragged pass 2222 ->
// 2123 us, the 16-sequence loop 2361 -> 2264 us, the 8-layer drafter at 4 x 32
// block rows 2326 -> 2286 us; with 512 or 1024 rows (anchored blocks) the
// 256-row tile stays ahead (4745 against 4870 us)
constexpr TileShape kTileHiLoN128{128, 128, 64, 32, 3};
// bf16 A (the context ingest) on 128 x 256 tiles (eight waves of 64 x 64,
// three 48 KB stages) rather than 256 x 256 with two: the inject GEMM (2048 x
// 10240 x 4096) 183 -> 173 us, the fuse unchanged (its 256 tiles then need no
// K split)
constexpr TileShape kTileBf16N128{128, 256, 64, 64, 3};
// ... and for 33-64 rows 128 x 64 tiles (eight waves of 32 x 32, three 32 KB
// stages; four measured slightly slower): the 8-layer drafter at 4 x 16 block
// rows 1766 -> 1715 us a loop iteration
constexpr TileShape kTileHiLoN128M64{128, 64, 32, 32, 3};

template <int AK>
__global__ __launch_bounds__(256) void gemm_tile_kernel(GemmArgs g) {
  constexpr int HL = (AK == A_F32_SPLIT) ? 2 : 1;
  constexpr int WFR = (kTileN / 16) * (kTileK / 32);        // W fragments per tile (16)
  constexpr int AFR = (kTileM / 16) * (kTileK / 32) * HL;   // A fragments per tile
  constexpr int BUF = (WFR + AFR) * 64;                     // uint4 per buffer
  extern __shared__ uint4 lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int n0 = blockIdx.x * kTileN, m0 = blockIdx.y * kTileM;
  const int split = blockIdx.z;
  const int ktiles = g.K / kTileK;
  const int kt_begin = split * g.chunks_per_split;
  const int kt_end = min(ktiles, kt_begin + g.chunks_per_split);

  // Per-thread global chunks: c = tid + 256*i -> row c / 8 (= tid/8 + 32 i), k8
  // group q = tid % 8 (the same for all four chunks of a thread).
  const int q = tid & 7, r0 = tid >> 3;
  const uint16_t* wbase[4];
  int64_t abase[4];
  uint32_t akeep = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + 32 * i;
    const int n = min(n0 + r, g.N - 1);
    wbase[i] = static_cast<const uint16_t*>(g.w) +
               (static_cast<int64_t>(n / g.w_rg) * g.w_gs + g.w_off + n % g.w_rg) * g.w_ld + 8 * q;
    const int m = m0 + r;
    if (m < g.M) akeep |= 1u << i;
    abase[i] = a_row_off(g, min(m, g.M - 1)) + 8 * q;   // rows past M load row M-1 and are zeroed
  }
  const int slot0 = (q >> 2) * 64 + (q & 3) * 16 + (r0 & 15);   // + (row/16)*2*64 (+ hl)

  uint4 wreg0, wreg1, wreg2, wreg3;
  uint4 areg_b[AK == A_BF16 ? 4 : 1];
  float areg_f[AK == A_F32_SPLIT ? 32 : 1];
  auto gload = [&](int kt) __attribute__((always_inline)) {
    const int kb = kt * kTileK;
    const int s = kb / g.a_cols, col = kb - s * g.a_cols;     // a 64-wide k tile never straddles sources
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 wv = *reinterpret_cast<const uint4*>(wbase[i] + kb);
      if (i == 0) wreg0 = wv; else if (i == 1) wreg1 = wv; else if (i == 2) wreg2 = wv; else wreg3 = wv;
      const bool ok = (akeep >> i) & 1u;
      if constexpr (AK == A_BF16) {
        const uint4 v = *reinterpret_cast<const uint4*>(pick_src<uint16_t>(g, s) + abase[i] + col);
        const uint32_t keep = ok ? 0xffffffffu : 0u;
        areg_b[i] = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
      } else {
        const float* p = pick_src<float>(g, s) + abase[i] + col;
        const float4 v0 = *reinterpret_cast<const float4*>(p), v1 = *reinterpret_cast<const float4*>(p + 4);
        const float keep = ok ? 1.0f : 0.0f;
        areg_f[8 * i + 0] = v0.x * keep; areg_f[8 * i + 1] = v0.y * keep;
        areg_f[8 * i + 2] = v0.z * keep; areg_f[8 * i + 3] = v0.w * keep;
        areg_f[8 * i + 4] = v1.x * keep; areg_f[8 * i + 5] = v1.y * keep;
        areg_f[8 * i + 6] = v1.z * keep; areg_f[8 * i + 7] = v1.w * keep;
      }
    }
  };
  auto lstore = [&](uint4* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int frag_row = ((r0 + 32 * i) >> 4) * 2;          // (row / 16) * (k steps per tile)
      buf[frag_row * 64 + slot0] = i == 0 ? wreg0 : (i == 1 ? wreg1 : (i == 2 ? wreg2 : wreg3));
      if constexpr (AK == A_BF16) {
        buf[WFR * 64 + frag_row * 64 + slot0] = areg_b[i];
      } else {
        uint4 hi, lo;
        split8(&areg_f[8 * i], hi, lo);
        const int sl = WFR * 64 + (frag_row * HL) * 64 + ((q >> 2) * HL) * 64 + (q & 3) * 16 + (r0 & 15);
        buf[sl] = hi;
        buf[sl + 64] = lo;
      }
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint4* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 wf[4], af[4], al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) wf[i] = buf[((wn * 4 + i) * 2 + ks) * 64 + lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        af[j] = buf[WFR * 64 + (((wm * 4 + j) * 2 + ks) * HL) * 64 + lane];
        if constexpr (HL == 2) al[j] = buf[WFR * 64 + (((wm * 4 + j) * 2 + ks) * HL + 1) * 64 + lane];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = mfma16x16x32(wf[i], af[j], acc[i][j]);
          if constexpr (HL == 2) acc[i][j] = mfma16x16x32(wf[i], al[j], acc[i][j]);
        }
    }
  };

  if (kt_begin < kt_end) {
    gload(kt_begin);
    lstore(lds);
    __syncthreads();
    int cur = 0;
    for (int kt = kt_begin; kt < kt_end; ++kt) {
      const bool more = kt + 1 < kt_end;
      if (more) gload(kt + 1);
      compute(lds + cur * BUF);
      if (more) lstore(lds + (cur ^ 1) * BUF);
      __syncthreads();
      cur ^= 1;
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + wn * 64 + i * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm * 64 + j * 16 + (lane & 15);
      if (m >= g.M) continue;
      float* out = g.part + (static_cast<int64_t>(split) * g.M + m) * g.N + n;
      if (n + 3 < g.N && (g.N & 3) == 0) {
        *reinterpret_cast<float4*>(out) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < g.N) out[r] = acc[i][j][r];
      }
    }
  }
}

// ------------------------------------------------------- tiled path, LDS-direct
// TN weight rows x TM activation rows x 64 k per tile, in waves of WN x WM
// outputs, fed by gfx950's global-to-LDS loads (a wave-wide 16-byte load lands lane l at
// LDS base + 16 l, no register staging).  Each load instruction brings whole
// 128-byte lines: 8 rows x 64 k (lane l: row l / 8, 16-byte chunk l % 8) --
// from L2 that runs 2.5x faster than MFMA-fragment order (16 rows x 64 bytes
// per instruction).  In LDS a tile is row-major, 128 bytes per row, with chunk
// c of row r stored at slot c ^ (r % 8): the 16-byte fragment reads of 8
// consecutive rows then hit 8 different bank groups.  NSTAGE k-tiles are in
// LDS at once; fragments are read one k-step ahead so that the LDS reads of the
// next k-step are in flight while this one's MFMAs issue; stage t % NSTAGE is
// refilled with tile t + NSTAGE right after the barrier that follows every
// wave's last read of tile t.  Past the end of the K range the loads repeat the
// last tile, so every wait has a fixed count.  A is exact bf16 (HL = 1) or the
// hi and lo planes of an fp32 matrix (HL = 2, two MFMAs per product).
// TOP2 (the LM head with a single K split): instead of partial sums the
// workgroup writes, for every activation row, the top-2 of its TN weight rows
// to top2[(n-tile * M + m) * 3] (value, index bits, runner-up; lower index on
// ties), plus the logits to g.part when that is set.
template <int HL, int NSTAGE, int TN, int TM, int WN, int WM, bool TOP2 = false, bool EARLY = false>
__global__ __launch_bounds__((TN / WN) * (TM / WM) * 64) void gemm_tile_lds_kernel(GemmArgs g, float* top2) {
  fetch_args_tile(g);
  constexpr int NW = (TN / WN) * (TM / WM);                 // waves of WN x WM outputs each
  constexpr int FN = WN / 16, FM = WM / 16;                 // 16-row fragments per wave: W, A
  constexpr int WROWS = TN, AROWS = TM * HL;                // LDS rows per stage (A: planes stacked)
  constexpr int NLD = (WROWS + AROWS) / 8;                  // 8-row load instructions per stage
  constexpr int BUF = (WROWS + AROWS) * 8;                  // uint4 per stage
  constexpr int LPW = NLD / NW;                             // loads per wave per stage
  static_assert(NLD % NW == 0 && kTileK == 64, "loads split evenly over the waves");
  extern __shared__ uint4 lds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave % (TN / WN), wm = wave / (TN / WN);
  int nt = blockIdx.x, mt = blockIdx.y, split = blockIdx.z;
  if (g.xcd_tiles) {
    // 1-D launch over T = S * ntiles * mtiles tiles, padded to a multiple of 8.
    // Workgroups go to the XCDs in turn (launch slot L on XCD L % 8), so XCD
    // x takes tile indices [x P, (x + 1) P) in launch order, the tile index
    // running m-tile fastest, then n-tile, then split: the m-tiles that read
    // one weight tile run together on one XCD and share its L2.
    const int T = g.S * g.ntiles * g.mtiles;
    const int P = (T + 7) / 8;
    const int w = (blockIdx.x & 7) * P + (blockIdx.x >> 3);
    if (w >= T) return;                                     // padding; uniform per workgroup
    mt = w % g.mtiles;
    nt = (w / g.mtiles) % g.ntiles;
    split = w / (g.mtiles * g.ntiles);
  }
  const int n0 = nt * TN, m0 = mt * TM;
  const int ktiles = g.K / kTileK;
  const int kt_begin = split * g.chunks_per_split;
  const int kt_end = min(ktiles, kt_begin + g.chunks_per_split);
  if (kt_begin >= kt_end) return;                           // uniform per workgroup
  const int nk = kt_end - kt_begin;

  // load q = wave + NW i of a stage covers LDS rows 8q .. 8q + 7 (W rows first,
  // then A: hi plane rows, lo plane rows); lane l fetches chunk
  // (l % 8) ^ (l / 8) of row 8q + l / 8, the chunk its LDS slot l % 8 holds.
  // voff[i] is that lane's byte offset from the load's scalar base (the W
  // tile's k column, or the A plane's column); the launcher keeps it below 2^31.
  const int kchunk = 8 * ((lane & 7) ^ (lane >> 3));
  uint32_t voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = 8 * (wave + NW * i) + (lane >> 3);
    int64_t e;
    if (row < WROWS) {
      const int n = min(n0 + row, g.N - 1);                 // rows past N: results dropped
      e = (static_cast<int64_t>(n / g.w_rg) * g.w_gs + g.w_off + n % g.w_rg) * g.w_ld + kchunk;
    } else {
      const int m = min(m0 + (row - WROWS) % TM, g.M - 1);       // rows past M: results dropped
      e = a_row_off(g, m) + kchunk;
    }
    voff[i] = static_cast<uint32_t>(e * 2);
  }
  const uint16_t* wbase = static_cast<const uint16_t*>(g.w);
  const unsigned lds0 = lds_addr(lds);
  // The tile whose loads go out next: tiles are issued in order, and past the
  // end of the K range the last one repeats.  Its W, A-hi and A-lo column
  // pointers advance by additions (a 64-wide k tile never straddles A sources,
  // a_cols % 64 == 0), so the loop does no division and the load bases stay
  // in scalar registers.  HL == 2: one source, its hi and lo planes.
  int c_t = 0;
  const uint16_t *c_wp, *c_ap, *c_lp;
  int c_s, c_col;
  auto uni = [](const uint16_t* p) __attribute__((always_inline)) {   // pin a wave-uniform pointer to SGPRs
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    // readfirstlane returns int: each half goes through uint32_t so that the
    // low word is not sign-extended into the high one
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
    return reinterpret_cast<const uint16_t*>((static_cast<uint64_t>(hi) << 32) | lo);
  };
  {
    const int kb = kt_begin * kTileK;
    c_s = kb / g.a_cols;
    c_col = kb - c_s * g.a_cols;
    c_wp = uni(wbase + kb);
    c_ap = uni(pick_src_reg<uint16_t>(g, c_s) + c_col);
    c_lp = HL == 2 ? uni(static_cast<const uint16_t*>(g.a_lo) + c_col) : c_ap;
  }
  auto advance = [&]() __attribute__((always_inline)) {
    if (c_t < nk - 1) {
      c_wp += kTileK;
      c_ap += kTileK;
      if constexpr (HL == 2) c_lp += kTileK;
      c_col += kTileK;
      if (c_col == g.a_cols) {                               // the next A source starts
        c_col = 0;
        ++c_s;
        c_ap = uni(pick_src_reg<uint16_t>(g, c_s));
      }
    }
    ++c_t;
  };
  // which operand load i of a wave feeds: W rows, then the A hi plane, then
  // the lo plane; known at compile time when the rows split evenly over the
  // waves' loads, otherwise a wave-uniform test
  auto base_of = [&](int i) __attribute__((always_inline)) -> const uint16_t* {
    constexpr int R8 = 8 * NW;                               // LDS rows one load index covers
    if constexpr (WROWS % R8 == 0 && (WROWS + TM) % R8 == 0) {
      if (i < WROWS / R8) return c_wp;
      if (HL == 2 && i >= (WROWS + TM) / R8) return c_lp;
      return c_ap;
    } else {
      const int row0 = 8 * (wave + NW * i);
      if (row0 < WROWS) return c_wp;
      return HL == 2 && row0 - WROWS >= TM ? c_lp : c_ap;
    }
  };
  auto issue_one = [&](int i, int stage) __attribute__((always_inline)) {
    const int q = wave + NW * i;                             // uniform per wave
    load_to_lds_sbase(voff[i], uni(base_of(i)),
                      __builtin_amdgcn_readfirstlane(lds0 + static_cast<unsigned>((stage * BUF + q * 64) * 16)));
  };
  auto issue = [&](int stage) __attribute__((always_inline)) {   // the cursor's tile into stage; then advance
#pragma unroll
    for (int i = 0; i < LPW; ++i) issue_one(i, stage);
    advance();
  };

  f32x4_t acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // fragment (row group of 16, k-step ks): lane l reads row (l % 16) of the
  // group, chunk 4 ks + l / 16, at slot chunk ^ (row % 8)
  const int xs = (lane >> 4) ^ (lane & 7);
  const int wrow = (wn * WN + (lane & 15)) * 8, arow = (WROWS + wm * WM + (lane & 15)) * 8;
  struct Frags { uint4 w[FN], a[FM * HL]; };
  auto rd = [&](Frags& f, const uint4* buf, int ks) __attribute__((always_inline)) {
    const int slot = xs ^ (ks << 2);
#pragma unroll
    for (int i = 0; i < FN; ++i) f.w[i] = buf[wrow + i * 128 + slot];
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int h = 0; h < HL; ++h) f.a[j * HL + h] = buf[arow + (h * TM + j * 16) * 8 + slot];
  };
  auto mm = [&](const Frags& f) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int h = 0; h < HL; ++h) acc[i][j] = mfma16x16x32(f.w[i], f.a[j * HL + h], acc[i][j]);
  };
  // the same MFMAs with the next tile's loads spread among them, so that the
  // wave keeps the MFMA pipe fed while the load instructions are accepted
  constexpr int NMF = FN * FM * HL, EVERY = (NMF + LPW - 1) / LPW;
  auto mm_issue = [&](const Frags& f, int stage) __attribute__((always_inline)) {
    int q = 0;
#pragma unroll
    for (int x = 0; x < NMF; ++x) {
      const int i = x / (FM * HL), j = (x / HL) % FM, h = x % HL;
      acc[i][j] = mfma16x16x32(f.w[i], f.a[j * HL + h], acc[i][j]);
      if (x % EVERY == EVERY - 1 && q < LPW) {
        __builtin_amdgcn_sched_barrier(0);
        issue_one(q++, stage);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int r = 0; r < LPW; ++r)
      if (r >= q) issue_one(r, stage);
    advance();
  };

#pragma unroll
  for (int st = 0; st < NSTAGE; ++st) issue(st);
  wait_vmcnt<(NSTAGE - 1) * LPW>();                          // tile 0 landed
  bare_barrier();
  Frags fa, fb;
  rd(fa, lds, 0);
  // stage of tile t (sc) and of tile t + 1 (sn); tile t + NSTAGE goes to sc
  int sc = 0, sn = 1 % NSTAGE;
  auto rotate = [&]() __attribute__((always_inline)) {
    sc = sn;
    sn = sn + 1 == NSTAGE ? 0 : sn + 1;
  };
  if constexpr (EARLY) {
    // Two barriers per tile: the first (every wave has read both k-steps of
    // tile t) frees its stage, so tile t + NSTAGE's loads go out among the
    // MFMAs of k-step 0; the second (tile t + 1 landed everywhere) comes half
    // a tile later.  A load then has NSTAGE - 1/2 tiles of MFMA work to land
    // in, against NSTAGE - 1 when it waits for the single mid-tile barrier.
    for (int t = 0; t < nk; ++t) {
      rd(fb, lds + sc * BUF, 1);
      __builtin_amdgcn_s_waitcnt(0xC07F);                     // lgkmcnt(0): this wave is done reading tile t
      bare_barrier();                                         // ... every wave is: its stage is free
      __builtin_amdgcn_sched_barrier(0);
      mm_issue(fa, sc);                                       // k-step 0 of tile t; tile t + NSTAGE loads
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<(NSTAGE - 1) * LPW>();                      // tile t + 1 landed (tiles t + 2 .. in flight)
      bare_barrier();                                         // ... for every wave
      rd(fa, lds + sn * BUF, 0);                              // past the end: a repeated tile, unused
      __builtin_amdgcn_sched_barrier(0);
      mm(fb);                                                 // k-step 1 of tile t
      __builtin_amdgcn_sched_barrier(0);
      rotate();
    }
  } else {
    for (int t = 0; t < nk; ++t) {
      rd(fb, lds + sc * BUF, 1);
      __builtin_amdgcn_sched_barrier(0);
      mm(fa);                                                 // k-step 0 of tile t
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);                     // lgkmcnt(0): this wave is done reading tile t
      wait_vmcnt<(NSTAGE - 2) * LPW>();                      // tile t + 1 landed
      bare_barrier();                                         // ... for every wave; tile t is free
      rd(fa, lds + sn * BUF, 0);                              // past the end: a repeated tile, unused
      __builtin_amdgcn_sched_barrier(0);
      mm_issue(fb, sc);                                       // k-step 1 of tile t; tile t + NSTAGE loads
      __builtin_amdgcn_sched_barrier(0);
      rotate();
    }
  }
  wait_vmcnt<0>();                                            // the trailing repeated tiles

  if constexpr (TOP2) {
    // lane l holds rows m0 + wm WM + 16 j + l % 16 against weight rows
    // n0 + wn WN + 16 i + 4 (l / 16) + r: a running top-2 per (j, lane), then
    // across the four lane groups, then across the TN / WN waves of a row
    __shared__ float tv1[TN / WN][TM], tv2[TN / WN][TM];
    __shared__ int ti1[TN / WN][TM];
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = m0 + wm * WM + j * 16 + (lane & 15);
      Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int n = n0 + wn * WN + i * 16 + 4 * (lane >> 4);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < g.N) t = top2_push(t, acc[i][j][r], n + r);
        if (g.part != nullptr && m < g.M) {
          float* out = g.part + static_cast<int64_t>(m) * g.N + n;
          if (n + 3 < g.N && (g.N & 3) == 0) {
            *reinterpret_cast<float4*>(out) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < g.N) out[r] = acc[i][j][r];
          }
        }
      }
      t = top2_merge(t, top2_shfl_xor(t, 16));
      t = top2_merge(t, top2_shfl_xor(t, 32));
      if (lane < 16) {
        const int row = wm * WM + j * 16 + lane;
        tv1[wn][row] = t.v1;
        ti1[wn][row] = t.i1;
        tv2[wn][row] = t.v2;
      }
    }
    __syncthreads();
    for (int row = threadIdx.x; row < TM; row += NW * 64) {
      const int m = m0 + row;
      if (m >= g.M) continue;
      Top2 t{tv1[0][row], ti1[0][row], tv2[0][row]};
#pragma unroll
      for (int w = 1; w < TN / WN; ++w) t = top2_merge(t, Top2{tv1[w][row], ti1[w][row], tv2[w][row]});
      float* o = top2 + (static_cast<int64_t>(nt) * g.M + m) * 3;
      o[0] = t.v1;
      o[1] = __int_as_float(t.i1);
      o[2] = t.v2;
    }
    return;
  }

#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int n = n0 + wn * WN + i * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = m0 + wm * WM + j * 16 + (lane & 15);
      if (m >= g.M) continue;
      float* out = g.part + (static_cast<int64_t>(split) * g.M + m) * g.N + n;
      if (n + 3 < g.N && (g.N & 3) == 0) {
        *reinterpret_cast<float4*>(out) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < g.N) out[r] = acc[i][j][r];
      }
    }
  }
}

__global__ __launch_bounds__(256) void split_hilo_kernel(const float* x, int64_t ld, int rg, int64_t gs, int M,
                                                          int K, uint16_t* hi, uint16_t* lo) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 8;
  if (i >= static_cast<int64_t>(M) * K) return;
  const int m = static_cast<int>(i / K), k = static_cast<int>(i % K);   // K % 8 == 0
  const float* p = x + (m / rg) * gs + (m % rg) * ld + k;
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint4 h, l;
  split8(v, h, l);
  *reinterpret_cast<uint4*>(hi + i) = h;
  *reinterpret_cast<uint4*>(lo + i) = l;
}

// ------------------------------------------------------------------ fp32 path
constexpr int kF32Tile = 64;
constexpr int kF32K = 16;

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  __shared__ float As[kF32K][kF32Tile + 1], Ws[kF32K][kF32Tile + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * kF32Tile, n0 = blockIdx.x * kF32Tile;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += kF32K) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = threadIdx.x + 256 * i, r = e >> 4, kk = e & 15, k = k0 + kk;
      float av = 0.f, wv = 0.f;
      if (m0 + r < g.M && k < g.K) {
        const int s = k / g.a_cols;
        av = pick_src<float>(g, s)[a_row_off(g, m0 + r) + (k - s * g.a_cols)];
      }
      if (n0 + r < g.N && k < g.K) {
        const int n = n0 + r;
        const int64_t row = static_cast<int64_t>(n / g.w_rg) * g.w_gs + g.w_off + n % g.w_rg;
        wv = static_cast<const float*>(g.w)[row * g.w_ld + k];
      }
      As[kk][r] = av;
      Ws[kk][r] = wv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kF32K; ++kk) {
      float a[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[kk][ty * 4 + i]; w[i] = Ws[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < g.N) g.part[static_cast<int64_t>(m) * g.N + n] = acc[i][j];
    }
  }
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (s == nullptr || *s == 0) return dflt;
  const int v = atoi(s);
  return v > 0 ? v : dflt;
}

template <int MT, int AK, int WAVES, int KR>
hipError_t launch_v(const GemmArgs& a, const GemmPlan& p, hipStream_t st) {
  constexpr int HL = (AK == A_F32_SPLIT) ? 2 : 1;
  const size_t lds = static_cast<size_t>(KR / 32) * (MT / 16) * HL * 64 * sizeof(uint4);
  auto kern = gemm_stream_kernel<MT, AK, WAVES, KR>;
  const hipError_t e = ensure_dyn_lds(reinterpret_cast<const void*>(kern), static_cast<int>(lds));
  if (e != hipSuccess) return e;
  launch_k(kern, dim3(p.grid), dim3(64 * WAVES), lds, st, a);
  return hipGetLastError();
}

// LDS holds KR k values of MT activation rows (hi + lo for fp32 activations):
// 64 KB per workgroup for the 8-wave variants, 128 KB for the 16-wave one.
template <int MT>
hipError_t launch_mt(const GemmArgs& a, GemmAKind ak, const GemmPlan& p, hipStream_t st) {
  if (p.waves == 16) {
    if (ak == A_BF16) return launch_v<MT, A_BF16, 16, 65536 / MT>(a, p, st);
    return launch_v<MT, A_F32_SPLIT, 16, 32768 / MT>(a, p, st);
  }
  if (ak == A_BF16) return launch_v<MT, A_BF16, 8, 32768 / MT>(a, p, st);
  return launch_v<MT, A_F32_SPLIT, 8, 16384 / MT>(a, p, st);
}

int device_cus() {
  static std::atomic<int> cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);   // every thread computes the same value
  }
  return n;
}

}  // namespace

PendingEvents& pending_events() {
  thread_local PendingEvents pe;
  return pe;
}

namespace {
std::mutex g_attr_mu;
std::map<std::pair<int, const void*>, int> g_dyn_lds;    // (device, kernel) -> limit set
std::map<std::pair<int, const void*>, int> g_lds_room;   // (device, kernel) -> room computed
}  // namespace

hipError_t ensure_dyn_lds(const void* fn, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_attr_mu);
  auto it = g_dyn_lds.find({dev, fn});
  if (it != g_dyn_lds.end() && it->second >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) g_dyn_lds[{dev, fn}] = bytes;
  return e;
}

int dyn_lds_room(const void* fn, int lds_bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lk(g_attr_mu);
  auto it = g_lds_room.find({dev, fn});
  if (it != g_lds_room.end()) return it->second;
  int cap = 0;
  hipFuncAttributes fa{};
  if (hipFuncGetAttributes(&fa, fn) == hipSuccess && fa.sharedSizeBytes + 1024 < static_cast<size_t>(lds_bytes)) {
    cap = static_cast<int>(lds_bytes - fa.sharedSizeBytes) / 1024 * 1024;
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, cap) != hipSuccess) cap = 0;
  }
  g_lds_room[{dev, fn}] = cap;
  if (cap > 0) g_dyn_lds[{dev, fn}] = cap;
  return cap;
}

// Tile = 16 rows per wave x WAVES.  The split-K count S and the wave count are
// chosen by a small cost model.  The persistent grid (workgroups resident at
// once: 2 per CU with a 64 KB activation slice and 8 waves, 1 with 128 KB and
// 16 waves, rounded down to a multiple of S) works through S * tiles units of
// cps k-steps each; a wave streams its k-steps in groups of kStreamU loads, so a
// unit costs ceil(cps / U) * U steps plus a fixed per-unit overhead.  The HBM
// stream is shared, so a workgroup that runs out of units leaves its bandwidth
// to the others: the estimate is the mean work per workgroup plus a quarter of
// the gap to the busiest one.  Ties prefer fewer rounds, then 16 waves for a
// single round (one contiguous unit per CU) and 8 waves otherwise (more
// workgroups to balance), then fewer splits.  The K range of a unit must fit
// the LDS slice.  wide = true restricts the choice to 16 waves.
GemmPlan plan_gemm_mfma(int M, int N, int K, GemmAKind ak, bool wide) {
  GemmPlan best;
  best.MT = M <= 16 ? 16 : (M <= 32 ? 32 : 64);
  best.mtiles = (M + best.MT - 1) / best.MT;
  const int hl = ak == A_F32_SPLIT ? 2 : 1;
  const int ksteps = K / 32;
  const int overhead = env_int("DFLASH_GEMM_UNIT_OVERHEAD", 4);   // in k steps
  double best_cost = -1.0;
  long best_rounds = 0;
  for (int waves = wide ? 16 : 8; waves <= 16; waves += 8) {
    const int kr_max = (waves == 16 ? 65536 : 32768) / best.MT / hl;   // k values the LDS slice holds
    const int ntiles = (N + 16 * waves - 1) / (16 * waves);
    const long tiles = static_cast<long>(ntiles) * best.mtiles;
    const int cap = device_cus() * (waves == 16 ? 1 : 2);
    const int max_cps = kr_max / 32;
    for (int cps = max_cps < ksteps ? max_cps : ksteps; cps >= 1; --cps) {
      const int S = (ksteps + cps - 1) / cps;
      if ((ksteps + S - 1) / S != cps) continue;                    // each S once, with its smallest cps
      int grid = cap / S * S;
      if (grid < S) grid = S;
      const long units = static_cast<long>(S) * tiles;
      const long used = units < grid ? units : grid;
      const long rounds = (units + used - 1) / used;
      const long per_unit = (cps + kStreamU - 1) / kStreamU * kStreamU + overhead;
      const double mean = static_cast<double>(units) * per_unit / used;
      const double cost = mean + (rounds * per_unit - mean) / 4.0;
      bool take = best_cost < 0 || cost < best_cost - 1e-9;
      if (!take && cost <= best_cost + 1e-9) {
        if (rounds != best_rounds) take = rounds < best_rounds;
        else if (waves != best.waves) take = (rounds == 1) == (waves == 16);
      }
      if (take) {
        best_cost = cost;
        best_rounds = rounds;
        best.waves = waves;
        best.ntiles = ntiles;
        best.cps = cps;
        best.S = S;
        best.grid = static_cast<int>(used);
      }
    }
  }
  best.nchunks = ksteps;
  best.part_floats = static_cast<size_t>(best.S) * M * N;
  return best;
}

GemmPlan plan_gemm_tiled(int M, int N, int K, GemmAKind ak) {
  GemmPlan p;
  p.tiled = true;
  // register-staged kernel (fp32 A) or LDS-direct kernel
  // hi / lo planes: the smallest of the 32-, 64- and 128-row tiles that holds M,
  // 128 weight rows wide for 33-256 rows against a weight of <= 32768 rows;
  // bf16 A: 128 x 256 tiles (DFLASH_TILE64=2: always 256 x 128 hi / lo and
  // 256 x 256 bf16 tiles, for measurement)
  const bool small_tiles = ak == A_BF16_HILO && env_int("DFLASH_TILE64", 1) == 1;
  TileShape hl = !small_tiles ? kTileHiLo : M <= kTileHiLo32.tm ? kTileHiLo32
                                          : M <= kTileHiLo64.tm ? kTileHiLo64 : kTileHiLo;
  if (small_tiles && M > kTileHiLo64.tm && M <= 256 && N <= 32768) hl = kTileHiLoN128;
  if (small_tiles && M > kTileHiLo32.tm && M <= kTileHiLo64.tm && N <= 32768) hl = kTileHiLoN128M64;
  const TileShape bf = env_int("DFLASH_TILE64", 1) == 1 ? kTileBf16N128 : kTileBf16;
  const int tn = ak == A_F32_SPLIT ? kTileN : ak == A_BF16 ? bf.tn : hl.tn;
  const int tm = ak == A_F32_SPLIT ? kTileM : ak == A_BF16 ? bf.tm : hl.tm;
  p.MT = tm;
  p.tn = tn;
  p.mtiles = (M + tm - 1) / tm;
  p.ntiles = (N + tn - 1) / tn;
  const int ktiles = K / kTileK;
  const int tiles = p.mtiles * p.ntiles;
  if (ak != A_F32_SPLIT) {
    // LDS-direct kernel: one workgroup per CU (its stages fill most of the
    // LDS).  Split K so that the CUs are kept busy: S splits cost
    // ceil(tiles * S / CUs) rounds of 1 / S of the K range (in units of the
    // whole product spread evenly over the CUs), plus the extra fp32 partials
    // the consumer reads: (S - 1) * 8 bytes per output against the product's
    // 2 * K FLOP per output per bf16 product, at ~200 FLOP per HBM byte for
    // this kernel.  At most 16 splits of at least 4 k-tiles each; the smallest
    // S of least cost wins.
    const int cus = device_cus();
    const int products = ak == A_BF16_HILO ? 2 : 1;
    int best_s = 1;
    double best_cost = 1e30;
    for (int s = 1; s <= 16 && s <= ktiles / 4; ++s) {
      const double rounds = static_cast<double>((static_cast<long>(tiles) * s + cus - 1) / cus) / s;
      const double cost = rounds * cus / tiles + (s - 1) * 800.0 / (static_cast<double>(products) * K);
      if (cost < best_cost - 1e-9) best_cost = cost, best_s = s;
    }
    p.cps = (ktiles + best_s - 1) / best_s;
    p.S = (ktiles + p.cps - 1) / p.cps;
    p.part_floats = static_cast<size_t>(p.S) * M * N;
    return p;
  }
  const int target = 2 * device_cus();
  int want = (target + tiles - 1) / tiles;
  if (want < 1) want = 1;
  if (want > ktiles / 4) want = ktiles / 4 > 0 ? ktiles / 4 : 1;   // keep >= 4 k tiles per split
  p.cps = (ktiles + want - 1) / want;
  p.S = (ktiles + p.cps - 1) / p.cps;
  p.part_floats = static_cast<size_t>(p.S) * M * N;
  return p;
}

template <int HL, int NS, int TN, int TM, int WN, int WM, bool TOP2 = false>
hipError_t launch_tile_lds(GemmArgs a, dim3 grid, hipStream_t st, float* top2 = nullptr) {
  const size_t lds = static_cast<size_t>(NS) * (TN + TM * HL) * 8 * sizeof(uint4);
  // the kernel addresses a tile load as a scalar base (the W tile's k column,
  // an A plane's column) plus a byte offset per lane, kept below 2^31
  if (a.N < 1 || a.M < 1 || a.w_rg < 1 || a.a_rg < 1) return hipErrorInvalidValue;
  const int64_t wrow = static_cast<int64_t>(a.N - 1) / a.w_rg * a.w_gs + a.w_off +
                       std::min<int64_t>(a.w_rg - 1, a.N - 1);
  const int64_t arow = static_cast<int64_t>(a.M - 1) / a.a_rg * a.a_gs +
                       std::min<int64_t>(a.a_rg - 1, a.M - 1) * a.a_ld;
  if ((wrow * a.w_ld + kTileK) * 2 >= (int64_t{1} << 31) || (arow + kTileK) * 2 >= (int64_t{1} << 31))
    return hipErrorInvalidValue;
  a.xcd_tiles = env_int("DFLASH_TILE_XCD", 1) == 1 ? 1 : 0;   // 2: grid order (measurement)
  if (a.xcd_tiles) {
    a.ntiles = static_cast<int>(grid.x);
    a.mtiles = static_cast<int>(grid.y);
    a.S = static_cast<int>(grid.z);
    const long T = static_cast<long>(grid.x) * grid.y * grid.z;
    grid = dim3(static_cast<unsigned>((T + 7) / 8 * 8));
  }
  // the two-barrier loop that issues a tile's loads half a tile earlier pays
  // off for the two-stage hi / lo tile (the 8-layer drafter at 4 x 32 block
  // rows 2575 -> 2521 us); with bf16 A on 256 x 256 tiles (context ingest 579
  // -> 591 us) and with three stages it does not
  constexpr bool EARLY = HL == 2 && NS == 2;
  const hipError_t e = ensure_dyn_lds(
      reinterpret_cast<const void*>(gemm_tile_lds_kernel<HL, NS, TN, TM, WN, WM, TOP2, EARLY>), static_cast<int>(lds));
  if (e != hipSuccess) return e;
  launch_k(gemm_tile_lds_kernel<HL, NS, TN, TM, WN, WM, TOP2, EARLY>, grid, dim3((TN / WN) * (TM / WM) * 64), lds, st,
           a, top2);
  return hipGetLastError();
}

hipError_t launch_gemm_tiled_top2(const GemmArgs& a0, const GemmPlan& p, float* top2, float* logits, hipStream_t st) {
  constexpr TileShape T = kTileHiLo, T64 = kTileHiLo64, T32 = kTileHiLo32;
  if (!p.tiled || p.S != 1 || (p.MT != T.tm && p.MT != T64.tm && p.MT != T32.tm) || top2 == nullptr ||
      a0.a_cols % kTileK != 0 || a0.a_lo == nullptr)
    return hipErrorInvalidValue;
  GemmArgs a = a0;
  a.chunks_per_split = p.cps;
  a.part = logits;
  const dim3 grid(p.ntiles, p.mtiles, 1);
  constexpr TileShape TN1 = kTileHiLoN128, TN2 = kTileHiLoN128M64;
  if (p.tn == TN1.tn && p.MT == TN1.tm)
    return launch_tile_lds<2, TN1.ns, TN1.tn, TN1.tm, TN1.wn, TN1.wm, true>(a, grid, st, top2);
  if (p.tn == TN2.tn && p.MT == TN2.tm)
    return launch_tile_lds<2, TN2.ns, TN2.tn, TN2.tm, TN2.wn, TN2.wm, true>(a, grid, st, top2);
  if (p.tn != T.tn) return hipErrorInvalidValue;
  if (p.MT == T32.tm) return launch_tile_lds<2, T32.ns, T32.tn, T32.tm, T32.wn, T32.wm, true>(a, grid, st, top2);
  if (p.MT == T64.tm) return launch_tile_lds<2, T64.ns, T64.tn, T64.tm, T64.wn, T64.wm, true>(a, grid, st, top2);
  return launch_tile_lds<2, T.ns, T.tn, T.tm, T.wn, T.wm, true>(a, grid, st, top2);
}

hipError_t launch_gemm_mfma(const GemmArgs& a0, GemmAKind ak, const GemmPlan& p, hipStream_t st) {
  if (p.rk) return launch_gemm_rk(a0, p, nullptr, nullptr, st, ak);
  if (p.tiled && ak != A_F32_SPLIT) {
    GemmArgs a = a0;
    a.chunks_per_split = p.cps;
    const dim3 grid(p.ntiles, p.mtiles, p.S);
    if (a.a_cols % kTileK != 0) return hipErrorInvalidValue;
    if (ak == A_BF16) {
      constexpr TileShape T = kTileBf16, T2 = kTileBf16N128;
      if (p.tn == T2.tn && p.MT == T2.tm) return launch_tile_lds<1, T2.ns, T2.tn, T2.tm, T2.wn, T2.wm>(a, grid, st);
      if (p.MT != T.tm) return hipErrorInvalidValue;
      return launch_tile_lds<1, T.ns, T.tn, T.tm, T.wn, T.wm>(a, grid, st);
    }
    constexpr TileShape T = kTileHiLo, T64 = kTileHiLo64, T32 = kTileHiLo32, TN1 = kTileHiLoN128;
    constexpr TileShape TN2 = kTileHiLoN128M64;
    if (p.tn == TN1.tn && p.MT == TN1.tm) return launch_tile_lds<2, TN1.ns, TN1.tn, TN1.tm, TN1.wn, TN1.wm>(a, grid, st);
    if (p.tn == TN2.tn && p.MT == TN2.tm) return launch_tile_lds<2, TN2.ns, TN2.tn, TN2.tm, TN2.wn, TN2.wm>(a, grid, st);
    if (p.MT == T32.tm) return launch_tile_lds<2, T32.ns, T32.tn, T32.tm, T32.wn, T32.wm>(a, grid, st);
    if (p.MT == T64.tm) return launch_tile_lds<2, T64.ns, T64.tn, T64.tm, T64.wn, T64.wm>(a, grid, st);
    if (p.MT != T.tm) return hipErrorInvalidValue;
    return launch_tile_lds<2, T.ns, T.tn, T.tm, T.wn, T.wm>(a, grid, st);
  }
  if (p.tiled) {
    GemmArgs a = a0;
    a.chunks_per_split = p.cps;
    const int hl = ak == A_F32_SPLIT ? 2 : 1;
    const size_t lds = static_cast<size_t>(2) * ((kTileN / 16) * 2 + (kTileM / 16) * 2 * hl) * 64 * sizeof(uint4);
    const dim3 grid(p.ntiles, p.mtiles, p.S);
    if (ak == A_BF16) {
      const hipError_t e = ensure_dyn_lds(reinterpret_cast<const void*>(gemm_tile_kernel<A_BF16>), static_cast<int>(lds));
      if (e != hipSuccess) return e;
      launch_k(gemm_tile_kernel<A_BF16>, grid, dim3(256), lds, st, a);
    } else {
      const hipError_t e =
          ensure_dyn_lds(reinterpret_cast<const void*>(gemm_tile_kernel<A_F32_SPLIT>), static_cast<int>(lds));
      if (e != hipSuccess) return e;
      launch_k(gemm_tile_kernel<A_F32_SPLIT>, grid, dim3(256), lds, st, a);
    }
    return hipGetLastError();
  }
  GemmArgs a = a0;
  a.chunks_per_split = p.cps;
  a.S = p.S;
  a.ntiles = p.ntiles;
  a.mtiles = p.mtiles;
  switch (p.MT) {
    case 16: return launch_mt<16>(a, ak, p, st);
    case 32: return launch_mt<32>(a, ak, p, st);
    default: return launch_mt<64>(a, ak, p, st);
  }
}

// Rows beyond 16 run as C = ceil(M / 16) chunks on C workgroups per unit
// group.  The chunks of a unit group read the same weight tiles at the same
// time, so the launch has only 1 / C as many distinct weight streams in flight
// (each latency-bound, as one stream per CU is at 16 rows): measured on the
// 151936 x 4096 LM head, 28 rows (C = 2) take 268 us against 296 us for the
// streaming kernel and its top-2 pass, but C = 4 takes 521 us and C = 8 1022
// us.  So the tall forms (LM head, gate/up with SwiGLU) take up to 32 rows and
// the short split-K form stays at 16.
int rk_max_rows(bool tall) {
  const int r = env_int("DFLASH_RK_MAX_ROWS", tall ? kRkMaxRowsTall : 16);
  return r < 16 ? 16 : (r > kRkMaxRows ? kRkMaxRows : r / 16 * 16);
}

// Unit groups P of a register-K launch over `units` units (a multiple of S),
// C chunks: one workgroup per CU in all, P a multiple of S (a workgroup keeps
// its K range) and, when C > 1, of 8 (the chunk layout); every unit group must
// own a unit.  0: the shape does not fit.
static int rk_unit_groups(int S, int C, long units) {
  const int cus = device_cus();
  if (C == 1) {
    int grid = cus / S * S;
    if (grid > kRkMaxGrid) grid = kRkMaxGrid / S * S;
    if (grid < S) grid = S;
    return static_cast<int>(units < grid ? units : grid);
  }
  int a = S, b = 8;
  while (b != 0) { const int t = a % b; a = b; b = t; }
  const int step = S / a * 8;                 // lcm(S, 8)
  int grid = cus / C / step * step;
  if (grid < step) grid = step;
  if (grid > kRkMaxGrid || grid > units) return 0;
  return grid;
}

// Register-K plan: 16-row chunks, K a multiple of 16 waves x KS k-steps (KS = 8,
// else 4), at most one workgroup per CU (the grid is a multiple of the split
// count so that a workgroup keeps its K range).  Only worth it when the weight
// is tall: every workgroup reads the whole activation block once (M x K x 4
// bytes from L2), which must stay small against its share of W.
GemmPlan plan_gemm_rk(int M, int N, int K, bool top2) {
  GemmPlan p;
  if (M < 1 || M > rk_max_rows(true) || N < kRkMinN || env_int("DFLASH_GEMM_NO_RK", 0) != 0) return p;
  int ks = 0;
  if (K % (32 * 8 * kRkWaves) == 0) ks = 8;
  else if (K % (32 * 4 * kRkWaves) == 0) ks = 4;
  if (ks == 0) return p;
  const int S = K / (32 * ks * kRkWaves);
  if (top2 && S != 1) return p;
  const int C = (M + 15) / 16;
  const int ntiles = (N + 15) / 16;
  const int grid = rk_unit_groups(S, C, static_cast<long>(S) * ntiles);
  if (grid == 0) return p;
  p.rk = true;
  p.ks = ks;
  p.waves = kRkWaves;
  p.S = S;
  p.MT = 16;
  p.mtiles = 1;
  p.mr = C;
  p.ntiles = ntiles;
  p.cps = ks * kRkWaves;
  p.nchunks = K / 32;
  p.grid = grid;
  p.part_floats = top2 ? 0 : static_cast<size_t>(S) * M * N;
  return p;
}

// Register-K for a short weight: 8 waves of 4 k-steps (a K range of 1024 per
// workgroup, S = K / 1024 splits), so that a workgroup reads only 64 KB of the
// activation block while 256 workgroups keep the stream of 32 KB weight
// pieces deep.  Eight waves rather than sixteen with 2 k-steps: the same bytes
// in flight per CU with half the waves to launch and to reduce over
// (0.2 us a call, the step 849 -> 845 us).
GemmPlan plan_gemm_rk_short(int M, int N, int K, bool ks6) {
  GemmPlan p;
  if (M < 1 || M > rk_max_rows(false) || env_int("DFLASH_GEMM_NO_RK", 0) != 0) return p;
  const int C = (M + 15) / 16;
  const int ntiles = (N + 15) / 16;
  // Four k-steps per wave (a 1024-wide K range) unless six (1536) leave the
  // workgroups a more even share of units: a workgroup keeps one split, so
  // the grid is a multiple of the split count and the busiest workgroup sets
  // the time.  The 4096 x 12288 down projection: 12 splits on 252 workgroups,
  // 12-13 units of 4 k-steps each, against 8 splits on 256, 8 units of 6.
  // (Six only for single-source activations: a wave's K range must not
  // straddle two sources.)
  int kKsShort = 0, S = 0, grid = 0;
  long best = -1;
  for (const int ks : {4, 6}) {
    if (ks == 6 && !ks6) continue;
    if (K % (32 * ks * kRkShortWaves) != 0) continue;
    const int s = K / (32 * ks * kRkShortWaves);
    const long units = static_cast<long>(s) * ntiles;
    const int gr = rk_unit_groups(s, C, units);
    if (gr == 0) continue;
    const long cost = (units + gr - 1) / gr * ks;
    if (best < 0 || cost < best) best = cost, kKsShort = ks, S = s, grid = gr;
  }
  if (best < 0) return p;
  p.rk = true;
  p.ks = kKsShort;
  p.waves = kRkShortWaves;
  p.S = S;
  p.MT = 16;
  p.mtiles = 1;
  p.mr = C;
  p.ntiles = ntiles;
  p.cps = kKsShort * kRkShortWaves;
  p.nchunks = K / 32;
  p.grid = grid;
  p.part_floats = static_cast<size_t>(p.S) * M * N;
  return p;
}

// From 33 rows the tiled kernel (one 128-row tile, MFMA-bound) beats the
// weight-streaming kernels, whose fragment reads from LDS grow with the rows:
// the 8-layer drafter at 4 x 16 block rows 2358 -> 2235 us; at 32 rows and
// below it loses (4 x 8 rows 1843 -> 1923 us, 16 rows 880 -> 1000 us a step).
GemmPlan plan_gemm(int M, int N, int K, GemmAKind ak, bool wide) {
  const int tiled_rows = env_int("DFLASH_TILED_MIN_ROWS", 33);   // (measurement)
  if (M >= tiled_rows && K % kTileK == 0 && env_int("DFLASH_GEMM_NO_TILED", 0) == 0)
    return plan_gemm_tiled(M, N, K, ak);
  if ((ak == A_F32_SPLIT || ak == A_BF16) && M <= rk_max_rows(true)) {
    const GemmPlan r = plan_gemm_rk(M, N, K, false);
    if (r.rk && r.S == 1) return r;
    const GemmPlan q = plan_gemm_rk_short(M, N, K, ak == A_F32_SPLIT);
    if (q.rk) return q;
  }
  return plan_gemm_mfma(M, N, K, ak, wide);
}

// Launch one register-K instantiation.  Epilogues that write per tile get
// their workgroup's output tiles staged in dynamic LDS (written out after the
// weight stream) whenever they fit beside the kernel's static LDS.
template <int KS, int EP, int T, int AK = A_F32_SPLIT, int NW = kRkWaves>
hipError_t rk_launch(GemmArgs a, const GemmPlan& p, float* top2, float* logits, hipStream_t st) {
  const void* kern = reinterpret_cast<const void*>(&gemm_rk_kernel<KS, EP, T, AK, NW>);
  const int stage_cap = EP != RK_TOP2 ? dyn_lds_room(kern, kLdsBytes) : 0;   // dynamic LDS bytes it may use
  const size_t tile_bytes = (EP == RK_SWIGLU ? 8 : 16) * 16 * sizeof(float);
  const int slots = (p.S * p.ntiles + p.grid - 1) / p.grid;   // units a workgroup handles
  // the chunk layout: M rows in mr chunks, and unit groups in whole XCD rounds
  if (p.mr < 1 || (p.mr - 1) * 16 >= a.M || p.mr * 16 < a.M || (p.mr > 1 && p.grid % 8 != 0))
    return hipErrorInvalidValue;
  size_t shm = 0;
  a.stage_tiles = 0;
  a.rchunks = p.mr;
  if (EP != RK_TOP2 && static_cast<size_t>(slots) * tile_bytes <= static_cast<size_t>(stage_cap)) {
    a.stage_tiles = slots;
    shm = static_cast<size_t>(slots) * tile_bytes;
  }
  // the plan fixes the k-steps of a workgroup (its K range); the epilogue picks
  // how they are spread over waves
  if (p.cps != KS * NW || a.a_cols % (32 * KS) != 0) return hipErrorInvalidValue;
  launch_k(gemm_rk_kernel<KS, EP, T, AK, NW>, dim3(p.grid * p.mr), dim3(64 * NW), shm, st, a, top2,
                     logits);
  return hipGetLastError();
}

hipError_t launch_gemm_rk(const GemmArgs& a0, const GemmPlan& p, float* top2, float* logits, hipStream_t st,
                          GemmAKind ak) {
  if (!p.rk || a0.a_cols % (32 * p.ks) != 0 || (top2 != nullptr && p.S != 1)) return hipErrorInvalidValue;
  if (ak != A_F32_SPLIT && (ak != A_BF16 || top2 != nullptr)) return hipErrorInvalidValue;
  GemmArgs a = a0;
  a.S = p.S;
  a.ntiles = p.ntiles;
  a.mtiles = 1;
  a.chunks_per_split = p.cps;
  if (top2 != nullptr) {
    // the LM head runs its K range on eight waves of twice the k-steps: 205 ->
    // 200 us at 15 rows x 151936 x 4096 (the gate/up projection, 6 tiles per
    // workgroup against ~37, gains nothing from it and keeps sixteen)
    if (p.ks == 8 && a.a_cols % (32 * 16) == 0) return rk_launch<16, RK_TOP2, 1, A_F32_SPLIT, 8>(a, p, top2, logits, st);
    if (p.ks == 4 && a.a_cols % (32 * 8) == 0) return rk_launch<8, RK_TOP2, 1, A_F32_SPLIT, 8>(a, p, top2, logits, st);
    if (p.ks == 8) return rk_launch<8, RK_TOP2, 1>(a, p, top2, logits, st);
    return rk_launch<4, RK_TOP2, 1>(a, p, top2, logits, st);
  }
  // the short form (8 waves) streams one tile at a time as well: on cold weights
  // (34-100 MB, rotated past the Infinity Cache) one tile in flight per wave
  // beats two by 0.5-0.8 us per call and four lose 1-3 us
  const bool short_form = p.waves == kRkShortWaves;
  if (ak == A_BF16) {
    if (short_form) return rk_launch<4, RK_PART, 1, A_BF16, kRkShortWaves>(a, p, nullptr, nullptr, st);
    if (p.ks == 8) return rk_launch<8, RK_PART, 1, A_BF16>(a, p, nullptr, nullptr, st);
    return rk_launch<4, RK_PART, 1, A_BF16>(a, p, nullptr, nullptr, st);
  }
  if (short_form && p.ks == 6) return rk_launch<6, RK_PART, 1, A_F32_SPLIT, kRkShortWaves>(a, p, nullptr, nullptr, st);
  if (short_form) return rk_launch<4, RK_PART, 1, A_F32_SPLIT, kRkShortWaves>(a, p, nullptr, nullptr, st);
  if (p.ks == 8) return rk_launch<8, RK_PART, 1>(a, p, nullptr, nullptr, st);
  return rk_launch<4, RK_PART, 1>(a, p, nullptr, nullptr, st);
}

hipError_t launch_gemm_rk_sample(const GemmArgs& a0, const GemmPlan& p, float4* stats, float* logits,
                                 hipStream_t st) {
  if (!p.rk || p.S != 1 || a0.a_cols % (32 * p.ks) != 0 || stats == nullptr || logits == nullptr ||
      a0.su == nullptr)
    return hipErrorInvalidValue;
  GemmArgs a = a0;
  a.S = 1;
  a.ntiles = p.ntiles;
  a.mtiles = 1;
  a.chunks_per_split = p.cps;
  float* sp = reinterpret_cast<float*>(stats);
  // eight waves as for the top-2 LM head: 210 -> 208 us at 15 rows x 151936 x 4096
  if (p.ks == 8 && a.a_cols % (32 * 16) == 0) return rk_launch<16, RK_SAMPLE, 1, A_F32_SPLIT, 8>(a, p, sp, logits, st);
  if (p.ks == 4 && a.a_cols % (32 * 8) == 0) return rk_launch<8, RK_SAMPLE, 1, A_F32_SPLIT, 8>(a, p, sp, logits, st);
  if (p.ks == 8) return rk_launch<8, RK_SAMPLE, 1>(a, p, sp, logits, st);
  return rk_launch<4, RK_SAMPLE, 1>(a, p, sp, logits, st);
}

GemmPlan plan_gemm_rk_swiglu(int M, int F, int K) {
  GemmPlan p = plan_gemm_rk(M, 2 * F, K, true);   // a single K split
  if (!p.rk) return p;
  p.ntiles = (F + 7) / 8;
  if (p.grid > p.ntiles) {
    if (p.mr > 1) return GemmPlan{};   // unit groups stay a multiple of 8
    p.grid = p.ntiles;
  }
  return p;
}

hipError_t launch_gemm_rk_swiglu(const GemmArgs& a0, const GemmPlan& p, float* s_out, hipStream_t st) {
  if (!p.rk || p.S != 1 || a0.a_cols % (32 * p.ks) != 0) return hipErrorInvalidValue;
  GemmArgs a = a0;
  a.S = 1;
  a.ntiles = p.ntiles;
  a.mtiles = 1;
  a.chunks_per_split = p.cps;
  a.part = s_out;
  if (p.ks == 8) return rk_launch<8, RK_SWIGLU, 1>(a, p, nullptr, nullptr, st);
  return rk_launch<4, RK_SWIGLU, 1>(a, p, nullptr, nullptr, st);
}

hipError_t launch_split_hilo(const float* x, int64_t ld, int M, int K, uint16_t* hi, uint16_t* lo, hipStream_t st,
                             int rg, int64_t gs) {
  if (K % 8 != 0 || ld % 4 != 0 || gs % 4 != 0 || rg < 1) return hipErrorInvalidValue;
  const int64_t groups = static_cast<int64_t>(M) * K / 8;
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(split_hilo_kernel, dim3(static_cast<unsigned>((groups + 255) / 256)), dim3(256), 0, st, x, ld, rg,
                     gs, M, K, hi, lo);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t st) {
  dim3 grid((a.N + kF32Tile - 1) / kF32Tile, (a.M + kF32Tile - 1) / kF32Tile);
  launch_k(gemm_f32_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dflash
