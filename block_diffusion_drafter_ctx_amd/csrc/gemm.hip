// Weight-streaming GEMMs of the drafter path: C[m][n] = sum_k A[m][k] W[n][k].
//
// Every projection on the drafting path is "few activation rows x a large bf16
// weight matrix" (M = B*gamma <= 256 rows against up to 151936 x 4096 weights),
// so the kernel is built to stream W from HBM once at full width:
//   * a workgroup of 4 waves owns 128 consecutive weight rows (each wave two
//     16-row MFMA strips) and one K range (split-K across workgroups);
//   * each lane loads 16 B of one weight row per 32-wide k step (the A operand
//     of v_mfma_f32_16x16x32_bf16), prefetched one 128-wide chunk ahead;
//   * the activation chunk [MT rows x 128 k] is staged once per workgroup in
//     LDS, already in MFMA B-operand order (one conflict-free 16 B read per
//     lane), double-buffered so one barrier per chunk suffices;
//   * fp32 activations are split into bf16 hi + lo and multiplied twice, which
//     keeps ~16 significant bits against the exact bf16 weights at no cost on an
//     HBM-bound kernel;
//   * partial sums go to a [split][M][N] fp32 buffer reduced in a fixed order by
//     the consumer (deterministic, no float atomics), or, for the LM head, are
//     reduced in-kernel to one top-2 (value, index) per row and weight tile.
// The fp32 storage path uses a plain LDS-tiled FMA GEMM (tiny workloads only).
#include "common.h"
#include "launch.h"

#include <stdlib.h>

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int kStrips = 2;
constexpr int kKS = kGemmKC / 32;   // 32-wide k steps per chunk

template <typename T>
__device__ __forceinline__ const T* pick_src(const GemmArgs& g, int s) {
  // Select chain instead of a dynamic index into the kernel-argument array.
  const void* p = g.a_src[0];
#pragma unroll
  for (int i = 1; i < kMaxSrc; ++i) p = (s == i) ? g.a_src[i] : p;
  return static_cast<const T*>(p);
}

__device__ __forceinline__ int64_t a_row_off(const GemmArgs& g, int r) {
  return static_cast<int64_t>(r / g.a_rg) * g.a_gs + static_cast<int64_t>(r % g.a_rg) * g.a_ld;
}

template <int MT, int AK, bool TOP2>
__global__ __launch_bounds__(kThreads) void gemm_mfma_kernel(GemmArgs g) {
  constexpr int MTL = MT / 16;
  constexpr int HL = (AK == A_F32_SPLIT) ? 2 : 1;
  constexpr int NG = MT / 16;                 // 8-wide A groups per thread per chunk
  constexpr int BUF = kKS * MTL * HL * 64;    // uint4 per LDS buffer
  __shared__ uint4 lds[2 * BUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntile = blockIdx.x, split = blockIdx.y, mtile = blockIdx.z;
  const int m0 = mtile * MT;
  const int nchunks = (g.K + kGemmKC - 1) / kGemmKC;
  const int c_begin = split * g.chunks_per_split;
  const int c_end = min(nchunks, c_begin + g.chunks_per_split);

  // ---- weight row pointers (rows past N are clamped; their results are dropped)
  const uint16_t* wrow[kStrips];
#pragma unroll
  for (int st = 0; st < kStrips; ++st) {
    int n = ntile * kGemmTileN + wave * 32 + st * 16 + (lane & 15);
    n = min(n, g.N - 1);
    const int64_t row = static_cast<int64_t>(n / g.w_rg) * g.w_gs + g.w_off + n % g.w_rg;
    wrow[st] = static_cast<const uint16_t*>(g.w) + row * g.w_ld + 8 * (lane >> 4);
  }

  // ---- A staging geometry: group q = tid + 256*i covers row q/16, k 8*(q%16)..+7
  int64_t arow[NG];
  bool avalid[NG];
  int lds_slot[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int q = tid + kThreads * i, m = q >> 4, k8 = q & 15;
    const int r = m0 + m;
    avalid[i] = r < g.M;
    arow[i] = avalid[i] ? a_row_off(g, r) : 0;
    lds_slot[i] = (((k8 >> 2) * MTL + (m >> 4)) * HL) * 64 + (k8 & 3) * 16 + (m & 15);
  }

  auto load_w = [&](uint4 (&wr)[kKS][kStrips], int c) {
    const int kb = c * kGemmKC;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      if (kb + ks * 32 < g.K) {
#pragma unroll
        for (int st = 0; st < kStrips; ++st)
          wr[ks][st] = *reinterpret_cast<const uint4*>(wrow[st] + kb + ks * 32);
      }
    }
  };

  // A registers for the chunk being staged
  float af[(AK == A_F32_SPLIT) ? NG * 8 : 1];
  uint4 ab[(AK == A_BF16) ? NG : 1];

  auto load_a = [&](int c) {
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int q = tid + kThreads * i;
      const int k = c * kGemmKC + 8 * (q & 15);
      const bool ok = avalid[i] && k < g.K;
      const int s = k / g.a_cols, col = k - s * g.a_cols;
      if constexpr (AK == A_F32_SPLIT) {
        float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
        if (ok) {
          const float* p = pick_src<float>(g, s) + arow[i] + col;
          x0 = *reinterpret_cast<const float4*>(p);
          x1 = *reinterpret_cast<const float4*>(p + 4);
        }
        af[i * 8 + 0] = x0.x; af[i * 8 + 1] = x0.y; af[i * 8 + 2] = x0.z; af[i * 8 + 3] = x0.w;
        af[i * 8 + 4] = x1.x; af[i * 8 + 5] = x1.y; af[i * 8 + 6] = x1.z; af[i * 8 + 7] = x1.w;
      } else {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (ok) v = *reinterpret_cast<const uint4*>(pick_src<uint16_t>(g, s) + arow[i] + col);
        ab[i] = v;
      }
    }
  };

  auto store_a = [&](uint4* buf) {
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      if constexpr (AK == A_F32_SPLIT) {
        uint4 hi, lo;
        split8(&af[i * 8], hi, lo);
        buf[lds_slot[i]] = hi;
        buf[lds_slot[i] + 64] = lo;
      } else {
        buf[lds_slot[i]] = ab[i];
      }
    }
  };

  f32x4_t acc[kStrips][MTL];
#pragma unroll
  for (int st = 0; st < kStrips; ++st)
#pragma unroll
    for (int mt = 0; mt < MTL; ++mt) acc[st][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint4 (&wr)[kKS][kStrips], const uint4* buf, int c) {
    const int nks = min(kKS, (g.K - c * kGemmKC) / 32);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      if (ks < nks) {
#pragma unroll
        for (int mt = 0; mt < MTL; ++mt) {
          const uint4 bh = buf[((ks * MTL + mt) * HL) * 64 + lane];
#pragma unroll
          for (int st = 0; st < kStrips; ++st) acc[st][mt] = mfma16x16x32(wr[ks][st], bh, acc[st][mt]);
          if constexpr (HL == 2) {
            const uint4 bl = buf[((ks * MTL + mt) * HL + 1) * 64 + lane];
#pragma unroll
            for (int st = 0; st < kStrips; ++st) acc[st][mt] = mfma16x16x32(wr[ks][st], bl, acc[st][mt]);
          }
        }
      }
    }
  };

  uint4 wr0[kKS][kStrips], wr1[kKS][kStrips];
  if (c_begin < c_end) {
    load_w(wr0, c_begin);
    load_a(c_begin);
    store_a(lds);
    __syncthreads();
    for (int c = c_begin; c < c_end; c += 2) {
      const bool has1 = c + 1 < c_end;
      if (has1) { load_w(wr1, c + 1); load_a(c + 1); }
      compute(wr0, lds, c);
      if (has1) store_a(lds + BUF);
      __syncthreads();
      if (!has1) break;
      const bool has2 = c + 2 < c_end;
      if (has2) { load_w(wr0, c + 2); load_a(c + 2); }
      compute(wr1, lds + BUF, c + 1);
      if (has2) store_a(lds);
      __syncthreads();
    }
  }

  const int nbase = ntile * kGemmTileN + wave * 32 + 4 * (lane >> 4);
  if constexpr (!TOP2) {
#pragma unroll
    for (int st = 0; st < kStrips; ++st) {
#pragma unroll
      for (int mt = 0; mt < MTL; ++mt) {
        const int m = m0 + mt * 16 + (lane & 15);
        const int n = nbase + st * 16;
        if (m < g.M) {
          float* out = g.part + (static_cast<int64_t>(split) * g.M + m) * g.N + n;
          if (n + 3 < g.N && (g.N & 3) == 0) {
            *reinterpret_cast<float4*>(out) =
                make_float4(acc[st][mt][0], acc[st][mt][1], acc[st][mt][2], acc[st][mt][3]);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < g.N) out[r] = acc[st][mt][r];
          }
        }
      }
    }
  } else {
    // LM head: per-row top-2 over this workgroup's 128 weight rows.
    __shared__ float red[4][MT][3];
#pragma unroll
    for (int mt = 0; mt < MTL; ++mt) {
      const int m = m0 + mt * 16 + (lane & 15);
      Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
#pragma unroll
      for (int st = 0; st < kStrips; ++st) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = nbase + st * 16 + r;
          if (n < g.N) {
            t = top2_push(t, acc[st][mt][r], n);
            if (g.logits != nullptr && m < g.M) g.logits[static_cast<int64_t>(m) * g.N + n] = acc[st][mt][r];
          }
        }
      }
      t = top2_merge(t, top2_shfl_xor(t, 16));
      t = top2_merge(t, top2_shfl_xor(t, 32));
      if (lane < 16) {
        red[wave][mt * 16 + lane][0] = t.v1;
        red[wave][mt * 16 + lane][1] = __int_as_float(t.i1);
        red[wave][mt * 16 + lane][2] = t.v2;
      }
    }
    __syncthreads();
    if (tid < MT && m0 + tid < g.M) {
      Top2 t{red[0][tid][0], __float_as_int(red[0][tid][1]), red[0][tid][2]};
#pragma unroll
      for (int w = 1; w < 4; ++w)
        t = top2_merge(t, Top2{red[w][tid][0], __float_as_int(red[w][tid][1]), red[w][tid][2]});
      float* o = g.top2 + (static_cast<int64_t>(ntile) * g.M + m0 + tid) * 3;
      o[0] = t.v1;
      o[1] = __int_as_float(t.i1);
      o[2] = t.v2;
    }
  }
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

template <int MT, int AK, bool TOP2>
hipError_t launch3(const GemmArgs& a, const GemmPlan& p, hipStream_t st) {
  dim3 grid(p.ntiles, p.S, p.mtiles);
  hipLaunchKernelGGL((gemm_mfma_kernel<MT, AK, TOP2>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int MT>
hipError_t launch2(const GemmArgs& a, GemmAKind ak, const GemmPlan& p, bool top2, hipStream_t st) {
  if (ak == A_BF16) return top2 ? launch3<MT, A_BF16, true>(a, p, st) : launch3<MT, A_BF16, false>(a, p, st);
  return top2 ? launch3<MT, A_F32_SPLIT, true>(a, p, st) : launch3<MT, A_F32_SPLIT, false>(a, p, st);
}

}  // namespace

GemmPlan plan_gemm_mfma(int M, int N, int K, bool force_single_split) {
  GemmPlan p;
  p.MT = M <= 16 ? 16 : (M <= 32 ? 32 : 64);
  p.mtiles = (M + p.MT - 1) / p.MT;
  p.ntiles = (N + kGemmTileN - 1) / kGemmTileN;
  p.nchunks = (K + kGemmKC - 1) / kGemmKC;
  int want = 1;
  if (!force_single_split) {
    const int target = env_int("DFLASH_GEMM_WG_TARGET", 512);
    const int tiles = p.ntiles * p.mtiles;
    want = (target + tiles - 1) / tiles;
    want = want < 1 ? 1 : (want > p.nchunks ? p.nchunks : want);
  }
  p.cps = (p.nchunks + want - 1) / want;
  p.S = (p.nchunks + p.cps - 1) / p.cps;
  p.part_floats = static_cast<size_t>(p.S) * M * N;
  return p;
}

hipError_t launch_gemm_mfma(const GemmArgs& a0, GemmAKind ak, const GemmPlan& p, bool top2,
                            hipStream_t st) {
  GemmArgs a = a0;
  a.chunks_per_split = p.cps;
  switch (p.MT) {
    case 16: return launch2<16>(a, ak, p, top2, st);
    case 32: return launch2<32>(a, ak, p, top2, st);
    default: return launch2<64>(a, ak, p, top2, st);
  }
}

hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t st) {
  dim3 grid((a.N + kF32Tile - 1) / kF32Tile, (a.M + kF32Tile - 1) / kF32Tile);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dflash
