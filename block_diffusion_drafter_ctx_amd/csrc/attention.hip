// Injected-context attention of the drafter block.
//
// For sequence b and KV head j, the G*gamma query rows of the block (all query
// heads of the group, all block rows) attend without a mask to every key of
// [context ; block] = cache rows [0, len_b + gamma) of that head ("DFlash:
// Block Diffusion for Flash Speculative Decoding 논문 정리", section "KV
// Injection 메커니즘"; bidirectional inside the block, section "추론 구조").
//
// gfx950 design (bf16 storage): few query rows against a long key stream, so
// the kernel is HBM-bound and is split over keys:
//   * one workgroup per (sequence, KV head, key range); one wave per 16 query
//     rows; all waves of a workgroup read the same keys (L1/L2 shared);
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16:
//     each lane loads 16 B of a key row straight from the row-major K cache;
//     the fp32 queries (pre-scaled by log2(e)/sqrt(d)) are split into bf16
//     hi + lo and multiplied twice;
//   * online softmax per row with exp2; the MFMA output layout of S^T (4 keys of
//     one row per lane) is exactly the B-operand layout P^T of the next MFMA
//     after a fixed permutation of the 32 keys, so probabilities never leave
//     registers;
//   * O^T = V^T P^T reads values from the transposed V cache ([d][cap], keys
//     contiguous) with two 8-byte loads per lane, P again split hi + lo;
//   * each workgroup writes (max, sum, O) per row; a combine kernel merges the
//     key ranges in a fixed order (log-sum-exp), so results are deterministic.
// An fp32 KV cache (with bf16 weights) runs the same kernel with K and V split
// into bf16 hi + lo on load (three MFMAs per product instead of two).  fp32
// weights use a plain one-wave-per-(row, head) online-softmax kernel.
#include "common.h"
#include "launch.h"

#include <stdlib.h>

#include <type_traits>

namespace dflash {
namespace {

constexpr int kRowsPerGroup = 128;   // query rows per workgroup (8 waves)

__device__ __forceinline__ void decode_item(const AttnArgs& a, int item, int& b, int& j, int& sp) {
  b = 0;
  while (b + 1 < a.B && item >= a.item_off[b + 1]) ++b;
  const int local = item - a.item_off[b];
  j = local / a.nsplit[b];
  sp = local - j * a.nsplit[b];
}

// Raw key / value loads (kept in registers until used, so the next block's
// loads can be in flight during this block's math) and their conversion into
// MFMA operands (bf16 as is; fp32 split into bf16 hi + lo).
template <typename TKV> struct KVLoad;
template <> struct KVLoad<uint16_t> {
  static constexpr bool kSplit = false;
  struct Raw { uint4 u; };
  // 8 consecutive elements
  static __device__ __forceinline__ Raw row8(const uint16_t* p) { return Raw{*reinterpret_cast<const uint4*>(p)}; }
  // elements [k, k+4) and [k+16, k+20) of one transposed value row
  static __device__ __forceinline__ Raw pair4(const uint16_t* p, int k) {
    const uint2 v0 = *reinterpret_cast<const uint2*>(p + k);
    const uint2 v1 = *reinterpret_cast<const uint2*>(p + k + 16);
    return Raw{make_uint4(v0.x, v0.y, v1.x, v1.y)};
  }
  // same with every index clamped to <= last
  static __device__ __forceinline__ Raw pair4_clamped(const uint16_t* p, int k, int last) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kl = min(k + (e >> 1) * 16 + 2 * (e & 1), last), kh = min(k + (e >> 1) * 16 + 2 * (e & 1) + 1, last);
      w[e] = static_cast<uint32_t>(p[kl]) | (static_cast<uint32_t>(p[kh]) << 16);
    }
    return Raw{make_uint4(w[0], w[1], w[2], w[3])};
  }
  static __device__ __forceinline__ void ops(const Raw& r, uint4& hi, uint4& lo) { hi = r.u; lo = r.u; }
};
template <> struct KVLoad<float> {
  static constexpr bool kSplit = true;
  struct Raw { float4 a, b; };
  static __device__ __forceinline__ Raw row8(const float* p) {
    return Raw{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
  }
  static __device__ __forceinline__ Raw pair4(const float* p, int k) {
    return Raw{*reinterpret_cast<const float4*>(p + k), *reinterpret_cast<const float4*>(p + k + 16)};
  }
  static __device__ __forceinline__ Raw pair4_clamped(const float* p, int k, int last) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = p[min(k + (e >> 2) * 16 + (e & 3), last)];
    return Raw{make_float4(x[0], x[1], x[2], x[3]), make_float4(x[4], x[5], x[6], x[7])};
  }
  static __device__ __forceinline__ void ops(const Raw& r, uint4& hi, uint4& lo) {
    const float x[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
    split8(x, hi, lo);
  }
};

template <int HD, typename TKV>
__global__ __launch_bounds__(512) void attn_mfma_kernel(AttnArgs a) {
  using LD = KVLoad<TKV>;
  constexpr int DS = HD / 32;   // 32-wide d steps of the score MFMA
  constexpr int DT = HD / 16;   // 16-wide d tiles of the output MFMA
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g4 = lane >> 4;
  const int item = blockIdx.x;
  int b, j, sp;
  decode_item(a, item, b, j, sp);
  const int nk = a.nkeys[b];
  const int kbeg = sp * a.split_keys;
  const int kend = min(nk, kbeg + a.split_keys);
  const int r = blockIdx.y * kRowsPerGroup + wave * 16 + (lane & 15);
  const int G = a.Hq / a.Hkv;

  uint4 qh[DS], ql[DS];
  if (r < a.R) {
    const int h = j * G + r / a.gamma, i = r % a.gamma;
    const float* qp = a.q + (static_cast<int64_t>(b * a.gamma + i) * a.Hq + h) * HD + 8 * g4;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const float4 x0 = *reinterpret_cast<const float4*>(qp + ds * 32);
      const float4 x1 = *reinterpret_cast<const float4*>(qp + ds * 32 + 4);
      float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= a.scale_log2;
      split8(x, qh[ds], ql[ds]);
    }
  } else {
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) { qh[ds] = make_uint4(0, 0, 0, 0); ql[ds] = qh[ds]; }
  }

  const int64_t head = static_cast<int64_t>(b) * a.Hkv + j;
  const TKV* kbase = static_cast<const TKV*>(a.kc) + head * a.cap * HD + 8 * g4;
  const TKV* vbase = static_cast<const TKV*>(a.vc) + head * HD * a.cap;

  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  using Raw = typename LD::Raw;
  Raw kr[2][DS], vr[DT];

  // Loads of one 32-key block; FULL blocks need no clamping (the ragged tail of
  // a key range is a separate, clamped block after the main loop).
  auto load_k = [&](int k0, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = FULL ? k0 + kt * 16 + (lane & 15) : min(k0 + kt * 16 + (lane & 15), kend - 1);
      const TKV* kp = kbase + static_cast<int64_t>(key) * HD;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) kr[kt][ds] = LD::row8(kp + ds * 32);
    }
  };
  auto load_v = [&](int k0, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const TKV* vp = vbase + static_cast<int64_t>(dt * 16 + (lane & 15)) * a.cap;
      vr[dt] = FULL ? LD::pair4(vp, k0 + 4 * g4) : LD::pair4_clamped(vp, k0 + 4 * g4, kend - 1);
    }
  };

  // One block in two phases: scores (reads kr), then online softmax (base 2;
  // the scale is folded into Q) and PV (reads vr).
  auto scores = [&](f32x4_t (&s)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        uint4 kh, kl;
        LD::ops(kr[kt][ds], kh, kl);
        s[kt] = mfma16x16x32(kh, qh[ds], s[kt]);
        s[kt] = mfma16x16x32(kh, ql[ds], s[kt]);
        if constexpr (LD::kSplit) s[kt] = mfma16x16x32(kl, qh[ds], s[kt]);
      }
    }
  };
  auto softmax_pv = [&](const f32x4_t (&s)[2], int k0, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    float p[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        p[kt * 4 + rr] = (FULL || k0 + kt * 16 + 4 * g4 + rr < kend) ? s[kt][rr] : -INFINITY;
    float mx = p[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, p[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = exp2f(p[e] - m_new);
      ps += p[e];
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
    if (__any(alpha != 1.0f)) {            // skipped once every row's max has settled
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    uint4 ph, pl;
    split8(p, ph, pl);
    // O^T += V^T P^T; k-slot e of lane group g4 <-> key k0 + 4*g4 + e (e < 4),
    // k0 + 16 + 4*g4 + (e - 4) (e >= 4): the layout S^T left in p[].
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      uint4 vh, vl;
      LD::ops(vr[dt], vh, vl);
      o[dt] = mfma16x16x32(vh, ph, o[dt]);
      o[dt] = mfma16x16x32(vh, pl, o[dt]);
      if constexpr (LD::kSplit) o[dt] = mfma16x16x32(vl, ph, o[dt]);
    }
  };

  using Full = std::integral_constant<bool, true>;
  using Tail = std::integral_constant<bool, false>;
  const int kfull = kbeg + ((kend - kbeg) / 32) * 32;   // end of the full blocks
  // bf16 caches prefetch the next block's keys during this block's softmax and
  // PV and its values right after; fp32 caches (twice the registers per key)
  // load keys and values together at the top of each block instead.
  constexpr bool kPrefetch = !LD::kSplit;
  if (kPrefetch && kbeg < kfull) {
    load_k(kbeg, Full{});
    load_v(kbeg, Full{});
  }
  for (int k0 = kbeg; k0 < kfull; k0 += 32) {
    f32x4_t s[2];
    if (!kPrefetch) {
      load_k(k0, Full{});
      load_v(k0, Full{});
      scores(s);
      softmax_pv(s, k0, Full{});
    } else {
      const bool more = k0 + 32 < kfull;
      scores(s);
      if (more) load_k(k0 + 32, Full{});   // next keys fly during softmax + PV
      softmax_pv(s, k0, Full{});
      if (more) load_v(k0 + 32, Full{});
    }
  }
  if (kfull < kend) {
    f32x4_t s[2];
    load_k(kfull, Tail{});
    load_v(kfull, Tail{});
    scores(s);
    softmax_pv(s, kfull, Tail{});
  }

  float l_tot = l_run + __shfl_xor(l_run, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);
  if (r < a.Rpad) {
    float* po = a.part_o + (static_cast<int64_t>(item) * a.Rpad + r) * HD + 4 * g4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(po + dt * 16) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (g4 == 0) {
      float* pm = a.part_ml + (static_cast<int64_t>(item) * a.Rpad + r) * 2;
      pm[0] = m_run;
      pm[1] = l_tot;
    }
  }
}

// Merge the key ranges of one (row, head): O = sum_s 2^(m_s-M) O_s / sum_s 2^(m_s-M) l_s.
// The split weights are computed once per row into LDS; the O loads of all
// splits are then independent.
constexpr int kMaxSplitsLds = 1024;

__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  __shared__ float wts[kMaxSplitsLds];
  __shared__ float inv_l;
  const int idx = blockIdx.x;
  const int m = idx / a.Hq, h = idx % a.Hq;
  const int b = m / a.gamma, i = m % a.gamma;
  const int G = a.Hq / a.Hkv, j = h / G;
  const int r = (h - j * G) * a.gamma + i;
  const int ns = a.nsplit[b];
  const int it0 = a.item_off[b] + j * ns;
  if (threadIdx.x < 64) {
    float M = -INFINITY;
    for (int s = threadIdx.x; s < ns; s += 64) M = fmaxf(M, a.part_ml[(static_cast<int64_t>(it0 + s) * a.Rpad + r) * 2]);
    M = wave_max(M);
    float L = 0.f;
    for (int s = threadIdx.x; s < ns; s += 64) {
      const float* ml = a.part_ml + (static_cast<int64_t>(it0 + s) * a.Rpad + r) * 2;
      const float w = exp2f(ml[0] - M);
      wts[s] = w;
      L += w * ml[1];
    }
    L = wave_sum(L);
    if (threadIdx.x == 0) inv_l = 1.0f / L;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < a.d; c += blockDim.x) {
    float O = 0.f;
#pragma unroll 8
    for (int s = 0; s < ns; ++s) O += wts[s] * a.part_o[(static_cast<int64_t>(it0 + s) * a.Rpad + r) * a.d + c];
    a.o_out[(static_cast<int64_t>(m) * a.Hq + h) * a.d + c] = O * inv_l;
  }
}

// fp32 storage: one wave per (block row, query head), keys walked in order.
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  const int idx = blockIdx.x, lane = threadIdx.x;
  const int m = idx / a.Hq, h = idx % a.Hq;
  const int b = m / a.gamma;
  const int G = a.Hq / a.Hkv, j = h / G;
  const float* qp = a.q + (static_cast<int64_t>(m) * a.Hq + h) * a.d;
  const float q0 = lane < a.d ? qp[lane] * a.scale_log2 : 0.f;
  const float q1 = lane + 64 < a.d ? qp[lane + 64] * a.scale_log2 : 0.f;
  const int64_t head = static_cast<int64_t>(b) * a.Hkv + j;
  const float* kb = static_cast<const float*>(a.kc) + head * a.cap * a.d;
  const float* vb = static_cast<const float*>(a.vc) + head * a.d * a.cap;
  float m_run = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int t = 0; t < a.nkeys[b]; ++t) {
    const float* kp = kb + static_cast<int64_t>(t) * a.d;
    float part = lane < a.d ? q0 * kp[lane] : 0.f;
    if (lane + 64 < a.d) part += q1 * kp[lane + 64];
    const float s = wave_sum(part);
    const float m_new = fmaxf(m_run, s);
    const float alpha = exp2f(m_run - m_new), p = exp2f(s - m_new);
    l = l * alpha + p;
    if (lane < a.d) o0 = o0 * alpha + p * vb[static_cast<int64_t>(lane) * a.cap + t];
    if (lane + 64 < a.d) o1 = o1 * alpha + p * vb[static_cast<int64_t>(lane + 64) * a.cap + t];
    m_run = m_new;
  }
  float* op = a.o_out + (static_cast<int64_t>(m) * a.Hq + h) * a.d;
  if (lane < a.d) op[lane] = o0 / l;
  if (lane + 64 < a.d) op[lane + 64] = o1 / l;
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (s == nullptr || *s == 0) return dflt;
  const int v = atoi(s);
  return v > 0 ? v : dflt;
}

int waves_per_group(int R) {
  const int w = (R + 15) / 16;
  return w < 8 ? w : 8;
}

}  // namespace

constexpr int kAttnItemTarget = 1024;

AttnPlan plan_attention(int B, const int32_t* nkeys, int Hkv, int R, int d) {
  AttnPlan p;
  int64_t total = 0;
  for (int b = 0; b < B; ++b) total += nkeys[b];
  const int target = env_int("DFLASH_ATTN_ITEMS", kAttnItemTarget);
  const int min_keys = env_int("DFLASH_ATTN_MIN_KEYS", 128);
  int64_t sk = (total * Hkv + target - 1) / target;
  sk = ((sk + 31) / 32) * 32;
  if (sk < min_keys) sk = ((min_keys + 31) / 32) * 32;
  int maxk = 0;
  for (int b = 0; b < B; ++b) maxk = nkeys[b] > maxk ? nkeys[b] : maxk;
  const int64_t sk_min = ((maxk + kMaxSplitsLds - 1) / kMaxSplitsLds + 31) / 32 * 32;   // combine's LDS table
  if (sk < sk_min) sk = sk_min;
  p.split_keys = static_cast<int>(sk);
  p.item_off[0] = 0;
  for (int b = 0; b < B; ++b) {
    p.nsplit[b] = static_cast<int>((nkeys[b] + sk - 1) / sk);
    p.item_off[b + 1] = p.item_off[b] + Hkv * p.nsplit[b];
  }
  p.items = p.item_off[B];
  p.row_groups = (R + kRowsPerGroup - 1) / kRowsPerGroup;
  p.Rpad = p.row_groups * waves_per_group(R) * 16;
  if (R > kRowsPerGroup) p.Rpad = p.row_groups * kRowsPerGroup;
  p.part_floats = static_cast<size_t>(p.items) * p.Rpad * (d + 2);
  return p;
}

size_t attention_part_bound(int B, int Hkv, int R, int d) {
  const int row_groups = (R + kRowsPerGroup - 1) / kRowsPerGroup;
  const int rpad = R > kRowsPerGroup ? row_groups * kRowsPerGroup : waves_per_group(R) * 16;
  const size_t items = static_cast<size_t>(env_int("DFLASH_ATTN_ITEMS", kAttnItemTarget)) + static_cast<size_t>(B) * Hkv;
  return items * rpad * (d + 2);
}

hipError_t launch_attention(const AttnArgs& a0, const AttnPlan& p, bool bf16_weights, bool bf16_cache,
                            hipStream_t st, void* stop_event) {
  AttnArgs a = a0;
  if (!bf16_weights) {
    hipLaunchKernelGGL(attn_f32_kernel, dim3(a.B * a.gamma * a.Hq), dim3(64), 0, st, a);
    if (stop_event != nullptr) (void)hipEventRecord(static_cast<hipEvent_t>(stop_event), st);
    return hipGetLastError();
  }
  a.split_keys = p.split_keys;
  a.items = p.items;
  a.Rpad = p.Rpad;
  for (int b = 0; b < a.B; ++b) { a.nsplit[b] = p.nsplit[b]; a.item_off[b] = p.item_off[b]; }
  a.item_off[a.B] = p.item_off[a.B];
  const dim3 grid(p.items, p.row_groups);
  const dim3 block(64 * waves_per_group(a.R));
  if (bf16_cache) {
    if (a.d == 128) hipLaunchKernelGGL((attn_mfma_kernel<128, uint16_t>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_mfma_kernel<64, uint16_t>), grid, block, 0, st, a);
  } else {
    if (a.d == 128) hipLaunchKernelGGL((attn_mfma_kernel<128, float>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_mfma_kernel<64, float>), grid, block, 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (stop_event != nullptr) (void)hipEventRecord(static_cast<hipEvent_t>(stop_event), st);
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.B * a.gamma * a.Hq), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace dflash
