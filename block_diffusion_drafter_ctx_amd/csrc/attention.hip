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

// Key / value staging.  A workgroup streams its key range in 32-key blocks;
// every block is loaded once, cooperatively by the first 256 threads (each owns
// a fixed set of MFMA fragments of it), converted once into the bf16 operand
// planes the MFMAs take (an fp32 element as hi + lo, a bf16 element as is) and
// written to LDS in fragment order, so each wave reads its operands with one
// conflict-free 16-byte LDS read per fragment, and the loads of the next block
// are in flight while the current one is multiplied.
//   K fragment (kt, ds, lane): key k0 + 16 kt + lane % 16, dims 32 ds + 8 (lane / 16) .. +7
//   V fragment (dt, lane):     dim 16 dt + lane % 16 of the transposed V cache, keys
//                              k0 + 4 (lane / 16) + {0..3} and k0 + 16 + 4 (lane / 16) + {0..3}
// Blocks start at multiples of 32 keys and the cache capacity is a multiple of
// 32, so a block never reads past its head's rows; keys at or past the end of
// the range (unwritten rows) get zero values and -inf scores.
template <typename TKV> struct KVStage;
template <> struct KVStage<uint16_t> {
  static constexpr int HL = 1;
  struct Raw { uint4 u; };
  static __device__ __forceinline__ Raw krow(const uint16_t* p) { return Raw{*reinterpret_cast<const uint4*>(p)}; }
  static __device__ __forceinline__ Raw vpair(const uint16_t* p) {
    const uint2 v0 = *reinterpret_cast<const uint2*>(p);
    const uint2 v1 = *reinterpret_cast<const uint2*>(p + 16);
    return Raw{make_uint4(v0.x, v0.y, v1.x, v1.y)};
  }
  // zero the elements whose key (k + (e / 4) * 16 + e % 4) is >= kend
  static __device__ __forceinline__ void vmask(Raw& r, int k, int kend) {
    uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = k + (e >> 1) * 16 + 2 * (e & 1);
      const uint32_t lo = key < kend ? 0x0000ffffu : 0u, hi = key + 1 < kend ? 0xffff0000u : 0u;
      w[e] &= lo | hi;
    }
    r.u = make_uint4(w[0], w[1], w[2], w[3]);
  }
  static __device__ __forceinline__ void put(uint4* dst, const Raw& r) { dst[0] = r.u; }
};
template <> struct KVStage<float> {
  static constexpr int HL = 2;
  struct Raw { float4 a, b; };
  static __device__ __forceinline__ Raw krow(const float* p) {
    return Raw{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
  }
  static __device__ __forceinline__ Raw vpair(const float* p) {
    return Raw{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 16)};
  }
  static __device__ __forceinline__ void vmask(Raw& r, int k, int kend) {
    r.a.x = k + 0 < kend ? r.a.x : 0.f;
    r.a.y = k + 1 < kend ? r.a.y : 0.f;
    r.a.z = k + 2 < kend ? r.a.z : 0.f;
    r.a.w = k + 3 < kend ? r.a.w : 0.f;
    r.b.x = k + 16 < kend ? r.b.x : 0.f;
    r.b.y = k + 17 < kend ? r.b.y : 0.f;
    r.b.z = k + 18 < kend ? r.b.z : 0.f;
    r.b.w = k + 19 < kend ? r.b.w : 0.f;
  }
  // hi plane at dst[0], lo plane 64 fragments further
  static __device__ __forceinline__ void put(uint4* dst, const Raw& r) {
    const float x[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
    uint4 hi, lo;
    split8(x, hi, lo);
    dst[0] = hi;
    dst[64] = lo;
  }
};


constexpr int kAttnDepth = 2;      // 32-key blocks in flight per workgroup
constexpr int kAttnWaves = 8;      // waves per workgroup: all stage, the first ceil(R / 16) compute

template <int HD, typename TKV>
__global__ __launch_bounds__(64 * kAttnWaves) void attn_mfma_kernel(AttnArgs a) {
  constexpr int NW = kAttnWaves, DEPTH = kAttnDepth;
  using KV = KVStage<TKV>;
  using Raw = typename KV::Raw;
  constexpr int HL = KV::HL;
  constexpr int DS = HD / 32;                 // 32-wide d steps of the score MFMA
  constexpr int DT = HD / 16;                 // 16-wide d tiles of the output MFMA
  constexpr int KFR = 2 * DS * 64;            // K fragments per block
  constexpr int NFR = KFR + DT * 64;          // K + V fragments per block
  constexpr int BUF = NFR * HL;               // uint4 per LDS block buffer
  extern __shared__ uint4 stage[];            // [2][BUF]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g4 = lane >> 4;
  const int item = blockIdx.x;
  int b, j, sp;
  decode_item(a, item, b, j, sp);
  const int nk = a.nkeys[b];
  const int kbeg = sp * a.split_keys;
  const int kend = min(nk, kbeg + a.split_keys);
  const int r = blockIdx.y * kRowsPerGroup + wave * 16 + (lane & 15);
  const int G = a.Hq / a.Hkv;
  const bool computes = blockIdx.y * kRowsPerGroup + wave * 16 < a.R;   // uniform per wave

  uint4 qh[DS], ql[DS];                       // query fragments, loaded after the first key blocks
  const int64_t head = static_cast<int64_t>(b) * a.Hkv + j;
  const TKV* kbase = static_cast<const TKV*>(a.kc) + head * a.cap * HD;
  const TKV* vbase = static_cast<const TKV*>(a.vc) + head * HD * a.cap;

  // every thread stages fragments f = t + 64 NW i of each block; i < PER_K are K fragments
  constexpr int STG = 64 * NW;
  constexpr int PER = NFR / STG, PER_K = KFR / STG;
  static_assert(NFR % STG == 0, "fragment split");
  // K or V for fragment slot i: known at compile time when STG divides KFR
  auto is_k = [&](int i, int f) { return (KFR % STG == 0) ? (i < PER_K) : (f < KFR); };
  const int t = threadIdx.x;
  auto load = [&](Raw (&rr)[PER], int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int f = t + STG * i;
      const int ln = f & 63;
      if (is_k(i, f)) {
        const int kt = f / (DS * 64), ds = (f / 64) % DS;
        const int key = k0 + kt * 16 + (ln & 15);
        rr[i] = KV::krow(kbase + static_cast<int64_t>(key) * HD + ds * 32 + 8 * (ln >> 4));
      } else {
        const int dt = (f - KFR) / 64;
        const int k = k0 + 4 * (ln >> 4);
        rr[i] = KV::vpair(vbase + static_cast<int64_t>(dt * 16 + (ln & 15)) * a.cap + k);
      }
    }
  };
  auto store = [&](Raw (&rr)[PER], uint4* buf, int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int f = t + STG * i;
      const int ln = f & 63, fr = f >> 6;       // fragment index: kt*DS + ds, or KFR/64 + dt
      if (!is_k(i, f)) KV::vmask(rr[i], k0 + 4 * (ln >> 4), kend);
      KV::put(buf + (fr * HL) * 64 + ln, rr[i]);
    }
  };

  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  auto compute = [&](const uint4* buf, int k0, int klim) {   // keys >= klim do not count
    // all K fragments of the block first (independent LDS reads, one wait), then
    // the score MFMAs in four independent accumulation chains
    uint4 kf[2][DS][HL];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
#pragma unroll
        for (int hl = 0; hl < HL; ++hl) kf[kt][ds][hl] = buf[((kt * DS + ds) * HL + hl) * 64 + lane];
    __builtin_amdgcn_sched_barrier(0);
    f32x4_t sa[2], sb[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) { sa[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f}; sb[kt] = sa[kt]; }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        sa[kt] = mfma16x16x32(kf[kt][ds][0], qh[ds], sa[kt]);
        sb[kt] = mfma16x16x32(kf[kt][ds][0], ql[ds], sb[kt]);
        if constexpr (HL == 2) sb[kt] = mfma16x16x32(kf[kt][ds][1], qh[ds], sb[kt]);
      }
    // the value fragments are read now; their latency hides behind the softmax
    uint4 vf[DT][HL];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int hl = 0; hl < HL; ++hl) vf[dt][hl] = buf[((KFR / 64 + dt) * HL + hl) * 64 + lane];
    __builtin_amdgcn_sched_barrier(0);
    f32x4_t s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[kt] = sa[kt] + sb[kt];
    float p[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) p[kt * 4 + e] = (k0 + kt * 16 + 4 * g4 + e < klim) ? s[kt][e] : -INFINITY;
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
    if (__any(alpha != 1.0f)) {               // skipped once every row's max has settled
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    uint4 ph, pl;
    split8(p, ph, pl);
    // O^T += V^T P^T; k-slot e of lane group g4 <-> key k0 + 4*g4 + e (e < 4),
    // k0 + 16 + 4*g4 + (e - 4) (e >= 4): the layout S^T left in p[]
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      o[dt] = mfma16x16x32(vf[dt][0], ph, o[dt]);
      o[dt] = mfma16x16x32(vf[dt][0], pl, o[dt]);
      if constexpr (HL == 2) o[dt] = mfma16x16x32(vf[dt][1], ph, o[dt]);
    }
  };

  // DEPTH blocks in flight in registers (block i in set i % DEPTH) and two LDS
  // buffers (block i in buffer i % 2), one barrier per block: the buffer written
  // for block i was last read for block i - 2, before the previous barrier.
  // The loop has no data-dependent branch around a load, so that every step
  // issues and retires its loads in the same order (precise waits): it runs a
  // whole number of DEPTH steps, the steps past the last block re-stage the
  // last block (a cache hit) and count no key.
  const int nblk = (kend - kbeg + 31) / 32;   // >= 1: every key range is non-empty
  auto blk = [&](int i) { return kbeg + min(i, nblk - 1) * 32; };
  Raw rr[DEPTH][PER];
#pragma unroll
  for (int dd = 0; dd < DEPTH; ++dd) load(rr[dd], blk(dd));
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

  for (int bi = 0; bi < nblk; bi += DEPTH) {
#pragma unroll
    for (int dd = 0; dd < DEPTH; ++dd) {
      uint4* buf = stage + ((bi + dd) & 1) * BUF;
      const int k0 = blk(bi + dd);
      store(rr[dd], buf, k0);
      load(rr[dd], blk(bi + dd + DEPTH));
      __syncthreads();
      if (computes) compute(buf, k0, bi + dd < nblk ? kend : k0);
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);
  if (computes && r < a.Rpad) {
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
  const dim3 block(64 * kAttnWaves);
  // LDS: two block buffers of (2 DS + DT) * 64 fragments, two planes for fp32
  const size_t lds = static_cast<size_t>(2) * (a.d / 16 + a.d / 16) * 64 * (bf16_cache ? 1 : 2) * sizeof(uint4);
  auto kern = bf16_cache ? (a.d == 128 ? attn_mfma_kernel<128, uint16_t> : attn_mfma_kernel<64, uint16_t>)
                         : (a.d == 128 ? attn_mfma_kernel<128, float> : attn_mfma_kernel<64, float>);
  hipLaunchKernelGGL(kern, grid, block, lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (stop_event != nullptr) (void)hipEventRecord(static_cast<hipEvent_t>(stop_event), st);
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.B * a.gamma * a.Hq), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace dflash
