// Injected-context attention of the drafter block.
//
// For sequence b and KV head j, the G*gamma query rows of the block (all query
// heads of the group, all block rows) attend without a mask to every key of
// [context ; block] = cache rows [0, len_b + gamma) of that head ("DFlash:
// Block Diffusion for Flash Speculative Decoding 논문 정리", section "KV
// Injection 메커니즘"; bidirectional inside the block, section "추론 구조").
//
// gfx950 design: few query rows against a long key stream, so the kernels are
// HBM-bound and split over keys:
//   * one workgroup per (sequence, KV head, key range); one wave per 16 query
//     rows, all waves sharing the key range's K/V blocks through LDS;
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16;
//     the fp32 queries (pre-scaled by log2(e)/sqrt(d)) are split into bf16
//     hi + lo and multiplied twice;
//   * online softmax per row with exp2; the MFMA output layout of S^T (4 keys of
//     one row per lane) is the B-operand layout P^T of the value MFMA, so
//     probabilities never leave registers;
//   * O^T = V^T P^T reads values from the transposed V cache (keys contiguous:
//     [d][cap] per head in an fp32 cache, [cap/32][d][32] in a bf16 one), P
//     again split hi + lo; a bf16 cache also stores each 32-key block of K in
//     the order of the score MFMA's fragments, so every K or V fragment is one
//     contiguous kilobyte;
//   * each workgroup writes (max, sum, O) per row; a combine kernel merges the
//     key ranges in a fixed order (log-sum-exp), so results are deterministic.
// A bf16 cache streams K/V blocks straight into LDS (attn_dma_kernel); an fp32
// cache stages them through registers, splitting each element once into bf16
// hi + lo planes (attn_mfma_kernel, three MFMAs per product).  fp32 weights
// use a plain one-wave-per-(row, head) online-softmax kernel.
#include "common.h"
#include "kv_layout.h"
#include "launch.h"

#include <stdlib.h>

#include <algorithm>
#include <type_traits>

namespace dflash {
namespace {

constexpr int kRowsPerGroup = 128;   // query rows per workgroup (8 waves)

// Sequence of packed block row m (qrow0[b] <= m < qrow0[b + 1]).
__device__ __forceinline__ int row_seq(const AttnArgs& a, int m) {
  int b = 0;
  while (b + 1 < a.B && m >= a.qrow0[b + 1]) ++b;
  return b;
}

// Key rows [kbeg, kend) of item (b, sp) in the cache of sequence kvseq[b]: a
// range of the context rows [0, nkeys[b]), or, for the last item of a block
// whose own rows are stored apart (blk0[b] >= 0), those gam[b] rows.
__device__ __forceinline__ void item_keys(const AttnArgs& a, int b, int sp, int& kbeg, int& kend) {
  if (a.blk0[b] >= 0 && sp == a.nsplit[b] - 1) {
    kbeg = a.blk0[b];
    kend = kbeg + a.gam[b];
  } else {
    kbeg = sp * a.split_keys;
    kend = min(a.nkeys[b], kbeg + a.split_keys);
  }
}

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
  int kbeg, kend;
  item_keys(a, b, sp, kbeg, kend);
  const int r = blockIdx.y * kRowsPerGroup + wave * 16 + (lane & 15);
  const int G = a.Hq / a.Hkv;
  const int gb = a.gam[b], Rb = G * gb;       // this sequence's block rows and query rows
  const bool computes = blockIdx.y * kRowsPerGroup + wave * 16 < Rb;   // uniform per wave
  // The keys this lane's query row sees within [kbeg, kend): all of them,
  // except in a group of two anchored blocks, where the rows of each block see
  // only their own context prefix and their own block rows.
  int klo = kbeg, khi = kend;
  if (a.causal) khi = min(khi, a.nkeys[b] - gb + r % gb + 1);   // keys up to this row's own
  if (a.blk0[b] >= 0) {
    const bool second = r % gb >= a.half[b];
    if (sp == a.nsplit[b] - 1) {
      klo = kbeg + (second ? a.half[b] : 0);
      khi = kbeg + (second ? gb : a.half[b]);
    } else {
      khi = min(kend, second ? a.ctx2[b] : a.ctx1[b]);
    }
  }

  uint4 qh[DS], ql[DS];                       // query fragments, loaded after the first key blocks
  const int64_t head = static_cast<int64_t>(a.kvseq[b]) * a.Hkv + j;
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

  auto compute = [&](const uint4* buf, int k0, int lo, int hi) {   // only keys in [lo, hi) count (per lane)
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
      for (int e = 0; e < 4; ++e) {
        const int key = k0 + kt * 16 + 4 * g4 + e;
        p[kt * 4 + e] = (key >= lo && key < hi) ? s[kt][e] : -INFINITY;
      }
    float mx = p[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, p[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;   // a row with no key yet: nothing to scale
    const float alpha = exp2f(m_run - m_use);
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = exp2f(p[e] - m_use);
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
  if (r < Rb) {
    const int h = j * G + r / gb, i = r % gb;
    const float* qp = a.q + (static_cast<int64_t>(a.qrow0[b] + i) * a.Hq + h) * HD + 8 * g4;
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
      const bool live = bi + dd < nblk;
      if (computes) compute(buf, k0, live ? klo : k0, live ? khi : k0);
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

// ----------------------------------------------------------- bf16 cache path
// K and V blocks go straight from HBM to LDS through gfx950's global-to-LDS
// loads (lane l of a wave-wide 16-byte load lands at LDS base + 16 l): no
// register staging, no conversion, and the stages in flight cost no
// registers.  Inside a 32-key block the score tile kt takes keys in the order
// row i -> key 8 (i / 4) + 4 kt + i % 4 (the cache stores the block's K in
// exactly these fragments, kt-major then 32-dimension slice, lane l's 16 bytes
// at 16 l, see k_frag_offset), so the S^T output leaves lane l (lane
// group g = l / 16) holding keys 8 g + 4 kt + r of its query column; as the B
// operand of the value MFMA, k-slot 8 g + e is then key 8 g + e, and the value
// fragment of lane l is 8 consecutive keys of one row of the block's V^T
// (one 16-byte load, like a K fragment).  With G * gamma <= 64 query rows the
// eight waves form two groups of four that take alternate blocks, each with its
// own online-softmax state, merged through LDS at the end (two waves per SIMD
// overlap one another's MFMA, softmax and LDS latency); with more rows one
// group of eight waves takes every block.
constexpr int kDmaStages = 3;   // LDS stages (one block per group each), two in flight

template <int HD, int NG>
__global__ __launch_bounds__(512) void attn_dma_kernel(AttnArgs a) {
  constexpr int NW = 8, WPG = NW / NG, NST = kDmaStages;
  constexpr int DS = HD / 32, DT = HD / 16;
  constexpr int KFR = 2 * DS, NFR = KFR + DT;   // K and V fragments of a block
  constexpr int LPW = NG * NFR / NW;            // loads per wave per stage
  static_assert((NG * NFR) % NW == 0, "fragments split evenly over the waves");
  extern __shared__ uint4 stage[];              // [NST][NG][NFR][64]
  const int lane = threadIdx.x & 63, g4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave / WPG, wq = wave % WPG;
  int b, j, sp;
  decode_item(a, blockIdx.x, b, j, sp);
  int kbeg, kend;
  item_keys(a, b, sp, kbeg, kend);
  const int nblk = (kend - kbeg + 31) / 32;     // >= 1: every key range is non-empty
  const int nstep = (nblk + NG - 1) / NG;
  const int row0 = blockIdx.y * 16 * WPG + wq * 16;
  const int r = row0 + (lane & 15);
  const int G = a.Hq / a.Hkv;
  const int gb = a.gam[b], Rb = G * gb;         // this sequence's block rows and query rows
  const bool computes = row0 < Rb;              // uniform per wave
  // causal pass: keys from ctail on are block rows, and this lane's row sees
  // them up to its own (kcaus = one past it)
  const int ctail = a.causal ? a.nkeys[b] - gb : INT_MAX;
  const int kcaus = a.causal ? ctail + r % gb + 1 : INT_MAX;
  const int64_t head = static_cast<int64_t>(a.kvseq[b]) * a.Hkv + j;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.kc) + head * a.cap * HD;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.vc) + head * HD * a.cap;
  const unsigned lds0 = lds_addr(stage);

  // byte offset of this lane's 16 bytes from its block's first key, for each
  // fragment F = wave + NW i this wave loads (group F / NFR, fragment F % NFR)
  uint32_t off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int f = (wave + NW * i) % NFR;
    if (f < KFR) {                              // K block in fragment order: one kilobyte per fragment
      off[i] = 2u * static_cast<uint32_t>(f * 512 + lane * 8);
    } else {                                    // V^T block [d][32]: dimension row, 8 keys
      off[i] = 2u * static_cast<uint32_t>(((f - KFR) * 16 + (lane & 15)) * 32 + 8 * g4);
    }
  }
  // step u loads blocks NG u .. NG u + NG - 1 into stage st; past the last
  // block it repeats the last one (so every wait has a fixed count)
  auto issue = [&](int u, int st) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int F = wave + NW * i, f = F % NFR;
      const int k0 = kbeg + min(NG * u + F / NFR, nblk - 1) * 32;
      const uint16_t* base = f < KFR ? kbase + static_cast<int64_t>(k0) * HD : vbase + static_cast<int64_t>(k0) * HD;
      load_to_lds_sbase(off[i], base, lds0 + static_cast<unsigned>((st * NG * NFR + F) * 1024));
    }
  };

  uint4 qh[DS], ql[DS];
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  auto compute = [&](const uint4* buf, int k0) {
    uint4 kf[2][DS];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) kf[kt][ds] = buf[(kt * DS + ds) * 64 + lane];
    __builtin_amdgcn_sched_barrier(0);
    f32x4_t sc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) sc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        sc[kt] = mfma16x16x32(kf[kt][ds], qh[ds], sc[kt]);
        sc[kt] = mfma16x16x32(kf[kt][ds], ql[ds], sc[kt]);
      }
    uint4 vf[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vf[dt] = buf[(KFR + dt) * 64 + lane];
    __builtin_amdgcn_sched_barrier(0);
    float p[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) p[kt * 4 + e] = sc[kt][e];
    const bool partial = k0 + 32 > kend;        // uniform: the last block of the range
    const bool crows = k0 + 32 > ctail;         // uniform: the block holds block rows of a causal pass
    if (partial || crows) {
      const int klim = min(kend, kcaus);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (k0 + 8 * g4 + 4 * kt + e >= klim) p[kt * 4 + e] = -INFINITY;
    }
    float mx = p[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, p[e]);
    // finite unless a causal row has seen no key yet (then nothing to scale)
    const float m_new = fmaxf(m_run, max_across16(mx));
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = __builtin_amdgcn_exp2f(p[e] - m_use);
      ps += p[e];
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
    if (__any(alpha != 1.0f)) {                 // skipped once every row's max has settled
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    if (partial) {                              // unwritten rows past the range: zero values
      const int nv = kend - (k0 + 8 * g4);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        uint32_t w[4] = {vf[dt].x, vf[dt].y, vf[dt].z, vf[dt].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] &= (2 * e < nv ? 0x0000ffffu : 0u) | (2 * e + 1 < nv ? 0xffff0000u : 0u);
        vf[dt] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    uint4 ph, pl;
    split8(p, ph, pl);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      o[dt] = mfma16x16x32(vf[dt], ph, o[dt]);
      o[dt] = mfma16x16x32(vf[dt], pl, o[dt]);
    }
  };

#pragma unroll
  for (int st = 0; st < NST - 1; ++st) issue(st, st);
  if (computes && r < Rb) {
    const int h = j * G + r / gb, i = r % gb;
    const float* qp = a.q + (static_cast<int64_t>(a.qrow0[b] + i) * a.Hq + h) * HD + 8 * g4;
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
  for (int u = 0; u < nstep; ++u) {
    wait_vmcnt<(NST - 2) * LPW>();              // this wave's loads of step u landed
    bare_barrier();                             // ... and every other wave's; step u - 1 is consumed
    issue(u + NST - 1, (u + NST - 1) % NST);
    const int t = NG * u + grp;
    if (computes && t < nblk) compute(stage + ((u % NST) * NG + grp) * NFR * 64, kbeg + t * 32);
  }
  wait_vmcnt<0>();                              // the trailing repeated blocks

  float l_tot = sum_across16(l_run);
  if constexpr (NG == 2) {
    // group 1 hands (m, l, O) to group 0 through LDS; a group that saw no block
    // has m = -inf, l = 0, O = 0 and weight 0
    __syncthreads();
    float* mo = reinterpret_cast<float*>(stage);   // [WPG][DT][64][4]
    float* mml = mo + WPG * DT * 64 * 4;           // [WPG][64][2]
    if (grp == 1 && computes) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<float4*>(mo + ((wq * DT + dt) * 64 + lane) * 4) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
      mml[(wq * 64 + lane) * 2] = m_run;
      mml[(wq * 64 + lane) * 2 + 1] = l_tot;
    }
    __syncthreads();
    if (grp == 1 || !computes) return;
    const float m1 = mml[(wq * 64 + lane) * 2], l1 = mml[(wq * 64 + lane) * 2 + 1];
    const float M = fmaxf(m_run, m1);
    const float M_use = M == -INFINITY ? 0.f : M;   // neither group saw a key (a causal row): weights 0
    const float w0 = __builtin_amdgcn_exp2f(m_run - M_use), w1 = __builtin_amdgcn_exp2f(m1 - M_use);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const float4 x = *reinterpret_cast<const float4*>(mo + ((wq * DT + dt) * 64 + lane) * 4);
      o[dt][0] = o[dt][0] * w0 + x.x * w1;
      o[dt][1] = o[dt][1] * w0 + x.y * w1;
      o[dt][2] = o[dt][2] * w0 + x.z * w1;
      o[dt][3] = o[dt][3] * w0 + x.w * w1;
    }
    l_tot = l_tot * w0 + l1 * w1;
    m_run = M;
  }
  if (computes && r < a.Rpad) {
    float* po = a.part_o + (static_cast<int64_t>(blockIdx.x) * a.Rpad + r) * HD + 4 * g4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(po + dt * 16) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (g4 == 0) {
      float* pm = a.part_ml + (static_cast<int64_t>(blockIdx.x) * a.Rpad + r) * 2;
      pm[0] = m_run;
      pm[1] = l_tot;
    }
  }
}

template <int HD, int NG>
size_t attn_dma_lds() {
  constexpr int DT = HD / 16, NFR = 2 * (HD / 32) + DT, WPG = 8 / NG;
  const size_t stages = static_cast<size_t>(kDmaStages) * NG * NFR * 64 * sizeof(uint4);
  const size_t merge = NG == 2 ? static_cast<size_t>(WPG) * DT * 64 * 16 + static_cast<size_t>(WPG) * 64 * 8 : 0;
  return stages > merge ? stages : merge;
}

template <int HD, int NG>
hipError_t launch_dma(const AttnArgs& a, const AttnPlan& p, hipStream_t st) {
  const size_t lds = attn_dma_lds<HD, NG>();
  const hipError_t e = ensure_dyn_lds(reinterpret_cast<const void*>(attn_dma_kernel<HD, NG>), static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const int rows = 16 * 8 / NG;   // query rows per workgroup
  launch_k(attn_dma_kernel<HD, NG>, dim3(p.items, (a.R + rows - 1) / rows), dim3(512), lds, st, a);
  return hipGetLastError();
}

// Merge the key ranges of one (row, head): O = sum_s 2^(m_s-M) O_s / sum_s 2^(m_s-M) l_s.
// The split weights are computed once per row into LDS. The O loads of all
// splits are independent of them and, for up to 32 splits, are in flight
// together with the (m, l) loads, so the merge waits on one memory round.
constexpr int kMaxSplitsLds = 1024;

__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  __shared__ float wts[kMaxSplitsLds];
  __shared__ float inv_l;
  const int idx = blockIdx.x;
  const int m = idx / a.Hq, h = idx % a.Hq;
  const int b = row_seq(a, m), i = m - a.qrow0[b];
  const int G = a.Hq / a.Hkv, j = h / G;
  const int r = (h - j * G) * a.gam[b] + i;
  const int ns = a.nsplit[b];
  const int it0 = a.item_off[b] + j * ns;
  // up to kCombRegs splits: each thread's O partials (one column, d <= block) are
  // requested at entry, beside wave 0's (m, l) loads, instead of after the
  // barrier; the sums below keep the split order either way
  constexpr int kCombRegs = 32;
  const bool in_regs = ns <= kCombRegs && a.d <= static_cast<int>(blockDim.x);  // uniform
  const int c0 = threadIdx.x;
  float ov[kCombRegs];
  if (in_regs && c0 < a.d) {
#pragma unroll
    for (int s = 0; s < kCombRegs; ++s)
      ov[s] = s < ns ? a.part_o[(static_cast<int64_t>(it0 + s) * a.Rpad + r) * a.d + c0] : 0.f;
  }
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
  if (in_regs) {
    if (c0 < a.d) {
      float O = 0.f;
#pragma unroll
      for (int s = 0; s < kCombRegs; ++s)
        if (s < ns) O += wts[s] * ov[s];
      const int64_t oi = (static_cast<int64_t>(m) * a.Hq + h) * a.d + c0;
      if (a.o_hi != nullptr) split1(O * inv_l, a.o_hi[oi], a.o_lo[oi]);
      else a.o_out[oi] = O * inv_l;
    }
    return;
  }
  for (int c = threadIdx.x; c < a.d; c += blockDim.x) {
    float O = 0.f;
#pragma unroll 8
    for (int s = 0; s < ns; ++s) O += wts[s] * a.part_o[(static_cast<int64_t>(it0 + s) * a.Rpad + r) * a.d + c];
    const int64_t oi = (static_cast<int64_t>(m) * a.Hq + h) * a.d + c;
    if (a.o_hi != nullptr) split1(O * inv_l, a.o_hi[oi], a.o_lo[oi]);
    else a.o_out[oi] = O * inv_l;
  }
}

// The same merge with one wave per (row, head), four per workgroup, for large
// batches of rows: lane e holds the weight of split c0 + e of the current
// chunk of 64 and every lane accumulates its columns of O (two at d = 128),
// the weight broadcast from lane e.  Same split order as the kernel above.
// Measured on 64 anchored blocks (32768 (row, head) pairs) 62 -> 43 us per
// layer, but slower at the bench shape (512 pairs, 17 splits: 4.8 -> 9.6 us),
// so the launcher takes it from kCombineWaveMin pairs.
constexpr int kCombineWaves = 4;
constexpr int kCombineWaveMin = 4096;

__global__ __launch_bounds__(64 * kCombineWaves) void attn_combine_wave_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
  if (idx >= a.qrow0[a.B] * a.Hq) return;     // uniform per wave; no barrier follows
  const int m = idx / a.Hq, h = idx % a.Hq;
  const int b = row_seq(a, m), i = m - a.qrow0[b];
  const int G = a.Hq / a.Hkv, j = h / G;
  const int r = (h - j * G) * a.gam[b] + i;
  const int ns = a.nsplit[b];
  const int it0 = a.item_off[b] + j * ns;
  auto ml_of = [&](int s) {
    return *reinterpret_cast<const float2*>(a.part_ml + (static_cast<int64_t>(it0 + s) * a.Rpad + r) * 2);
  };
  float M = -INFINITY;
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, ml_of(s).x);
  M = wave_max(M);
  const bool two = a.d == 128;                // columns per lane: 2 (d = 128) or 1 (d = 64)
  const int c = two ? 2 * lane : lane;
  float o0 = 0.f, o1 = 0.f, L = 0.f;
  for (int c0 = 0; c0 < ns; c0 += 64) {
    float w = 0.f;
    if (c0 + lane < ns) {
      const float2 v = ml_of(c0 + lane);
      w = exp2f(v.x - M);
      L += w * v.y;
    }
    const int cn = min(64, ns - c0);
    const float* po = a.part_o + (static_cast<int64_t>(it0 + c0) * a.Rpad + r) * a.d + c;
    const int64_t stride = static_cast<int64_t>(a.Rpad) * a.d;   // between consecutive splits
    for (int e = 0; e < cn; ++e) {
      const float we = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), e));
      if (two) {
        const float2 x = *reinterpret_cast<const float2*>(po + e * stride);
        o0 += we * x.x;
        o1 += we * x.y;
      } else {
        o0 += we * po[e * stride];
      }
    }
  }
  const float inv_l = 1.0f / wave_sum(L);
  const int64_t oi = (static_cast<int64_t>(m) * a.Hq + h) * a.d + c;
  if (a.o_hi != nullptr) {
    split1(o0 * inv_l, a.o_hi[oi], a.o_lo[oi]);
    if (two) split1(o1 * inv_l, a.o_hi[oi + 1], a.o_lo[oi + 1]);
  } else if (two) {
    *reinterpret_cast<float2*>(a.o_out + oi) = make_float2(o0 * inv_l, o1 * inv_l);
  } else {
    a.o_out[oi] = o0 * inv_l;
  }
}

// fp32 storage: one wave per (block row, query head), keys walked in order.
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  const int idx = blockIdx.x, lane = threadIdx.x;
  const int m = idx / a.Hq, h = idx % a.Hq;
  const int b = row_seq(a, m);
  const int G = a.Hq / a.Hkv, j = h / G;
  const float* qp = a.q + (static_cast<int64_t>(m) * a.Hq + h) * a.d;
  const float q0 = lane < a.d ? qp[lane] * a.scale_log2 : 0.f;
  const float q1 = lane + 64 < a.d ? qp[lane + 64] * a.scale_log2 : 0.f;
  const int64_t head = static_cast<int64_t>(a.kvseq[b]) * a.Hkv + j;
  const float* kb = static_cast<const float*>(a.kc) + head * a.cap * a.d;
  const float* vb = static_cast<const float*>(a.vc) + head * a.d * a.cap;
  float m_run = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  const int nctx = a.nkeys[b];
  // a causal pass stops at this row's own key (block rows follow the context)
  const int nall = a.causal ? nctx - a.gam[b] + (m - a.qrow0[b]) + 1 : nctx + (a.blk0[b] >= 0 ? a.gam[b] : 0);
  for (int tt = 0; tt < nall; ++tt) {
    const int t = tt < nctx ? tt : a.blk0[b] + (tt - nctx);   // the block's own rows when stored apart
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

// Work items (key ranges) per launch: about one per CU.  Each workgroup fills
// most of a CU (eight waves; the bf16 path's stages take 96 KB of LDS), and
// fewer, longer key ranges spend less on each range's start-up and on the
// combine step.  The workspace bound allows up to kAttnItemMax.
constexpr int kAttnItemMax = 1024;

static int attn_item_target() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  const int t = env_int("DFLASH_ATTN_ITEMS", n);
  return t < kAttnItemMax ? t : kAttnItemMax;
}

AttnPlan plan_attention(int B, const int32_t* nkeys, int Hkv, int R, int d, const int32_t* apart) {
  AttnPlan p;
  int64_t total = 0;
  for (int b = 0; b < B; ++b) total += nkeys[b];
  const int target = attn_item_target();
  const int min_keys = env_int("DFLASH_ATTN_MIN_KEYS", 128);
  int64_t sk = (total * Hkv + target - 1) / target;
  sk = ((sk + 31) / 32) * 32;
  if (sk < min_keys) sk = ((min_keys + 31) / 32) * 32;
  int maxk = 0;
  for (int b = 0; b < B; ++b) maxk = nkeys[b] > maxk ? nkeys[b] : maxk;
  // the combine's LDS table holds kMaxSplitsLds splits: at most kMaxSplitsLds - 1
  // context ranges, leaving room for a block stored apart
  const int64_t sk_min = ((maxk + kMaxSplitsLds - 2) / (kMaxSplitsLds - 1) + 31) / 32 * 32;
  if (sk < sk_min) sk = sk_min;
  // Many sequences: rounding each sequence's key count up to whole ranges can
  // leave a few more items than CUs, and the CUs that take two items set the
  // time (16 sequences of 1024-4096 keys: 312 items of <= 1280 keys, 135 us
  // per layer, against ~100 us with 500-800 shorter items).  So the range
  // length is the one of least ceil(items / CUs) * (longest item + 32 keys of
  // start-up), searched in 32-key steps down to a quarter of the
  // one-range-per-CU length (at most ~256 candidates); ties keep the longer
  // ranges (fewer items, a cheaper combine).  A single long sequence keeps one
  // range per CU.
  if (getenv("DFLASH_ATTN_ITEMS") == nullptr) {
    const int cus = attn_item_target();
    const int64_t lo_keys = std::max<int64_t>(std::max<int64_t>((min_keys + 31) / 32 * 32, sk_min), (sk / 4 + 31) / 32 * 32);
    const int64_t max_items = kAttnItemMax + 2 * static_cast<int64_t>(B) * Hkv;   // workspace bound
    auto items_of = [&](int64_t k) {
      int64_t n = 0;
      for (int b = 0; b < B; ++b) n += ((nkeys[b] + k - 1) / k + (apart != nullptr && apart[b] ? 1 : 0)) * Hkv;
      return n;
    };
    int64_t best_sk = sk, best_cost = -1;
    const int64_t step = std::max<int64_t>(32, (sk - lo_keys) / 256 / 32 * 32);   // at most ~256 candidates
    for (int64_t k = sk; k >= lo_keys; k -= step) {
      const int64_t n = items_of(k);
      if (n > max_items) continue;
      const int64_t cost = (n + cus - 1) / cus * (std::min<int64_t>(k, std::max(maxk, 1)) + 32);
      if (best_cost < 0 || cost < best_cost) best_cost = cost, best_sk = k;
    }
    sk = best_sk;
  }
  p.split_keys = static_cast<int>(sk);
  p.item_off[0] = 0;
  for (int b = 0; b < B; ++b) {
    p.nsplit[b] = static_cast<int>((nkeys[b] + sk - 1) / sk) + (apart != nullptr && apart[b] ? 1 : 0);
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
  // rounding up every (sequence, head)'s split count, plus one item per
  // (sequence, head) for a block stored apart
  const size_t items = static_cast<size_t>(kAttnItemMax) + 2 * static_cast<size_t>(B) * Hkv;
  return items * rpad * (d + 2);
}

hipError_t launch_attention(const AttnArgs& a0, const AttnPlan& p, bool bf16_weights, bool bf16_cache,
                            hipStream_t st) {
  AttnArgs a = a0;
  if (!bf16_weights) {
    launch_k(attn_f32_kernel, dim3(a.qrow0[a.B] * a.Hq), dim3(64), 0, st, a);
    return hipGetLastError();
  }
  a.split_keys = p.split_keys;
  a.items = p.items;
  a.Rpad = p.Rpad;
  for (int b = 0; b < a.B; ++b) { a.nsplit[b] = p.nsplit[b]; a.item_off[b] = p.item_off[b]; }
  a.item_off[a.B] = p.item_off[a.B];
  hipError_t e;
  if (bf16_cache) {
    // the DMA kernel's per-lane byte offsets into one head's K or V are 32-bit
    // (the entry points reject such caches before any launch)
    if (static_cast<int64_t>(a.cap) * a.d * 2 >= (int64_t{1} << 32)) return hipErrorInvalidValue;
    // V is read in whole blocks of 32 keys ([cap / 32][d][32] per head): every
    // key range starts on a block (context ranges at multiples of split_keys,
    // an anchored block's own rows in a 32-aligned slot)
    if (a.split_keys % 32 != 0 || a.cap % 32 != 0) return hipErrorInvalidValue;
    for (int b = 0; b < a.B; ++b)
      if (a.blk0[b] >= 0 && a.blk0[b] % 32 != 0) return hipErrorInvalidValue;
    const bool two = a.R <= 64;
    e = a.d == 128 ? (two ? launch_dma<128, 2>(a, p, st) : launch_dma<128, 1>(a, p, st))
                   : (two ? launch_dma<64, 2>(a, p, st) : launch_dma<64, 1>(a, p, st));
  } else {
    // LDS: two block buffers of (2 DS + DT) * 64 fragments, hi and lo planes
    const size_t lds = static_cast<size_t>(2) * (a.d / 16 + a.d / 16) * 64 * 2 * sizeof(uint4);
    auto kern = a.d == 128 ? attn_mfma_kernel<128, float> : attn_mfma_kernel<64, float>;
    launch_k(kern, dim3(p.items, p.row_groups), dim3(64 * kAttnWaves), lds, st, a);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  const int pairs = a.qrow0[a.B] * a.Hq;      // (row, head) pairs to merge
  if (pairs >= kCombineWaveMin)
    hipLaunchKernelGGL(attn_combine_wave_kernel, dim3((pairs + kCombineWaves - 1) / kCombineWaves),
                       dim3(64 * kCombineWaves), 0, st, a);
  else
    hipLaunchKernelGGL(attn_combine_kernel, dim3(pairs), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace dflash
