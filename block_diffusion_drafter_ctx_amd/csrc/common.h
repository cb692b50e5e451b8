// Device-side helpers shared by the gfx950 kernels of the DFlash drafter path:
// bf16 storage conversions, the 16x16x32 bf16 MFMA wrapper, fp32 -> (hi, lo)
// bf16 splitting and wave-level reductions.  gfx950 only (64-wide waves).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 storage
__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round to nearest even (gfx950's v_cvt_pk_bf16_f32 in the default rounding mode).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats -> packed bf16 pair (a in the low half), one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

// Storage-type traits: bf16 is held as uint16_t bit patterns.
template <typename T> struct Store;
template <> struct Store<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void st(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};
template <> struct Store<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};

// Pack 8 floats as bf16 (hi) and the bf16 of the remainder (lo): x ~= hi + lo
// with |x - hi - lo| <= 2^-16 |x| (so an MFMA pair on (hi, lo) keeps ~16
// significant bits of an fp32 activation against exact bf16 weights).
__device__ __forceinline__ void split8(const float* x, uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    const float h0 = __uint_as_float(h[i] << 16), h1 = __uint_as_float(h[i] & 0xffff0000u);
    l[i] = pack_bf16x2(x[2 * i] - h0, x[2 * i + 1] - h1);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// The same split for 4 values (two packed pairs each) and for one value.
__device__ __forceinline__ void split4(const float4& x, uint2& hi, uint2& lo) {
  const uint32_t h0 = pack_bf16x2(x.x, x.y), h1 = pack_bf16x2(x.z, x.w);
  hi = make_uint2(h0, h1);
  lo = make_uint2(pack_bf16x2(x.x - __uint_as_float(h0 << 16), x.y - __uint_as_float(h0 & 0xffff0000u)),
                  pack_bf16x2(x.z - __uint_as_float(h1 << 16), x.w - __uint_as_float(h1 & 0xffff0000u)));
}
__device__ __forceinline__ void split1(float x, uint16_t& hi, uint16_t& lo) {
  const uint32_t h = pack_bf16x2(x, 0.f);
  hi = static_cast<uint16_t>(h & 0xffffu);
  lo = static_cast<uint16_t>(pack_bf16x2(x - __uint_as_float(h << 16), 0.f) & 0xffffu);
}

// D += A (16 rows x 32 k) * B (32 k x 16 cols).  Lane l supplies A row (l % 16)
// and B column (l % 16), k-slots 8*(l/16)..+7 of each; D lane l holds rows
// 4*(l/16)+r, column l%16 (r = 0..3).  The k-slot -> k map only has to agree
// between A and B.
__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ------------------------------------------------------- global-to-LDS loads
// gfx950's wave-wide 16-byte global-to-LDS load lands lane l's 16 bytes at LDS
// address M0 + 16 l, with no register staging.  Both forms are issued as inline
// assembly so that the compiler does not treat every later LDS read as
// depending on them (it would wait for all loads in flight); kernels wait on
// exact counts with wait_vmcnt.
typedef __attribute__((address_space(3))) void lds_void;


__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(static_cast<unsigned>(reinterpret_cast<uintptr_t>((const lds_void*)p)));
}

// M0 is declared as an output of the statement (written by its s_mov, read by
// the load when it issues) rather than as a clobber: the compiler then knows
// the statement overwrites it.  The load itself writes no register.

// lane l reads src (its own address) into LDS lds_frag + 16 l (lds_frag wave-uniform)
__device__ __forceinline__ void load_frag_to_lds(const void* src, uint4* lds_frag) {
  const unsigned la = lds_addr(lds_frag);
  unsigned m0_set;
  asm volatile("s_mov_b32 %0, %2\n\tglobal_load_lds_dwordx4 %1, off" : "={m0}"(m0_set) : "v"(src), "s"(la) : "memory");
}

// lane l reads base + voff (base wave-uniform, in scalar registers; voff a byte
// offset) into LDS byte address m0 + 16 l
__device__ __forceinline__ void load_to_lds_sbase(uint32_t voff, const void* base, unsigned m0) {
  unsigned m0_set;
  asm volatile("s_mov_b32 %0, %3\n\tglobal_load_lds_dwordx4 %1, %2" : "={m0}"(m0_set) : "v"(voff), "s"(base), "s"(m0)
               : "memory");
}

// s_waitcnt with vmcnt = n (the other counters at their maximum): gfx9 encoding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// A workgroup barrier that waits for nothing else: the empty asm statements
// keep the compiler from moving LDS accesses across it, and unlike
// __syncthreads it does not wait for global-to-LDS loads still in flight.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------- lane-group reductions
// max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (gfx950 lane swaps:
// permlane32_swap pairs lane l with l ^ 32, permlane16_swap pairs l with l ^ 16)
__device__ __forceinline__ float max_across16(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_across16(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Sum over a workgroup of up to 1024 threads; `red` holds >= 16 floats of LDS.
// Every thread returns the total.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];   // fixed order: deterministic
  return t;
}

// Top-2 candidate (value, index) with "larger value, then lower index" order.
struct Top2 {
  float v1;
  int i1;
  float v2;
};

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__device__ __forceinline__ Top2 top2_merge(Top2 a, Top2 b) {
  Top2 r;
  if (better(b.v1, b.i1, a.v1, a.i1)) {
    r.v1 = b.v1; r.i1 = b.i1; r.v2 = fmaxf(a.v1, b.v2);
  } else {
    r.v1 = a.v1; r.i1 = a.i1; r.v2 = fmaxf(a.v2, b.v1);
  }
  return r;
}

__device__ __forceinline__ Top2 top2_push(Top2 a, float v, int i) {
  Top2 b{v, i, -INFINITY};
  return top2_merge(a, b);
}

__device__ __forceinline__ Top2 top2_shfl_xor(Top2 a, int m) {
  Top2 b;
  b.v1 = __shfl_xor(a.v1, m, kWave);
  b.i1 = __shfl_xor(a.i1, m, kWave);
  b.v2 = __shfl_xor(a.v2, m, kWave);
  return b;
}

// Temperature sampling statistics of (a piece of) one logits row: the best
// Gumbel-perturbed key with its index ("larger key, then lower index"), and the
// running log-sum-exp state of x = logit / T as (mx, se) with
// sum exp(x) = se * exp(mx).  An empty piece is {-inf, INT_MAX, -inf, 0}.
struct SampleStat {
  float key;
  int idx;
  float mx;
  float se;
};

__device__ __forceinline__ SampleStat sstat_empty() { return SampleStat{-INFINITY, 0x7fffffff, -INFINITY, 0.f}; }

// exp and log through the hardware base-2 units (v_exp_f32 / v_log_f32, about
// one ulp, plus the rounding of the change of base): the sampling kernels'
// per-element work, where the library functions' extra instructions would make
// the large-batch passes ALU-bound.
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.693147180559945309f;
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float fast_log(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

// A standard Gumbel variate from a uniform u in (0, 1).
__device__ __forceinline__ float gumbel_noise(float u) { return -fast_log(-fast_log(u)); }

__device__ __forceinline__ void sstat_push_lse(SampleStat& s, float x) {
  if (x > s.mx) {
    s.se = s.se * fast_exp(s.mx - x) + 1.f;
    s.mx = x;
  } else {
    s.se += fast_exp(x - s.mx);
  }
}

__device__ __forceinline__ void sstat_push_key(SampleStat& s, float key, int i) {
  if (better(key, i, s.key, s.idx)) {
    s.key = key;
    s.idx = i;
  }
}

__device__ __forceinline__ SampleStat sstat_merge(SampleStat a, SampleStat b) {
  SampleStat r;
  const bool bk = better(b.key, b.idx, a.key, a.idx);
  r.key = bk ? b.key : a.key;
  r.idx = bk ? b.idx : a.idx;
  r.mx = fmaxf(a.mx, b.mx);
  r.se = r.mx == -INFINITY ? 0.f : a.se * fast_exp(a.mx - r.mx) + b.se * fast_exp(b.mx - r.mx);
  return r;
}

__device__ __forceinline__ SampleStat sstat_shfl_xor(SampleStat a, int m) {
  SampleStat b;
  b.key = __shfl_xor(a.key, m, kWave);
  b.idx = __shfl_xor(a.idx, m, kWave);
  b.mx = __shfl_xor(a.mx, m, kWave);
  b.se = __shfl_xor(a.se, m, kWave);
  return b;
}

__device__ __forceinline__ float4 sstat_pack(SampleStat s) {
  return make_float4(s.key, __int_as_float(s.idx), s.mx, s.se);
}

__device__ __forceinline__ SampleStat sstat_unpack(float4 v) {
  return SampleStat{v.x, __float_as_int(v.y), v.z, v.w};
}

}  // namespace dflash
