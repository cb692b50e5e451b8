// Split-K reductions fused with each GEMM's consumer step, plus the small
// row-wise kernels of the drafter path:
//   ctx_norm       fusion epilogue: sum partials, RMSNorm with g_c, store H_t
//   scatter_kv     sum partials; query columns -> fp32 Q; key / value columns ->
//                  the KV cache (keys row-major, values transposed; a bf16
//                  cache keeps both per block of 32 keys, keys in fragment order)
//   residual_norm  h += sum partials; a = RMSNorm(h; g)
//   swiglu         s = SiLU(gate) * up
//   embed_norm     h = embedding rows (or override rows); a = RMSNorm(h; g)
//   argmax_final   merge per-tile top-2 into draft ids and top-2 gaps
//   argmax_rows    same from plain fp32 logits rows (fp32 storage path)
//   accept         greedy acceptance length and next anchor (one wave per sequence)
//   gather_rows    a ragged batch's mask rows into one dense block for the LM head
//   accept_ragged  acceptance with a draft count per sequence
// Every reduction sums partials in split order: results are bit-reproducible.
#include "common.h"
#include "kv_layout.h"
#include "launch.h"

namespace dflash {
namespace {

// Threads per row kernel: one float4 group per thread where possible.
int row_threads(int D) {
  int t = D / 4;
  t = t < 64 ? 64 : (t > 1024 ? 1024 : t);
  return (t + 63) / 64 * 64;
}

template <typename T>
__device__ __forceinline__ float ldw(const void* p, int64_t i) {
  return Store<T>::ld(static_cast<const T*>(p) + i);
}

__device__ __forceinline__ float sum_parts(const float* part, int S, int64_t stride, int64_t i) {
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[s * stride + i];
  return v;
}

// Row kernels: one workgroup per row, each thread owns float4 column groups
// (D / 4 / blockDim of them); every split-K partial of a group is loaded before
// any is added, so a row costs one or two memory latencies instead of S*D/256.
constexpr int kRowMaxGroups = 4;     // float4 groups per thread (D <= 4 * 4 * blockDim)

__device__ __forceinline__ float4 f4add(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

__device__ __forceinline__ float4 sum_parts4(const float* part, int S, int64_t stride, int64_t i) {
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  int s = 0;
  for (; s + 4 <= S; s += 4) {
    const float4 a = *reinterpret_cast<const float4*>(part + (s + 0) * stride + i);
    const float4 b = *reinterpret_cast<const float4*>(part + (s + 1) * stride + i);
    const float4 c = *reinterpret_cast<const float4*>(part + (s + 2) * stride + i);
    const float4 d = *reinterpret_cast<const float4*>(part + (s + 3) * stride + i);
    v = f4add(f4add(f4add(f4add(v, a), b), c), d);
  }
  for (; s < S; ++s) v = f4add(v, *reinterpret_cast<const float4*>(part + s * stride + i));
  return v;
}

template <typename T>
__device__ __forceinline__ float4 ld4(const void* p, int64_t i) {
  if constexpr (sizeof(T) == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    return make_float4(bf16_to_f32(u.x & 0xffff), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xffff),
                       bf16_to_f32(u.y >> 16));
  } else {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
  }
}

template <typename T>
__device__ __forceinline__ void st4(void* p, int64_t i, float4 v) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t lo = f32_to_bf16(v.x) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16);
    const uint32_t hi = f32_to_bf16(v.z) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = make_uint2(lo, hi);
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(p) + i) = v;
  }
}

__device__ __forceinline__ float4 f4scale(float4 a, float4 g, float s) {
  return make_float4(g.x * (a.x * s), g.y * (a.y * s), g.z * (a.z * s), g.w * (a.w * s));
}

// ------------------------------------------------------------- ctx_norm
template <typename TW, typename TC>
__global__ __launch_bounds__(1024) void ctx_norm_kernel(const float* part, int S, int T_, int D,
                                                        const void* g, float eps, TC* out) {
  __shared__ float red[16];
  const int t = blockIdx.x;
  const int64_t stride = static_cast<int64_t>(T_) * D;
  float4 u[kRowMaxGroups];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kRowMaxGroups; ++j) {
    const int c = 4 * (threadIdx.x + j * blockDim.x);
    if (c < D) {
      u[j] = sum_parts4(part, S, stride, static_cast<int64_t>(t) * D + c);
      ss += u[j].x * u[j].x + u[j].y * u[j].y + u[j].z * u[j].z + u[j].w * u[j].w;
    }
  }
  const float inv = 1.0f / sqrtf(block_sum(ss, red) / D + eps);
#pragma unroll
  for (int j = 0; j < kRowMaxGroups; ++j) {
    const int c = 4 * (threadIdx.x + j * blockDim.x);
    if (c < D) st4<TC>(out, static_cast<int64_t>(t) * D + c, f4scale(u[j], ld4<TW>(g, c), inv));
  }
}

// ------------------------------------------------------------- scatter_kv
// Tile of 16 rows x 64 columns, 256 threads: thread t owns row t % 16 and the
// float4 column group t / 16.  Query and key columns are written along the
// column index; value columns go to the transposed value rows, where the 16
// threads of a column group write 16 consecutive cache positions.
template <typename T>
__global__ __launch_bounds__(256) void scatter_kv_kernel(ScatterArgs a) {
  if (a.len_dev != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < a.B)
    a.len_dev[threadIdx.x] = a.len_new[threadIdx.x];
  const int rr = threadIdx.x & 15, cg = threadIdx.x >> 4;
  const int r = blockIdx.y * 16 + rr, n = blockIdx.x * 64 + 4 * cg;
  if (r >= a.M || n >= a.N) return;
  const int64_t stride = static_cast<int64_t>(a.M) * a.N;
  const float4 v = sum_parts4(a.part, a.S, stride, static_cast<int64_t>(r) * a.N + n);
  if (n < a.nq) {
    *reinterpret_cast<float4*>(a.q_out + static_cast<int64_t>(r) * a.nq + n) = v;
    return;
  }
  const int hd = a.Hkv * a.d;
  const int kvn = n - a.nq;
  const int layer = a.layer0 + kvn / (2 * hd);
  const int rem = kvn % (2 * hd);
  int b = 0;
  while (b + 1 < a.rows.B && r >= a.rows.row_off[b + 1]) ++b;
  const int pos = a.rows.pos0[b] + (r - a.rows.row_off[b]);
  const int64_t head0 = (static_cast<int64_t>(layer) * a.B + a.rows.seq[b]) * a.Hkv;
  if (rem < hd) {
    const int j = rem / a.d, c = rem % a.d;
    // fp32 cache: row-major keys; bf16 cache: each 32-key block in fragment
    // order (dimensions c .. c + 3 stay adjacent: c % 8 is 0 or 4)
    const int64_t ki = sizeof(T) == 2
                           ? (head0 + j) * a.cap * a.d + static_cast<int64_t>(pos / 32) * (32 * a.d) +
                                 k_frag_offset(pos, c, a.d)
                           : ((head0 + j) * a.cap + pos) * a.d + c;
    st4<T>(a.kc, ki, v);
  } else {
    const int j = (rem - hd) / a.d, c = (rem - hd) % a.d;
    // fp32 cache: V^T [d][cap] per head; bf16 cache: V^T per block of 32 keys
    // ([cap / 32][d][32] per head), so dimension c + e of key pos sits e * 32 on
    const bool blocked = sizeof(T) == 2;
    T* vp = blocked ? static_cast<T*>(a.vc) + (head0 + j) * a.cap * a.d + static_cast<int64_t>(pos / 32) * (a.d * 32) +
                          c * 32 + pos % 32
                    : static_cast<T*>(a.vc) + ((head0 + j) * a.d + c) * a.cap + pos;
    const int64_t vs = blocked ? 32 : a.cap;
    Store<T>::st(vp, v.x);
    Store<T>::st(vp + vs, v.y);
    Store<T>::st(vp + 2 * vs, v.z);
    Store<T>::st(vp + 3 * vs, v.w);
  }
}

// ------------------------------------------------------------- residual_norm
template <typename T>
__global__ __launch_bounds__(1024) void residual_norm_kernel(const float* part, int S, int M, int D, float* h,
                                                             const void* g, float eps, float* a_out, HiLo pl,
                                                             void* tap) {
  __shared__ float red[16];
  const int m = blockIdx.x;
  const int64_t stride = static_cast<int64_t>(M) * D;
  float4 v[kRowMaxGroups];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kRowMaxGroups; ++j) {
    const int c = 4 * (threadIdx.x + j * blockDim.x);
    if (c < D) {
      const int64_t i = static_cast<int64_t>(m) * D + c;
      v[j] = *reinterpret_cast<const float4*>(h + i);
      if (part != nullptr) v[j] = f4add(v[j], sum_parts4(part, S, stride, i));
      *reinterpret_cast<float4*>(h + i) = v[j];
      if (tap != nullptr) st4<T>(tap, i, v[j]);
      ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    }
  }
  const float inv = 1.0f / sqrtf(block_sum(ss, red) / D + eps);
#pragma unroll
  for (int j = 0; j < kRowMaxGroups; ++j) {
    const int c = 4 * (threadIdx.x + j * blockDim.x);
    if (c < D) {
      const float4 y = f4scale(v[j], ld4<T>(g, c), inv);
      const int64_t o = static_cast<int64_t>(m) * D + c;
      if (pl.hi != nullptr) {
        uint2 hh, ll;
        split4(y, hh, ll);
        *reinterpret_cast<uint2*>(pl.hi + o) = hh;
        *reinterpret_cast<uint2*>(pl.lo + o) = ll;
      } else {
        *reinterpret_cast<float4*>(a_out + o) = y;
      }
    }
  }
}

// ------------------------------------------------------------- swiglu
__global__ __launch_bounds__(256) void swiglu_kernel(const float* part, int S, int M, int F, float* s_out, HiLo pl) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(M) * F) return;
  const int m = static_cast<int>(i / F), f = static_cast<int>(i % F);
  const int64_t stride = static_cast<int64_t>(M) * 2 * F;
  const float gt = sum_parts(part, S, stride, static_cast<int64_t>(m) * 2 * F + f);
  const float up = sum_parts(part, S, stride, static_cast<int64_t>(m) * 2 * F + F + f);
  const float v = gt / (1.0f + expf(-gt)) * up;
  if (pl.hi != nullptr) split1(v, pl.hi[i], pl.lo[i]);
  else s_out[i] = v;
}

// ------------------------------------------------------------- embed_norm
// Token ids come from device memory and cannot be checked on the host: ids
// outside [0, V) are clamped into range so a bad id can never read outside the
// embedding table.
template <typename T>
__global__ __launch_bounds__(1024) void embed_norm_kernel(const int32_t* tok, const float* ov, const void* embed,
                                                          int V, int D, const void* g, float eps, float* h,
                                                          float* a, HiLo pl) {
  __shared__ float red[16];
  const int m = blockIdx.x;
  const int64_t src = ov != nullptr ? 0 : static_cast<int64_t>(min(max(tok[m], 0), V - 1)) * D;
  float4 v[kRowMaxGroups];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kRowMaxGroups; ++j) {
    const int c = 4 * (threadIdx.x + j * blockDim.x);
    if (c < D) {
      v[j] = ov != nullptr ? *reinterpret_cast<const float4*>(ov + static_cast<int64_t>(m) * D + c)
                           : ld4<T>(embed, src + c);
      *reinterpret_cast<float4*>(h + static_cast<int64_t>(m) * D + c) = v[j];
      ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    }
  }
  const float inv = 1.0f / sqrtf(block_sum(ss, red) / D + eps);
#pragma unroll
  for (int j = 0; j < kRowMaxGroups; ++j) {
    const int c = 4 * (threadIdx.x + j * blockDim.x);
    if (c < D) {
      const float4 y = f4scale(v[j], ld4<T>(g, c), inv);
      const int64_t o = static_cast<int64_t>(m) * D + c;
      if (pl.hi != nullptr) {
        uint2 hh, ll;
        split4(y, hh, ll);
        *reinterpret_cast<uint2*>(pl.hi + o) = hh;
        *reinterpret_cast<uint2*>(pl.lo + o) = ll;
      } else {
        *reinterpret_cast<float4*>(a + o) = y;
      }
    }
  }
}

// ------------------------------------------------------------- argmax
__device__ void block_top2_write(Top2 t, int m, int32_t* draft, float* gap) {
  __shared__ float rv1[16], rv2[16];
  __shared__ int ri1[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) t = top2_merge(t, top2_shfl_xor(t, o));
  if (lane == 0) { rv1[w] = t.v1; ri1[w] = t.i1; rv2[w] = t.v2; }
  __syncthreads();
  if (threadIdx.x == 0) {
    Top2 r{rv1[0], ri1[0], rv2[0]};
    for (int i = 1; i < nw; ++i) r = top2_merge(r, Top2{rv1[i], ri1[i], rv2[i]});
    draft[m] = r.i1;
    if (gap != nullptr) gap[m] = r.v1 - r.v2;
  }
}

__global__ __launch_bounds__(256) void argmax_final_kernel(const float* top2, int ntiles, int M,
                                                           int32_t* draft, float* gap) {
  const int m = blockIdx.x;
  Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
  for (int i = threadIdx.x; i < ntiles; i += blockDim.x) {
    const float* p = top2 + (static_cast<int64_t>(i) * M + m) * 3;
    t = top2_merge(t, Top2{p[0], __float_as_int(p[1]), p[2]});
  }
  block_top2_write(t, m, draft, gap);
}

__global__ __launch_bounds__(256) void argmax_rows_kernel(const float* logits, int V, int32_t* draft,
                                                          float* gap) {
  const int m = blockIdx.x;
  Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
  for (int i = threadIdx.x; i < V; i += blockDim.x) t = top2_push(t, logits[static_cast<int64_t>(m) * V + i], i);
  block_top2_write(t, m, draft, gap);
}

// ------------------------------------------------------------- reduce_top2
// LM head: one workgroup of 128 threads per (512-column tile, row); each thread
// sums the split-K partials of 4 consecutive logits, optionally stores them, and
// the tile's top-2 is merged over the workgroup.
constexpr int kTop2Tile = 512;

__global__ __launch_bounds__(128) void reduce_top2_kernel(const float* part, int S, int M, int N, float* logits,
                                                          float* top2) {
  __shared__ float sv1[2], sv2[2];
  __shared__ int si1[2];
  const int tile = blockIdx.x, m = blockIdx.y;
  const int n = tile * kTop2Tile + 4 * threadIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t stride = static_cast<int64_t>(M) * N;
  const int64_t i = static_cast<int64_t>(m) * N + n;
  Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
  if ((N & 3) == 0 && n + 3 < N) {
    const float4 v = sum_parts4(part, S, stride, i);
    if (logits != nullptr) *reinterpret_cast<float4*>(logits + i) = v;
    t = top2_push(t, v.x, n);
    t = top2_push(t, v.y, n + 1);
    t = top2_push(t, v.z, n + 2);
    t = top2_push(t, v.w, n + 3);
  } else {
    for (int e = 0; e < 4 && n + e < N; ++e) {
      float v = 0.f;
      for (int s = 0; s < S; ++s) v += part[s * stride + i + e];
      if (logits != nullptr) logits[i + e] = v;
      t = top2_push(t, v, n + e);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) t = top2_merge(t, top2_shfl_xor(t, o));
  if (lane == 0) { sv1[w] = t.v1; si1[w] = t.i1; sv2[w] = t.v2; }
  __syncthreads();
  if (threadIdx.x == 0) {
    const Top2 r = top2_merge(Top2{sv1[0], si1[0], sv2[0]}, Top2{sv1[1], si1[1], sv2[1]});
    float* o = top2 + (static_cast<int64_t>(tile) * M + m) * 3;
    o[0] = r.v1;
    o[1] = __int_as_float(r.i1);
    o[2] = r.v2;
  }
}

// ------------------------------------------------------------- accept
__global__ __launch_bounds__(64) void accept_kernel(const int32_t* draft, const int32_t* target, int n,
                                                    int32_t* tau, int32_t* next_anchor) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const bool miss = lane < n && draft[static_cast<int64_t>(b) * n + lane] != target[static_cast<int64_t>(b) * (n + 1) + lane];
  const unsigned long long mask = __ballot(miss);
  const int m = mask ? __ffsll(mask) - 1 : n;
  if (lane == 0) {
    tau[b] = m + 1;
    next_anchor[b] = target[static_cast<int64_t>(b) * (n + 1) + m];
  }
}

// ------------------------------------------------------------- ragged blocks
// dst row m of sequence b (t.row_off[b] <= m < t.row_off[b + 1]) is src row
// t.pos0[b] + (m - t.row_off[b]); one workgroup per row, float4 columns.
__global__ __launch_bounds__(256) void gather_rows_kernel(const float* src, float* dst, int D, SeqRows t) {
  const int m = blockIdx.x;
  int b = 0;
  while (b + 1 < t.B && m >= t.row_off[b + 1]) ++b;
  const int64_t sr = t.pos0[b] + (m - t.row_off[b]);
  for (int c = 4 * threadIdx.x; c < D; c += 4 * blockDim.x)
    *reinterpret_cast<float4*>(dst + static_cast<int64_t>(m) * D + c) =
        *reinterpret_cast<const float4*>(src + sr * D + c);
}

// Sequence b's n_b = t.row_off[b + 1] - t.row_off[b] drafts start at draft +
// t.row_off[b] and its n_b + 1 target tokens at target + t.pos0[b].
__global__ __launch_bounds__(64) void accept_ragged_kernel(const int32_t* draft, const int32_t* target, SeqRows t,
                                                           int32_t* tau, int32_t* next_anchor) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int n = t.row_off[b + 1] - t.row_off[b];
  const int32_t* d = draft + t.row_off[b];
  const int32_t* tg = target + t.pos0[b];
  const bool miss = lane < n && d[lane] != tg[lane];
  const unsigned long long mask = __ballot(miss);
  const int m = mask ? __ffsll(mask) - 1 : n;
  if (lane == 0) {
    tau[b] = m + 1;
    next_anchor[b] = tg[m];
  }
}

}  // namespace

hipError_t launch_gather_rows(const float* src, float* dst, int D, const SeqRows& t, hipStream_t st) {
  const int M = t.row_off[t.B];
  if (M <= 0) return hipSuccess;
  if (D % 4 != 0) return hipErrorInvalidValue;
  int threads = D / 4 < 256 ? (D / 4 + 63) / 64 * 64 : 256;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(M), dim3(threads), 0, st, src, dst, D, t);
  return hipGetLastError();
}

hipError_t launch_accept_ragged(const int32_t* draft, const int32_t* target, const SeqRows& t, int32_t* tau,
                                int32_t* next_anchor, hipStream_t st) {
  hipLaunchKernelGGL(accept_ragged_kernel, dim3(t.B), dim3(64), 0, st, draft, target, t, tau, next_anchor);
  return hipGetLastError();
}

hipError_t launch_ctx_norm(const float* part, int S, int T, int D, const void* g, float eps, void* out,
                           bool bf16_weights, bool bf16_cache, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const size_t sh = 0;
  const dim3 grid(T), block(row_threads(D));
  if (bf16_weights && bf16_cache)
    hipLaunchKernelGGL((ctx_norm_kernel<uint16_t, uint16_t>), grid, block, sh, st, part, S, T, D, g, eps,
                       static_cast<uint16_t*>(out));
  else if (bf16_weights)
    hipLaunchKernelGGL((ctx_norm_kernel<uint16_t, float>), grid, block, sh, st, part, S, T, D, g, eps,
                       static_cast<float*>(out));
  else
    hipLaunchKernelGGL((ctx_norm_kernel<float, float>), grid, block, sh, st, part, S, T, D, g, eps,
                       static_cast<float*>(out));
  return hipGetLastError();
}

hipError_t launch_scatter_kv(const ScatterArgs& a, bool bf16_cache, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  dim3 grid((a.N + 63) / 64, (a.M + 15) / 16);
  if (bf16_cache) hipLaunchKernelGGL(scatter_kv_kernel<uint16_t>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(scatter_kv_kernel<float>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_residual_norm(const float* part, int S, int M, int D, float* h, const void* g, float eps,
                                float* a_out, bool bf16, hipStream_t st, HiLo pl, void* tap) {
  const dim3 block(row_threads(D));
  if ((pl.hi == nullptr) != (pl.lo == nullptr) || (pl.hi != nullptr && !bf16)) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(residual_norm_kernel<uint16_t>, dim3(M), block, 0, st, part, S, M, D, h, g, eps, a_out, pl,
                       tap);
  else
    hipLaunchKernelGGL(residual_norm_kernel<float>, dim3(M), block, 0, st, part, S, M, D, h, g, eps, a_out, pl, tap);
  return hipGetLastError();
}

hipError_t launch_swiglu(const float* part, int S, int M, int F, float* s_out, hipStream_t st, HiLo pl) {
  if ((pl.hi == nullptr) != (pl.lo == nullptr)) return hipErrorInvalidValue;
  const int64_t n = static_cast<int64_t>(M) * F;
  hipLaunchKernelGGL(swiglu_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, part, S, M, F, s_out,
                     pl);
  return hipGetLastError();
}

hipError_t launch_embed_norm(const int32_t* tok, const float* ov, const void* embed, int V, int M, int D,
                             const void* g, float eps, float* h, float* a, bool bf16, hipStream_t st, HiLo pl) {
  const dim3 block(row_threads(D));
  if ((pl.hi == nullptr) != (pl.lo == nullptr) || (pl.hi != nullptr && !bf16)) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(embed_norm_kernel<uint16_t>, dim3(M), block, 0, st, tok, ov, embed, V, D, g, eps, h, a, pl);
  else hipLaunchKernelGGL(embed_norm_kernel<float>, dim3(M), block, 0, st, tok, ov, embed, V, D, g, eps, h, a, pl);
  return hipGetLastError();
}

hipError_t launch_reduce_top2(const float* part, int S, int M, int N, float* logits, float* top2, int* ntiles_out,
                              hipStream_t st) {
  const int nt = (N + kTop2Tile - 1) / kTop2Tile;
  if (ntiles_out != nullptr) *ntiles_out = nt;
  hipLaunchKernelGGL(reduce_top2_kernel, dim3(nt, M), dim3(128), 0, st, part, S, M, N, logits, top2);
  return hipGetLastError();
}

hipError_t launch_argmax_final(const float* top2, int ntiles, int M, int32_t* draft, float* gap, hipStream_t st) {
  hipLaunchKernelGGL(argmax_final_kernel, dim3(M), dim3(256), 0, st, top2, ntiles, M, draft, gap);
  return hipGetLastError();
}

hipError_t launch_argmax_rows(const float* logits, int M, int V, int32_t* draft, float* gap, hipStream_t st) {
  hipLaunchKernelGGL(argmax_rows_kernel, dim3(M), dim3(256), 0, st, logits, V, draft, gap);
  return hipGetLastError();
}

hipError_t launch_accept(const int32_t* draft, const int32_t* target, int B, int n, int32_t* tau,
                         int32_t* next_anchor, hipStream_t st) {
  hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(64), 0, st, draft, target, n, tau, next_anchor);
  return hipGetLastError();
}

}  // namespace dflash
