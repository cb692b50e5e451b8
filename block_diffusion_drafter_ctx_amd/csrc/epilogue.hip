// Split-K reductions fused with each GEMM's consumer step, plus the small
// row-wise kernels of the drafter path:
//   ctx_norm       fusion epilogue: sum partials, RMSNorm with g_c, store H_t
//   scatter_kv     sum partials; query columns -> fp32 Q; key / value columns ->
//                  the KV cache (keys row-major, values transposed)
//   residual_norm  h += sum partials; a = RMSNorm(h; g)
//   swiglu         s = SiLU(gate) * up
//   embed_norm     h = embedding rows (or override rows); a = RMSNorm(h; g)
//   argmax_final   merge per-tile top-2 into draft ids and top-2 gaps
//   argmax_rows    same from plain fp32 logits rows (fp32 storage path)
//   accept         greedy acceptance length and next anchor (one wave per sequence)
// Every reduction sums partials in split order: results are bit-reproducible.
#include "common.h"
#include "launch.h"

namespace dflash {
namespace {

constexpr int kRowThreads = 256;

template <typename T>
__device__ __forceinline__ float ldw(const void* p, int64_t i) {
  return Store<T>::ld(static_cast<const T*>(p) + i);
}

__device__ __forceinline__ float sum_parts(const float* part, int S, int64_t stride, int64_t i) {
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[s * stride + i];
  return v;
}

// ------------------------------------------------------------- ctx_norm
template <typename TW, typename TC>
__global__ __launch_bounds__(kRowThreads) void ctx_norm_kernel(const float* part, int S, int T_, int D,
                                                               const void* g, float eps, TC* out) {
  __shared__ float red[16];
  extern __shared__ float row[];
  const int t = blockIdx.x;
  const int64_t stride = static_cast<int64_t>(T_) * D;
  float ss = 0.f;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    const float u = sum_parts(part, S, stride, static_cast<int64_t>(t) * D + c);
    row[c] = u;
    ss += u * u;
  }
  const float inv = 1.0f / sqrtf(block_sum(ss, red) / D + eps);
  for (int c = threadIdx.x; c < D; c += blockDim.x)
    Store<TC>::st(out + static_cast<int64_t>(t) * D + c, ldw<TW>(g, c) * (row[c] * inv));
}

// ------------------------------------------------------------- scatter_kv
// Tile of 32 rows x 64 columns; keys are written along d, values along rows.
template <typename T>
__global__ __launch_bounds__(256) void scatter_kv_kernel(ScatterArgs a) {
  __shared__ float tile[32][65];
  const int n0 = blockIdx.x * 64, r0 = blockIdx.y * 32;
  const int64_t stride = static_cast<int64_t>(a.M) * a.N;
  for (int e = threadIdx.x; e < 32 * 64; e += 256) {
    const int rr = e >> 6, cc = e & 63, r = r0 + rr, n = n0 + cc;
    float v = 0.f;
    if (r < a.M && n < a.N) v = sum_parts(a.part, a.S, stride, static_cast<int64_t>(r) * a.N + n);
    tile[rr][cc] = v;
  }
  __syncthreads();
  const int hd = a.Hkv * a.d;
  // query columns and key columns: write along the column index
  for (int e = threadIdx.x; e < 32 * 64; e += 256) {
    const int rr = e >> 6, cc = e & 63, r = r0 + rr, n = n0 + cc;
    if (r >= a.M || n >= a.N) continue;
    if (n < a.nq) {
      a.q_out[static_cast<int64_t>(r) * a.nq + n] = tile[rr][cc];
      continue;
    }
    const int kvn = n - a.nq;
    const int layer = a.layer0 + kvn / (2 * hd);
    const int rem = kvn % (2 * hd);
    if (rem >= hd) continue;                       // value column: second pass
    int b = 0;
    while (b + 1 < a.rows.B && r >= a.rows.row_off[b + 1]) ++b;
    const int pos = a.rows.pos0[b] + (r - a.rows.row_off[b]);
    const int j = rem / a.d, c = rem % a.d;
    const int64_t off = ((static_cast<int64_t>(layer) * a.B + b) * a.Hkv + j) * a.cap + pos;
    Store<T>::st(static_cast<T*>(a.kc) + off * a.d + c, tile[rr][cc]);
  }
  // value columns: write along the row (cache position) index
  for (int e = threadIdx.x; e < 32 * 64; e += 256) {
    const int cc = e >> 5, rr = e & 31, r = r0 + rr, n = n0 + cc;
    if (r >= a.M || n >= a.N || n < a.nq) continue;
    const int kvn = n - a.nq;
    const int layer = a.layer0 + kvn / (2 * hd);
    const int rem = kvn % (2 * hd);
    if (rem < hd) continue;
    int b = 0;
    while (b + 1 < a.rows.B && r >= a.rows.row_off[b + 1]) ++b;
    const int pos = a.rows.pos0[b] + (r - a.rows.row_off[b]);
    const int j = (rem - hd) / a.d, c = (rem - hd) % a.d;
    const int64_t off = (((static_cast<int64_t>(layer) * a.B + b) * a.Hkv + j) * a.d + c) * a.cap + pos;
    Store<T>::st(static_cast<T*>(a.vc) + off, tile[rr][cc]);
  }
}

// ------------------------------------------------------------- residual_norm
template <typename T>
__global__ __launch_bounds__(kRowThreads) void residual_norm_kernel(const float* part, int S, int M, int D,
                                                                    float* h, const void* g, float eps,
                                                                    float* a_out) {
  __shared__ float red[16];
  const int m = blockIdx.x;
  const int64_t stride = static_cast<int64_t>(M) * D;
  float* hr = h + static_cast<int64_t>(m) * D;
  float ss = 0.f;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float v = hr[c];
    if (part != nullptr) v += sum_parts(part, S, stride, static_cast<int64_t>(m) * D + c);
    hr[c] = v;
    ss += v * v;
  }
  const float inv = 1.0f / sqrtf(block_sum(ss, red) / D + eps);
  for (int c = threadIdx.x; c < D; c += blockDim.x)
    a_out[static_cast<int64_t>(m) * D + c] = ldw<T>(g, c) * (hr[c] * inv);
}

// ------------------------------------------------------------- swiglu
__global__ __launch_bounds__(256) void swiglu_kernel(const float* part, int S, int M, int F, float* s_out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(M) * F) return;
  const int m = static_cast<int>(i / F), f = static_cast<int>(i % F);
  const int64_t stride = static_cast<int64_t>(M) * 2 * F;
  const float gt = sum_parts(part, S, stride, static_cast<int64_t>(m) * 2 * F + f);
  const float up = sum_parts(part, S, stride, static_cast<int64_t>(m) * 2 * F + F + f);
  s_out[i] = gt / (1.0f + expf(-gt)) * up;
}

// ------------------------------------------------------------- embed_norm
// Token ids come from device memory and cannot be checked on the host: ids
// outside [0, V) are clamped into range so a bad id can never read outside the
// embedding table.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void embed_norm_kernel(const int32_t* tok, const float* ov,
                                                                 const void* embed, int V, int D, const void* g,
                                                                 float eps, float* h, float* a) {
  __shared__ float red[16];
  const int m = blockIdx.x;
  float* hr = h + static_cast<int64_t>(m) * D;
  const int64_t src = ov != nullptr ? 0 : static_cast<int64_t>(min(max(tok[m], 0), V - 1)) * D;
  float ss = 0.f;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    const float v = ov != nullptr ? ov[static_cast<int64_t>(m) * D + c] : ldw<T>(embed, src + c);
    hr[c] = v;
    ss += v * v;
  }
  const float inv = 1.0f / sqrtf(block_sum(ss, red) / D + eps);
  for (int c = threadIdx.x; c < D; c += blockDim.x)
    a[static_cast<int64_t>(m) * D + c] = ldw<T>(g, c) * (hr[c] * inv);
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

}  // namespace

hipError_t launch_ctx_norm(const float* part, int S, int T, int D, const void* g, float eps, void* out,
                           bool bf16_weights, bool bf16_cache, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const size_t sh = static_cast<size_t>(D) * sizeof(float);
  const dim3 grid(T), block(kRowThreads);
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
  dim3 grid((a.N + 63) / 64, (a.M + 31) / 32);
  if (bf16_cache) hipLaunchKernelGGL(scatter_kv_kernel<uint16_t>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(scatter_kv_kernel<float>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_residual_norm(const float* part, int S, int M, int D, float* h, const void* g, float eps,
                                float* a_out, bool bf16, hipStream_t st) {
  if (bf16) hipLaunchKernelGGL(residual_norm_kernel<uint16_t>, dim3(M), dim3(kRowThreads), 0, st, part, S, M, D, h, g, eps, a_out);
  else hipLaunchKernelGGL(residual_norm_kernel<float>, dim3(M), dim3(kRowThreads), 0, st, part, S, M, D, h, g, eps, a_out);
  return hipGetLastError();
}

hipError_t launch_swiglu(const float* part, int S, int M, int F, float* s_out, hipStream_t st) {
  const int64_t n = static_cast<int64_t>(M) * F;
  hipLaunchKernelGGL(swiglu_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, part, S, M, F, s_out);
  return hipGetLastError();
}

hipError_t launch_embed_norm(const int32_t* tok, const float* ov, const void* embed, int V, int M, int D,
                             const void* g, float eps, float* h, float* a, bool bf16, hipStream_t st) {
  if (bf16) hipLaunchKernelGGL(embed_norm_kernel<uint16_t>, dim3(M), dim3(kRowThreads), 0, st, tok, ov, embed, V, D, g, eps, h, a);
  else hipLaunchKernelGGL(embed_norm_kernel<float>, dim3(M), dim3(kRowThreads), 0, st, tok, ov, embed, V, D, g, eps, h, a);
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
