// Temperature sampling of the draft block and its lossless verification.
//
//   row_stats     per (row, 4096-column chunk): sum split-K partials if any,
//                 optionally store the logits, and write the chunk's SampleStat
//                 (best Gumbel key of x = logit / T when uniforms are given, and
//                 the log-sum-exp state of x)
//   sample_final  merge a row's SampleStat pieces: draft id and log sum exp(x)
//   spec_verify   per (sequence, 1024-column chunk): every workgroup of a sequence
//                 merges the row log-normalisers, finds the first rejected draft
//                 m, then draws its chunk's share of the emitted token: the best
//                 Gumbel key of the residual max(0, p_m - q_m) and of p_m (or of
//                 the bonus row p_n when nothing was rejected)
//   spec_final    merge the chunks: tau and the emitted token (next anchor)
//
// Merges run in a fixed order (lanes by xor-shuffle tree, waves and chunks in
// index order), so every result is bit-reproducible.
#include "common.h"
#include "launch.h"

namespace dflash {
namespace {

constexpr int kStatThreads = 256;
constexpr int kStatVec = 4 * kStatThreads;   // columns per float4 sweep of a workgroup
constexpr int kSweeps = kSampleChunk / kStatVec;   // float4 sweeps whose loads are issued together

__device__ __forceinline__ SampleStat wave_sstat(SampleStat s) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s = sstat_merge(s, sstat_shfl_xor(s, o));
  return s;
}

// Merge one SampleStat per thread over the workgroup (kStatThreads threads);
// the result is valid in thread 0.
__device__ __forceinline__ SampleStat block_sstat(SampleStat s) {
  __shared__ float4 w4[kStatThreads / kWave];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  s = wave_sstat(s);
  if (lane == 0) w4[w] = sstat_pack(s);
  __syncthreads();
  SampleStat r = sstat_unpack(w4[0]);
  for (int i = 1; i < kStatThreads / kWave; ++i) r = sstat_merge(r, sstat_unpack(w4[i]));
  return r;
}

__device__ __forceinline__ void stat_push(SampleStat& s, float v, int c, float inv_t, const float* su_row,
                                          bool sample) {
  const float x = v * inv_t;
  sstat_push_lse(s, x);
  if (sample) sstat_push_key(s, x + gumbel_noise(su_row[c]), c);
}

__global__ __launch_bounds__(kStatThreads) void row_stats_kernel(RowStatArgs a) {
  const int chunk = blockIdx.x, r = blockIdx.y;
  const bool second = r >= a.rows1;
  const float* src = second ? a.src2 + static_cast<int64_t>(r - a.rows1) * a.N : a.src + static_cast<int64_t>(r) * a.N;
  const int S = second ? 1 : a.S;
  const bool sample = a.su != nullptr;
  const float* su_row = sample ? a.su + static_cast<int64_t>(r) * a.N : nullptr;
  float* lo = (a.logits_out != nullptr && !second) ? a.logits_out + static_cast<int64_t>(r) * a.N : nullptr;
  const int c0 = chunk * a.chunk;
  const int c1 = min(a.N, c0 + a.chunk);
  SampleStat s = sstat_empty();
  if (a.vec) {
    // whole float4 groups (N % 4 == 0, 16-byte aligned rows); the loads of
    // kSweeps sweeps (and of each split level) are in flight together
    for (int c = c0 + 4 * threadIdx.x; c < c1; c += kStatVec * kSweeps) {
      float4 v[kSweeps], uv[kSweeps];
#pragma unroll
      for (int k = 0; k < kSweeps; ++k) {
        const int ck = c + k * kStatVec;
        v[k] = ck < c1 ? *reinterpret_cast<const float4*>(src + ck) : make_float4(0.f, 0.f, 0.f, 0.f);
        uv[k] = (sample && ck < c1) ? *reinterpret_cast<const float4*>(su_row + ck) : make_float4(0.5f, 0.5f, 0.5f, 0.5f);
      }
      for (int sp = 1; sp < S; ++sp) {
        float4 t[kSweeps];
#pragma unroll
        for (int k = 0; k < kSweeps; ++k) {
          const int ck = c + k * kStatVec;
          t[k] = ck < c1 ? *reinterpret_cast<const float4*>(src + sp * a.split_stride + ck) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < kSweeps; ++k) v[k] = make_float4(v[k].x + t[k].x, v[k].y + t[k].y, v[k].z + t[k].z, v[k].w + t[k].w);
      }
      // this thread's values of the block: maximum first, then one exp each
      float xs[kSweeps * 4];
      float bm = -INFINITY;
#pragma unroll
      for (int k = 0; k < kSweeps; ++k) {
        const int ck = c + k * kStatVec;
        const bool ok = ck < c1;
        if (ok && lo != nullptr) *reinterpret_cast<float4*>(lo + ck) = v[k];
        xs[4 * k + 0] = ok ? v[k].x * a.inv_t : -INFINITY;
        xs[4 * k + 1] = ok ? v[k].y * a.inv_t : -INFINITY;
        xs[4 * k + 2] = ok ? v[k].z * a.inv_t : -INFINITY;
        xs[4 * k + 3] = ok ? v[k].w * a.inv_t : -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) bm = fmaxf(bm, xs[4 * k + e]);
        if (sample && ok) {
          sstat_push_key(s, xs[4 * k + 0] + gumbel_noise(uv[k].x), ck);
          sstat_push_key(s, xs[4 * k + 1] + gumbel_noise(uv[k].y), ck + 1);
          sstat_push_key(s, xs[4 * k + 2] + gumbel_noise(uv[k].z), ck + 2);
          sstat_push_key(s, xs[4 * k + 3] + gumbel_noise(uv[k].w), ck + 3);
        }
      }
      if (bm != -INFINITY) {
        float se = 0.f;
#pragma unroll
        for (int e = 0; e < kSweeps * 4; ++e) se += fast_exp(xs[e] - bm);   // 0 for columns past the row
        SampleStat blk = sstat_empty();
        blk.mx = bm;
        blk.se = se;
        s = sstat_merge(s, blk);
      }
    }
  } else {
    for (int c = c0 + threadIdx.x; c < c1; c += kStatThreads) {
      float v = src[c];
      for (int sp = 1; sp < S; ++sp) v += src[sp * a.split_stride + c];
      if (lo != nullptr) lo[c] = v;
      stat_push(s, v, c, a.inv_t, su_row, sample);
    }
  }
  s = block_sstat(s);
  if (threadIdx.x == 0) a.stats[static_cast<int64_t>(chunk) * a.rows + r] = sstat_pack(s);
}

__global__ __launch_bounds__(kStatThreads) void sample_final_kernel(const float4* stats, int nparts, int M,
                                                                    int32_t* draft, float* lse) {
  const int m = blockIdx.x;
  SampleStat s = sstat_empty();
  for (int i = threadIdx.x; i < nparts; i += kStatThreads) s = sstat_merge(s, sstat_unpack(stats[static_cast<int64_t>(i) * M + m]));
  s = block_sstat(s);
  if (threadIdx.x == 0) {
    draft[m] = s.idx;
    if (lse != nullptr) lse[m] = s.mx + logf(s.se);
  }
}

// ------------------------------------------------------------- verification
constexpr int kSpecRowsPerWave = 2 * kSpecMaxN / (kStatThreads / kWave);

// The two candidate draws of the emitted token: best residual key (kr, ir) and
// best target key (kp, ip), each "larger key, then lower index".
struct Picks {
  float kr;
  int ir;
  float kp;
  int ip;
};

__device__ __forceinline__ Picks picks_empty() { return Picks{-INFINITY, 0x7fffffff, -INFINITY, 0x7fffffff}; }

__device__ __forceinline__ Picks picks_merge(Picks a, Picks b) {
  if (better(b.kr, b.ir, a.kr, a.ir)) { a.kr = b.kr; a.ir = b.ir; }
  if (better(b.kp, b.ip, a.kp, a.ip)) { a.kp = b.kp; a.ip = b.ip; }
  return a;
}

__device__ __forceinline__ Picks picks_shfl_xor(Picks a, int m) {
  return Picks{__shfl_xor(a.kr, m, kWave), __shfl_xor(a.ir, m, kWave), __shfl_xor(a.kp, m, kWave),
               __shfl_xor(a.ip, m, kWave)};
}

__device__ __forceinline__ float4 picks_pack(Picks a) {
  return make_float4(a.kr, __int_as_float(a.ir), a.kp, __int_as_float(a.ip));
}

__device__ __forceinline__ Picks picks_unpack(float4 v) {
  return Picks{v.x, __float_as_int(v.y), v.z, __float_as_int(v.w)};
}

__global__ __launch_bounds__(kStatThreads) void spec_verify_kernel(SpecArgs a) {
  __shared__ float s_lp[kSpecMaxN], s_lq[kSpecMaxN];
  __shared__ int s_m;
  __shared__ float4 w4[kStatThreads / kWave];
  const int chunk = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = a.n, V = a.V;
  const int c0 = chunk * kSpecDrawChunk, c1 = min(V, c0 + kSpecDrawChunk);
  const float* ru = a.resid_u + static_cast<int64_t>(b) * V;
  // the emitting uniforms do not depend on the decision: their load goes out first
  const int cv = c0 + 4 * static_cast<int>(threadIdx.x);
  float4 uv = make_float4(0.5f, 0.5f, 0.5f, 0.5f);
  if (a.vec && cv < c1) uv = *reinterpret_cast<const float4*>(ru + cv);
  // draft ids and acceptance uniforms (wave 0, lane j < n), then the gathered
  // logits, overlapped with the row-statistics loads below
  int dj = 0;
  float uj = 0.f;
  if (w == 0 && lane < n) {
    dj = a.draft[b * n + lane];
    dj = dj < 0 ? 0 : (dj >= V ? V - 1 : dj);
    uj = a.accept_u[b * n + lane];
  }
  // ---- log-normalisers of rows j < n: target rows, then draft rows unless given.
  // Wave w owns rows w, w + 4, ...; lane c < nchunk holds chunk c's piece.
  const int nrows = a.lse_q != nullptr ? n : 2 * n;
  SampleStat acc[kSpecRowsPerWave];
#pragma unroll
  for (int k = 0; k < kSpecRowsPerWave; ++k) {
    const int r = w + 4 * k;
    acc[k] = sstat_empty();
    if (r < nrows && lane < a.nchunk) {
      const int row = r < n ? b * (n + 1) + r : a.B * (n + 1) + b * n + (r - n);
      acc[k] = sstat_unpack(a.stats[static_cast<int64_t>(lane) * a.rows + row]);
    }
  }
#pragma unroll
  for (int k = 0; k < kSpecRowsPerWave; ++k) {
    const int r = w + 4 * k;
    if (r < nrows) {                         // uniform per wave
      const SampleStat t = wave_sstat(acc[k]);
      if (lane == 0) {
        const float l = t.mx + logf(t.se);
        if (r < n) s_lp[r] = l;
        else s_lq[r - n] = l;
      }
    }
  }
  float tp = 0.f, zq = 0.f;
  if (w == 0 && lane < n) {
    tp = a.zp[(static_cast<int64_t>(b) * (n + 1) + lane) * V + dj];
    zq = a.zq[(static_cast<int64_t>(b) * n + lane) * V + dj];
  }
  if (a.lse_q != nullptr && threadIdx.x < n) s_lq[threadIdx.x] = a.lse_q[b * n + threadIdx.x];
  __syncthreads();
  // ---- first rejection: draft j is kept when u_j < p_j(d_j) / q_j(d_j)
  if (w == 0) {
    bool rej = false;
    if (lane < n) {
      const float lr = (tp * a.inv_t - s_lp[lane]) - (zq * a.inv_t - s_lq[lane]);
      rej = !(uj < expf(lr));
    }
    const unsigned long long mask = __ballot(rej);
    if (lane == 0) s_m = mask ? __ffsll(mask) - 1 : n;
  }
  __syncthreads();
  // ---- this chunk's share of the emitted token's draw
  const int m = s_m;
  const bool resid = m < n;
  const float* rp = a.zp + (static_cast<int64_t>(b) * (n + 1) + m) * V;
  const float* rq = a.zq + (static_cast<int64_t>(b) * n + (resid ? m : 0)) * V;
  const float lp0 = resid ? s_lp[m] : 0.f, lq0 = resid ? s_lq[m] : 0.f;
  Picks pk = picks_empty();
  auto push = [&](float tv, float qv, float uv, int c) {
    const float g = gumbel_noise(uv);
    const float lp = tv * a.inv_t - lp0;
    const float key_p = lp + g;
    if (better(key_p, c, pk.kp, pk.ip)) { pk.kp = key_p; pk.ip = c; }
    if (resid) {
      const float lq = qv * a.inv_t - lq0;
      // log(p - q) = log p + log(1 - q / p) for p > q
      if (lp > lq) {
        const float key_r = lp + fast_log(-expm1f(lq - lp)) + g;
        if (better(key_r, c, pk.kr, pk.ir)) { pk.kr = key_r; pk.ir = c; }
      }
    }
  };
  if (a.vec) {
    // one float4 per thread (the chunk is one sweep of the workgroup)
    if (cv < c1) {
      const float4 tv = *reinterpret_cast<const float4*>(rp + cv);
      const float4 qv = resid ? *reinterpret_cast<const float4*>(rq + cv) : make_float4(0.f, 0.f, 0.f, 0.f);
      push(tv.x, qv.x, uv.x, cv);
      push(tv.y, qv.y, uv.y, cv + 1);
      push(tv.z, qv.z, uv.z, cv + 2);
      push(tv.w, qv.w, uv.w, cv + 3);
    }
  } else {
    for (int c = c0 + threadIdx.x; c < c1; c += kStatThreads) push(rp[c], resid ? rq[c] : 0.f, ru[c], c);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) pk = picks_merge(pk, picks_shfl_xor(pk, o));
  if (lane == 0) w4[w] = picks_pack(pk);
  __syncthreads();
  if (threadIdx.x == 0) {
    Picks r = picks_unpack(w4[0]);
    for (int i = 1; i < kStatThreads / kWave; ++i) r = picks_merge(r, picks_unpack(w4[i]));
    a.part[static_cast<int64_t>(b) * a.ndraw + chunk] = picks_pack(r);
    if (chunk == 0) a.m_out[b] = m;
  }
}

__global__ __launch_bounds__(64) void spec_final_kernel(const float4* part, const int32_t* m_in, int nchunk, int n,
                                                        int32_t* tau, int32_t* next_anchor) {
  const int b = blockIdx.x, lane = threadIdx.x;
  Picks pk = picks_empty();
  for (int c = lane; c < nchunk; c += 64) pk = picks_merge(pk, picks_unpack(part[static_cast<int64_t>(b) * nchunk + c]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) pk = picks_merge(pk, picks_shfl_xor(pk, o));
  if (lane == 0) {
    const int m = m_in[b];
    // an empty residual (possible only through rounding) falls back to p_m itself
    next_anchor[b] = (m < n && pk.kr != -INFINITY) ? pk.ir : pk.ip;
    tau[b] = m + 1;
  }
}

}  // namespace

int sample_chunk(int V, int rows) {
  // chunks of 4096 columns, widened so that a row has at most 64 of them and
  // the pass has about kStatTargetGroups workgroups (short-lived workgroups
  // cost more than their bytes)
  auto round_up = [](long x) { return static_cast<int>((x + kSampleChunk - 1) / kSampleChunk * kSampleChunk); };
  int c = round_up((V + kSpecMaxChunks - 1) / kSpecMaxChunks);
  const long want = rows > 0 ? (kStatTargetGroups + rows - 1) / rows : kSpecMaxChunks;   // chunks per row
  const int by_groups = round_up((V + want - 1) / want);
  if (by_groups > c) c = by_groups;
  return c > kSampleChunk ? c : kSampleChunk;
}

hipError_t launch_row_stats(const RowStatArgs& a0, hipStream_t st) {
  RowStatArgs a = a0;
  if (a.rows <= 0) return hipSuccess;
  if (a.chunk <= 0 || a.chunk % kStatVec != 0) return hipErrorInvalidValue;
  const int nchunk = (a.N + a.chunk - 1) / a.chunk;
  launch_k(row_stats_kernel, dim3(nchunk, a.rows), dim3(kStatThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_sample_final(const float4* stats, int nparts, int M, int32_t* draft, float* lse, hipStream_t st) {
  hipLaunchKernelGGL(sample_final_kernel, dim3(M), dim3(kStatThreads), 0, st, stats, nparts, M, draft, lse);
  return hipGetLastError();
}

hipError_t launch_spec_verify(const SpecArgs& a, hipStream_t st) {
  if (a.n < 1 || a.n > kSpecMaxN || a.nchunk < 1 || a.nchunk > kSpecMaxChunks ||
      a.ndraw != (a.V + kSpecDrawChunk - 1) / kSpecDrawChunk)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(spec_verify_kernel, dim3(a.ndraw, a.B), dim3(kStatThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(spec_final_kernel, dim3(a.B), dim3(64), 0, st, a.part, a.m_out, a.ndraw, a.n, a.tau,
                     a.next_anchor);
  return hipGetLastError();
}

}  // namespace dflash
