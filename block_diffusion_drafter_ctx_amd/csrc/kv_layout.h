// Layout of the bf16 KV cache, shared by its writer (scatter_kv) and its reader
// (the attention).  Per (layer, sequence, kv head) the cache holds blocks of 32
// keys, each block contiguous (32 * d elements of K, then of V, in two arrays):
//   V: the block's V^T, [d][32];
//   K: the block in the order of the attention's score fragments, 2 * (d / 32)
//      fragments of 512 elements.  Fragment t * (d / 32) + s holds keys
//      8 q + 4 t + r (q, r < 4) at dimensions [32 s, 32 s + 32); inside it lane
//      l = 16 g + 4 q + r owns the 8 dimensions from 32 s + 8 g of key
//      8 q + 4 t + r, so each fragment is one contiguous kilobyte.
#pragma once

#include <hip/hip_runtime.h>

namespace dflash {

// Element offset of (key i, dimension c) of a bf16 K cache from the start of
// the block that holds key i.
__host__ __device__ __forceinline__ int k_frag_offset(int i, int c, int d) {
  const int kk = i & 31;
  const int f = ((kk & 7) >> 2) * (d >> 5) + (c >> 5);
  const int l = 16 * ((c & 31) >> 3) + 4 * (kk >> 3) + (kk & 3);
  return f * 512 + l * 8 + (c & 7);
}

}  // namespace dflash
