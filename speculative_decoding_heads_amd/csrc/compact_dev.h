// Device body of the KV rollback, shared by kv_compact_kernel and the fused
// acceptance walk (accept.hip).
//
// inferensys.com "Medusa Heads": after verification the process rolls back to
// the last accepted position; the speculative KV cache manages the entries of
// the candidate tree.  The tree nodes' K/V sit in cache slots P .. P+T-1 in
// node order; the accepted path (node path[d] at depth d, d = 0..L) moves to
// slots P + d for every kv head, K and V alike.
//
// In-place hazard: slot P + d is written while slot P + path[d'] may still be
// needed.  Nodes are numbered breadth-first, so path[d'] >= d' for every d';
// each thread owns a fixed 16-byte column of the (kv head, dim) slab and walks
// d = 0..L in order, reading slot P + path[d] before writing slot P + d.  A
// later source path[d'] (d' > d) is never a slot written earlier (path[d'] >= d'
// > d), and different threads touch disjoint columns, so no barrier is needed
// between the moves.
#pragma once

#include "common.h"

namespace medusa {

__device__ __forceinline__ void compact_columns(uint8_t* __restrict__ Kc, uint8_t* __restrict__ Vc,
                                                int s, int P, int L, const int* pth, int nkv,
                                                int Pmax, int row_bytes) {
  const int cols = row_bytes / 16;                // 16-byte columns per kv head row
  const int64_t slab = (int64_t)Pmax * row_bytes;  // bytes per (sequence, kv head)
  for (int item = threadIdx.x; item < 2 * nkv * cols; item += blockDim.x) {
    const int which = item / (nkv * cols);
    const int rem = item - which * nkv * cols;
    const int g = rem / cols, c = rem - g * cols;
    uint8_t* base = (which ? Vc : Kc) + ((int64_t)s * nkv + g) * slab + (int64_t)c * 16;
    for (int d = 0; d <= L; ++d) {
      const int src = pth[d];
      if (src == d || src < 0 || P + src >= Pmax || P + d >= Pmax) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(base + (int64_t)(P + src) * row_bytes);
      *reinterpret_cast<uint4*>(base + (int64_t)(P + d) * row_bytes) = v;
    }
  }
}

}  // namespace medusa
