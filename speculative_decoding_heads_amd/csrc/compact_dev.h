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
// each thread owns a fixed 16-byte column of the (kv head, dim) slab and moves
// d = 0..L in order (reads of a group of four before its writes), so a later
// source path[d'] (d' > d) is never a slot written earlier, and different
// threads touch disjoint columns: no barrier is needed between the moves.
#pragma once

#include "common.h"
#include "kernels.h"

namespace medusa {

// Moves of one sequence; pth[d], d = 0..L <= kMaxHeads, is the accepted path.
// A thread takes up to four of its columns at a time and moves them in
// groups of four consecutive d: all sixteen source reads are in flight
// together before the group's writes.  Safe because path[d'] >= d' > d for
// every later d', so no later read hits a slot written before it.  Slots out
// of range (only with an inconsistent seq_len or path) are left alone.
__device__ __forceinline__ void compact_columns(uint8_t* __restrict__ Kc, uint8_t* __restrict__ Vc,
                                                int s, int P, int L, const int* pth, int nkv,
                                                int Pmax, int row_bytes) {
  constexpr int IB = 4;                           // columns per thread per pass
  const int cols = row_bytes / 16;                // 16-byte columns per kv head row
  const int64_t slab = (int64_t)Pmax * row_bytes;  // bytes per (sequence, kv head)
  const int nitems = 2 * nkv * cols;
  for (int i0 = threadIdx.x; i0 < nitems; i0 += IB * blockDim.x) {
    uint8_t* base[IB];
    bool live[IB];
#pragma unroll
    for (int j = 0; j < IB; ++j) {
      const int item = i0 + j * blockDim.x;
      live[j] = item < nitems;
      const int it = live[j] ? item : i0;
      const int which = it / (nkv * cols);
      const int rem = it - which * nkv * cols;
      const int g = rem / cols, c = rem - g * cols;
      base[j] = (which ? Vc : Kc) + ((int64_t)s * nkv + g) * slab + (int64_t)c * 16;
    }
    // the root never moves (path[0] = 0): start the groups of four at depth 1
    for (int d0 = pth[0] == 0 ? 1 : 0; d0 <= L; d0 += 4) {
      int src[4];
      bool mv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = d0 + q;
        const int sd = d <= L ? pth[d] : d;
        mv[q] = !(sd == d || sd < 0 || P + sd >= Pmax || P + d >= Pmax);
        src[q] = mv[q] ? P + sd : min(P, Pmax - 1);   // otherwise a discarded in-range read
      }
      if (!(mv[0] || mv[1] || mv[2] || mv[3])) continue;   // nothing moves in this group
      typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
      u32x4 v[IB][4];
#pragma unroll
      for (int j = 0; j < IB; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[j][q] = *reinterpret_cast<const u32x4*>(base[j] + (int64_t)src[q] * row_bytes);
#pragma unroll
      for (int j = 0; j < IB; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (live[j] && mv[q])
            *reinterpret_cast<u32x4*>(base[j] + (int64_t)(P + d0 + q) * row_bytes) = v[j][q];
    }
  }
}

}  // namespace medusa
