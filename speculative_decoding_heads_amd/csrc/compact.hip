// Rollback / compaction of the accepted path's K/V entries.
//
// inferensys.com "Medusa Heads": after verification the process rolls back to
// the last accepted position; the speculative KV cache manages the entries of
// the candidate tree.  The tree nodes' K/V sit in cache slots P .. P+T-1 in
// node order; the accepted path (node path[d] at depth d, d = 0..L) moves to
// slots P + d for every kv head, K and V alike, and seq_len becomes P + L + 1.
//
// In-place hazard: slot P + d is written while slot P + path[d'] may still be
// needed.  Nodes are numbered breadth-first, so path[d'] >= d' for every d';
// each thread owns a fixed 16-byte column of the (kv head, dim) slab and walks
// d = 0..L in order, reading slot P + path[d] before writing slot P + d.  A
// later source path[d'] (d' > d) is never a slot written earlier (path[d'] >= d'
// > d), and different threads touch disjoint columns, so no barrier is needed
// between the moves.  The seq_len update waits for every thread's read of it.

#include "common.h"
#include "kernels.h"

namespace medusa {

__global__ __launch_bounds__(256) void kv_compact_kernel(uint8_t* __restrict__ Kc,
                                                         uint8_t* __restrict__ Vc,
                                                         int* __restrict__ seq_len,
                                                         const int* __restrict__ path,
                                                         const int* __restrict__ Lin, int nkv,
                                                         int Pmax, int row_bytes, int K) {
  const int s = blockIdx.x;
  const int P = seq_len[s];
  const int L = Lin[s];
  const bool ok = P >= 0 && L >= 0 && L <= K;
  const int* pth = path + (int64_t)s * (K + 1);
  const int cols = row_bytes / 16;                // 16-byte columns per kv head row
  const int64_t slab = (int64_t)Pmax * row_bytes;  // bytes per (sequence, kv head)
  if (ok) {
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
  __syncthreads();
  if (threadIdx.x == 0 && ok) seq_len[s] = P + L + 1;
}

hipError_t run_kv_compact(void* Kc, void* Vc, int* seq_len, const int* path, const int* L, int b,
                          int nkv, int Pmax, int d, int K, int dtype, hipStream_t st) {
  const int row_bytes = d * (dtype == kBF16 ? 2 : 4);
  hipLaunchKernelGGL(kv_compact_kernel, dim3(b), dim3(256), 0, st, static_cast<uint8_t*>(Kc),
                     static_cast<uint8_t*>(Vc), seq_len, path, L, nkv, Pmax, row_bytes, K);
  return hipGetLastError();
}

}  // namespace medusa
