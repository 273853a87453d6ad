// Rollback / compaction of the accepted path's K/V entries (the moves are in
// compact_dev.h); seq_len becomes P + L + 1 once every thread has read it.

#include "common.h"
#include "compact_dev.h"
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
  if (ok) compact_columns(Kc, Vc, s, P, L, path + (int64_t)s * (K + 1), nkv, Pmax, row_bytes);
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
