// State carried from one draft-and-verify step to the next.
//
// inferensys.com "Medusa Heads" (decoding loop; speculative KV cache): each
// step drafts from the hidden state at the last accepted position, the tree's
// key/value entries enter the cache behind the accepted prefix, and after
// verification the cache is rolled back to the accepted path (compaction, in
// compact_dev.h).  These two kernels move the rest of that state:
//   kv_append_kernel  - the step's tree K/V (one row per tree node, from the
//                       verification pass) into cache slots P .. P+T-1,
//                       P = seq_len[s];
//   next_hidden_kernel - the verification state of the chosen node (the last
//                       accepted position) becomes the next step's hidden
//                       state: h[s] = O[s, path[s, L[s]]].
// Both are byte copies in 16-byte units; sequences whose seq_len, L or path
// are out of range are left untouched.
//
// accept_tally_kernel counts, over the steps of a run, how often each (depth,
// rank) candidate was offered (its parent lay on the accepted path) and
// accepted: the per-rank acceptance rates from which the tree budget is
// planned (aicassindra.com "Medusa deep dive", "From top-k heads to a sparse
// candidate tree": the tree shape is a tuned budget).

#include "common.h"
#include "kernels.h"

namespace medusa {

__global__ __launch_bounds__(256) void kv_append_kernel(uint8_t* __restrict__ Kc,
                                                        uint8_t* __restrict__ Vc,
                                                        const int* __restrict__ seq_len,
                                                        const uint8_t* __restrict__ Kn,
                                                        const uint8_t* __restrict__ Vn, int nkv,
                                                        int Pmax, int T, int row_bytes) {
  const int sg = blockIdx.x;                 // s * nkv + g
  const int s = sg / nkv;
  const int P = seq_len[s];
  if (P < 0 || P > Pmax - T) return;
  const int64_t units = (int64_t)T * row_bytes / 16;
  const uint4* ks = reinterpret_cast<const uint4*>(Kn + (int64_t)sg * T * row_bytes);
  const uint4* vs = reinterpret_cast<const uint4*>(Vn + (int64_t)sg * T * row_bytes);
  uint4* kd = reinterpret_cast<uint4*>(Kc + ((int64_t)sg * Pmax + P) * row_bytes);
  uint4* vd = reinterpret_cast<uint4*>(Vc + ((int64_t)sg * Pmax + P) * row_bytes);
  for (int64_t u = threadIdx.x; u < units; u += blockDim.x) {
    const uint4 a = ks[u], b = vs[u];
    kd[u] = a;
    vd[u] = b;
  }
}

__global__ __launch_bounds__(256) void next_hidden_kernel(const uint8_t* __restrict__ O,
                                                          const int* __restrict__ path,
                                                          const int* __restrict__ L, int T, int K,
                                                          int row_bytes, uint8_t* __restrict__ h) {
  const int s = blockIdx.x;
  const int l = L[s];
  if (l < 0 || l > K) return;
  const int node = path[(int64_t)s * (K + 1) + l];
  if (node < 0 || node >= T) return;
  const uint4* src = reinterpret_cast<const uint4*>(O + ((int64_t)s * T + node) * row_bytes);
  uint4* dst = reinterpret_cast<uint4*>(h + (int64_t)s * row_bytes);
  for (int u = threadIdx.x; u < row_bytes / 16; u += blockDim.x) dst[u] = src[u];
}

// One workgroup per sequence, one thread per tree node.  onpath[n] = the depth
// at which node n lies on the accepted path (-1 if it does not); a node of
// depth D was offered when its parent lies on the path at depth D-1, and
// accepted when it lies on the path itself.  Counts are [K][16] (depth-1,
// rank), added to.
__global__ __launch_bounds__(kMaxT) void accept_tally_kernel(const int* __restrict__ L,
                                                             const int* __restrict__ path, int K,
                                                             TreeDev t,
                                                             unsigned long long* __restrict__ acc,
                                                             unsigned long long* __restrict__ off) {
  const int s = blockIdx.x, tid = threadIdx.x;
  __shared__ int onpath[kMaxT];
  const int l = L[s];
  if (l < 0 || l > K) return;            // uniform across the workgroup
  onpath[tid] = -1;
  __syncthreads();
  if (tid <= l) {
    const int n = path[(int64_t)s * (K + 1) + tid];
    if (n >= 0 && n < t.T) onpath[n] = tid;
  }
  __syncthreads();
  if (tid >= 1 && tid < t.T) {
    const int D = t.depth[tid], r = t.rank[tid];
    if (onpath[t.parent[tid]] == D - 1) {
      atomicAdd(&off[(D - 1) * 16 + r], 1ull);
      if (onpath[tid] == D) atomicAdd(&acc[(D - 1) * 16 + r], 1ull);
    }
  }
}

hipError_t run_accept_tally(const int* L, const int* path, int b, int K, const TreeDev& t,
                            int64_t* accepted, int64_t* offered, hipStream_t st) {
  hipLaunchKernelGGL(accept_tally_kernel, dim3(b), dim3(kMaxT), 0, st, L, path, K, t,
                     reinterpret_cast<unsigned long long*>(accepted),
                     reinterpret_cast<unsigned long long*>(offered));
  return hipGetLastError();
}

hipError_t run_kv_append(void* Kc, void* Vc, const int* seq_len, const void* Knew,
                         const void* Vnew, int b, int nkv, int Pmax, int T, int d, int dtype,
                         hipStream_t st) {
  const int row_bytes = d * (dtype == kBF16 ? 2 : 4);
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)b * nkv), dim3(256), 0, st,
                     static_cast<uint8_t*>(Kc), static_cast<uint8_t*>(Vc), seq_len,
                     static_cast<const uint8_t*>(Knew), static_cast<const uint8_t*>(Vnew), nkv,
                     Pmax, T, row_bytes);
  return hipGetLastError();
}

hipError_t run_next_hidden(const void* O, const int* path, const int* L, int b, int T, int K,
                           int H, int dtype, void* h, hipStream_t st) {
  const int row_bytes = H * (dtype == kBF16 ? 2 : 4);
  hipLaunchKernelGGL(next_hidden_kernel, dim3(b), dim3(256), 0, st,
                     static_cast<const uint8_t*>(O), path, L, T, K, row_bytes,
                     static_cast<uint8_t*>(h));
  return hipGetLastError();
}

}  // namespace medusa
