// Per-step gather of the candidate tree (tokens, position ids) and the static
// tree tables (parent, depth, ancestor bitmask).
//
// aicassindra.com "Medusa deep dive", "From top-k heads to a sparse candidate
// tree": the tree is a flat node sequence with a matching attention mask and
// position ids; zackli.ai "Speculative Decoding Deep Dive II" ("Medusa"):
// Anc(i), the ancestors of node i.  The plan (which rank tuples are kept and
// their order) is computed on the host (tree_plan.cpp) and passed by value.
//
// Mask layout: bit (j mod 64) of word j/64 in row i is set iff j is i or an
// ancestor of i.  Position id of node i = seq_len + depth(i).

#include "common.h"
#include "kernels.h"

namespace medusa {

__global__ __launch_bounds__(256) void build_tree_kernel(TreeDev t, const int* __restrict__ root,
                                                         const int* __restrict__ idx,
                                                         const int* __restrict__ seq_len,
                                                         int* __restrict__ tokens,
                                                         int* __restrict__ pos,
                                                         int* __restrict__ parent,
                                                         int* __restrict__ depth,
                                                         uint64_t* __restrict__ anc) {
  const int s = blockIdx.x;
  const int P = seq_len[s];
  for (int j = threadIdx.x; j < t.T; j += blockDim.x) {
    const int dj = t.depth[j];
    int tok;
    if (j == 0) tok = root[s];
    else tok = idx[((int64_t)s * t.K + (dj - 1)) * t.kmax + t.rank[j]];
    tokens[(int64_t)s * t.T + j] = tok;
    pos[(int64_t)s * t.T + j] = P + dj;
    if (s == 0) {
      parent[j] = t.parent[j];
      depth[j] = dj;
      uint64_t w[kMaxAncWords] = {0, 0, 0, 0};
      for (int a = j; a >= 0; a = t.parent[a]) w[a >> 6] |= 1ull << (a & 63);
      for (int q = 0; q < t.anc_words; ++q) anc[(int64_t)j * t.anc_words + q] = q < kMaxAncWords ? w[q] : 0;
    }
  }
}

hipError_t run_build_tree(const TreeDev& t, const int* root, const int* idx, int b,
                          const int* seq_len, int* tokens, int* pos, int* parent, int* depth,
                          uint64_t* anc, hipStream_t st) {
  hipLaunchKernelGGL(build_tree_kernel, dim3(b), dim3(256), 0, st, t, root, idx, seq_len, tokens,
                     pos, parent, depth, anc);
  return hipGetLastError();
}

}  // namespace medusa
