// Hydra-style sequentially dependent draft heads.
//
// zackli.ai "Speculative Decoding Deep Dive II: Medusa, MTP", section
// "Medusa": Medusa heads see only the hidden state h_t, never the token just
// drafted, so their accuracy falls with the offset; Hydra gives the later
// heads that token (better drafts, less parallelism).  aicassindra.com
// "Medusa deep dive", "The heads are residual blocks, not linear layers": a
// head is u = y + SiLU(W y) projected by the shared LM head.
//
// Reading taken (the pages give Hydra one sentence): head d (1..K) takes
// y = bf16(h + e(x)) in place of h, where e is the base model's input
// embedding table and x the token one position earlier on the candidate's
// path (the root for head 1, the depth-(d-1) token for head d).  Every node
// at depth d-1 therefore gets its own head-d logits and shortlist, and node
// (r_1, ..., r_d) of the tree plan takes rank r_d of its parent's shortlist.
// With e = 0 this is the Medusa draft.  The tree plan, its tables, positions
// and everything after the draft are the Medusa step's.
//
// Per depth d (sequential; one pass of the LM weights per depth):
//   gemm (heads)   u = y + SiLU(W_d y), bf16, y the rows (s, node of depth d-1)
//                  of bf16(h[s] + e[token])                 (run_heads_hidden)
//   gemm (LM)      logits of every parent row               (run_lm_logits)
//   topk_rows      the parent rows' top-k_d                 (run_topk, no root)
//   hydra_next     token(child) = shortlist(parent)[rank(child)], and the
//                  children's rows of y for depth d+1
// (hydra_embed writes depth 1's rows from the root.)
// The root (argmax / sample of LM h, or given) and the tree tables come from
// one run_topk launch on the plan before depth 1.

#include "common.h"
#include "kernels.h"

namespace medusa {

// Head input of depth 1, one workgroup per sequence: y[s] = bf16(h[s] +
// e[root[s]]), 16-byte pieces added in float and rounded once.  Tokens outside
// [0, V) are clamped into it, so every read stays inside e.
__global__ __launch_bounds__(256) void hydra_embed(const uint16_t* __restrict__ h,
                                                   const uint16_t* __restrict__ E,
                                                   const int* __restrict__ root, int H, int V,
                                                   uint16_t* __restrict__ y) {
  const int r = blockIdx.x, s = r;
  int tok = root[s];
  tok = min(max(tok, 0), V - 1);
  const uint4* hp = reinterpret_cast<const uint4*>(h + (int64_t)s * H);
  const uint4* ep = reinterpret_cast<const uint4*>(E + (int64_t)tok * H);
  uint4* yp = reinterpret_cast<uint4*>(y + (int64_t)r * H);
  for (int c = threadIdx.x; c < H / 8; c += blockDim.x) {
    const uint4 a = hp[c], e = ep[c];
    uint4 o;
    o.x = pack_bf16x2(bf16_lo(a.x) + bf16_lo(e.x), bf16_hi(a.x) + bf16_hi(e.x));
    o.y = pack_bf16x2(bf16_lo(a.y) + bf16_lo(e.y), bf16_hi(a.y) + bf16_hi(e.y));
    o.z = pack_bf16x2(bf16_lo(a.z) + bf16_lo(e.z), bf16_hi(a.z) + bf16_hi(e.z));
    o.w = pack_bf16x2(bf16_lo(a.w) + bf16_lo(e.w), bf16_hi(a.w) + bf16_hi(e.w));
    yp[c] = o;
  }
}

// One workgroup per (sequence, node c of depth d), row r = s * nchild + (c -
// first): c's token is rank r_c of its parent's shortlist (idx row s * n_par +
// (parent - first_par)); when a deeper depth follows (y != nullptr) the same
// workgroup also writes c's row of the next depth's head input,
// y[r] = bf16(h[s] + e[token]), as hydra_embed does for the root.
__global__ __launch_bounds__(256) void hydra_next(const int* __restrict__ idx, int kmax,
                                                  TreeDev t, int first, int nchild, int first_par,
                                                  int n_par, const uint16_t* __restrict__ h,
                                                  const uint16_t* __restrict__ E, int H, int V,
                                                  int* __restrict__ tokens,
                                                  uint16_t* __restrict__ y) {
  const int r = blockIdx.x;
  const int s = r / nchild, c = first + (r - s * nchild);
  const int p = t.parent[c];
  int tok = idx[((int64_t)s * n_par + (p - first_par)) * kmax + t.rank[c]];
  if (threadIdx.x == 0) tokens[(int64_t)s * t.T + c] = tok;
  if (y == nullptr) return;
  tok = min(max(tok, 0), V - 1);
  const uint4* hp = reinterpret_cast<const uint4*>(h + (int64_t)s * H);
  const uint4* ep = reinterpret_cast<const uint4*>(E + (int64_t)tok * H);
  uint4* yp = reinterpret_cast<uint4*>(y + (int64_t)r * H);
  for (int q = threadIdx.x; q < H / 8; q += blockDim.x) {
    const uint4 a = hp[q], e = ep[q];
    uint4 o;
    o.x = pack_bf16x2(bf16_lo(a.x) + bf16_lo(e.x), bf16_hi(a.x) + bf16_hi(e.x));
    o.y = pack_bf16x2(bf16_lo(a.y) + bf16_lo(e.y), bf16_hi(a.y) + bf16_hi(e.y));
    o.z = pack_bf16x2(bf16_lo(a.z) + bf16_lo(e.z), bf16_hi(a.z) + bf16_hi(e.z));
    o.w = pack_bf16x2(bf16_lo(a.w) + bf16_lo(e.w), bf16_hi(a.w) + bf16_hi(e.w));
    yp[q] = o;
  }
}

// logits_out rows (s, first + j) <- parent row r = s * n + j of the pass
// (rows of the pass are 2V apart: row 0 of each pair is the unused root slot).
__global__ __launch_bounds__(256) void hydra_copy_rows(const float* __restrict__ lg, int V, int T,
                                                       int first, int n, float* __restrict__ out) {
  const int r = blockIdx.x;
  const int s = r / n, j = r - s * n;
  const float* src = lg + ((int64_t)2 * r + 1) * V;
  float* dst = out + ((int64_t)s * T + first + j) * V;
  for (int c = threadIdx.x; c < V; c += blockDim.x) dst[c] = src[c];
}

HydraShape hydra_shape(const TreeDev& t) {
  HydraShape hs{};
  hs.D = 0;
  for (int i = 0; i < t.T; ++i) {
    const int d = t.depth[i];
    if (hs.n[d] == 0) hs.first[d] = i;
    ++hs.n[d];
    hs.D = d > hs.D ? d : hs.D;
  }
  return hs;
}

static int64_t hydra_rows(int b, const HydraShape& hs) {
  int m = 1;
  for (int d = 0; d < hs.D; ++d) m = hs.n[d] > m ? hs.n[d] : m;
  return (int64_t)b * m;
}

static size_t up16(size_t x) { return (x + 15) & ~(size_t)15; }

// y | u (bf16 [M, H]) | logits (float [M, 2, V]) | idx (int [M, kmax]) |
// val (float [M, kmax]) | top-k workspace of M rows
size_t hydra_workspace(int b, int H, int V, int kmax, const HydraShape& hs) {
  const size_t M = (size_t)hydra_rows(b, hs);
  return 2 * up16(M * H * 2) + up16(M * 2 * V * 4) + 2 * up16(M * kmax * 4) +
         up16(topk_workspace((int)M, 1, V, kmax));
}

hipError_t run_hydra_draft(const void* h, const void* E, const void* W, const void* LM, int H,
                           const TopkArgs& a, const TreeDev& t, const TreeOut& o, int* root,
                           float* logits_out, void* ws, hipStream_t st) {
  const int b = a.b, V = a.V, kmax = a.kmax;
  const HydraShape hs = hydra_shape(t);
  const size_t M = (size_t)hydra_rows(b, hs);
  char* p = static_cast<char*>(ws);
  uint16_t* y = reinterpret_cast<uint16_t*>(p);
  p += up16(M * H * 2);
  uint16_t* u = reinterpret_cast<uint16_t*>(p);
  p += up16(M * H * 2);
  float* lg = reinterpret_cast<float*>(p);
  p += up16(M * 2 * V * 4);
  int* idx = reinterpret_cast<int*>(p);
  p += up16(M * kmax * 4);
  float* val = reinterpret_cast<float*>(p);
  p += up16(M * kmax * 4);
  void* tws = p;

  // root (argmax / sample of LM h, or given) and the tree tables; head rows
  // of this launch have k = 0 and return at once
  if (a.root_mode != kRootGiven) {
    hipError_t e = run_lm_logits(h, b, H, LM, V, kBF16, lg, st, false, 2 * (int64_t)V);
    if (e != hipSuccess) return e;
  }
  TopkArgs r = a;
  r.K = 1;
  r.k[0] = 0;
  hipError_t e = run_topk(lg, r, root, idx, val, tws, st, &t, &o);
  if (e != hipSuccess) return e;

  const uint16_t* Wb = static_cast<const uint16_t*>(W);
  for (int d = 1; d <= hs.D; ++d) {
    const int n = hs.n[d - 1], first = hs.first[d - 1];
    const int rows = b * n;
    if (d == 1) {
      hipLaunchKernelGGL(hydra_embed, dim3(b), dim3(256), 0, st, static_cast<const uint16_t*>(h),
                         static_cast<const uint16_t*>(E), root, H, V, y);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    e = run_heads_hidden(y, rows, H, Wb + (size_t)(d - 1) * H * H, 1, kBF16, u, 1, 0, st);
    if (e != hipSuccess) return e;
    // consecutive passes walk the weights' K chunks in opposite directions, so
    // each starts on what the previous pass read last (still in the last-level
    // cache); the root pass, when there is one, walks forwards
    e = run_lm_logits(u, rows, H, LM, V, kBF16, lg + V, st, (d & 1) != 0, 2 * (int64_t)V);
    if (e != hipSuccess) return e;
    if (logits_out) {
      hipLaunchKernelGGL(hydra_copy_rows, dim3(rows), dim3(256), 0, st, lg, V, t.T, first, n,
                         logits_out);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    TopkArgs q{};
    q.b = rows; q.K = 1; q.V = V; q.kmax = kmax; q.root_mode = kRootGiven;
    q.k[0] = a.k[d - 1];
    e = run_topk(lg, q, nullptr, idx, val, tws, st);
    if (e != hipSuccess) return e;
    // the children's tokens and, below the deepest depth, their head inputs
    const int nchild = hs.n[d];
    hipLaunchKernelGGL(hydra_next, dim3(b * nchild), dim3(256), 0, st, idx, kmax, t, hs.first[d],
                       nchild, first, n, static_cast<const uint16_t*>(h),
                       static_cast<const uint16_t*>(E), H, V, o.tokens, d < hs.D ? y : nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace medusa
