// MTP-style draft heads: one transformer layer per head, shared unembedding.
//
// zackli.ai "Speculative Decoding Deep Dive II: Medusa, MTP", section "MTP":
// n heads on the trunk's h_t, each a transformer layer f_{h_i}, the logits
// f_u(f_{h_i}(h_t)) through one shared unembedding; the drafts then take the
// same tree verification as Medusa heads.  The page gives no layer shape; the
// layer here is one pre-norm transformer layer of the trunk's kind, at the
// current position:
//   a  = RMSNorm(h; g1)        q, k, v = a Wq^T, a Wk^T, a Wv^T
//   o  = attention of q over the head's cache [0, P) plus (k, v) at slot P
//   x1 = h + o Wo^T            a2 = RMSNorm(x1; g2)
//   y  = x1 + (SiLU(a2 Wg^T) * (a2 Wu^T)) Wd^T
//   logits = LM y  (slot 0: LM h, the base head)
// Every stage runs for all K heads in one launch: the GEMMs batched over
// heads (gemm.hip epilogues EpiQKV, EpiResid, EpiSwiGLU), the attention as
// the tree attention kernel with a one-node tree over the (head, sequence)
// pairs, the LM projection as one weight stream over all K + 1 rows of every
// sequence.  bf16 operands, f32 accumulation, intermediates stored in bf16.

#include "common.h"
#include "kernels.h"

namespace medusa {

// out[hd, m, :] = bf16(x[hd, m, :] / sqrt(mean(x^2) + eps) * g[hd, :]), the
// row of x at x + hd * sx + m * H (sx = 0: the same row for every head).
// One 256-thread workgroup per (row, head); H % 8 == 0.  The first launch of
// a draft also copies h into slot 0 of u, expands seq_len over the heads and
// writes the one-node ancestor mask (the pointers are NULL otherwise).
__global__ __launch_bounds__(256) void rmsnorm_bf16(const uint16_t* __restrict__ x, int64_t sx,
                                                    const uint16_t* __restrict__ g, int H,
                                                    float eps, int M, uint16_t* __restrict__ out,
                                                    uint16_t* __restrict__ u, int R,
                                                    const int* __restrict__ seq_len,
                                                    int* __restrict__ seq_exp,
                                                    uint64_t* __restrict__ anc1) {
  const int m = blockIdx.x, hd = blockIdx.y;
  const uint16_t* xr = x + hd * sx + (int64_t)m * H;
  const int pieces = H >> 3;
  float ss = 0.f;
  for (int c = threadIdx.x; c < pieces; c += 256) {
    const uint4 w = ldg16(xr + 8 * c);
    const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = bf16_lo(q[j]), hi = bf16_hi(q[j]);
      ss = fmaf(lo, lo, ss);
      ss = fmaf(hi, hi, ss);
    }
  }
  ss = wave_sum(ss);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  ss = (part[0] + part[1]) + (part[2] + part[3]);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  const uint16_t* gr = g + (int64_t)hd * H;
  uint16_t* orow = out + ((int64_t)hd * M + m) * H;
  for (int c = threadIdx.x; c < pieces; c += 256) {
    const uint4 w = ldg16(xr + 8 * c);
    const uint4 gw = ldg16(gr + 8 * c);
    const uint32_t q[4] = {w.x, w.y, w.z, w.w};
    const uint32_t gq[4] = {gw.x, gw.y, gw.z, gw.w};
    uint4 o;
    uint32_t* op = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      op[j] = pack_bf16x2(bf16_lo(q[j]) * r * bf16_lo(gq[j]), bf16_hi(q[j]) * r * bf16_hi(gq[j]));
    *reinterpret_cast<uint4*>(orow + 8 * c) = o;
    if (u && hd == 0) *reinterpret_cast<uint4*>(u + (int64_t)m * R * H + 8 * c) = w;
  }
  if (seq_exp && threadIdx.x == 0) seq_exp[hd * M + m] = seq_len[m];
  if (anc1 && m == 0 && hd == 0 && threadIdx.x == 0) anc1[0] = 1ull;
}

static size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace: a, a2, x1 [K, M, H]; attention q and o [K * M, nq d]; SwiGLU
// output [K, M, F]; u [M, K+1, H] when the caller keeps none; the expanded
// seq_len [K * M]; the one-word ancestor mask; the attention partials.
MtpLayout mtp_layout(int M, int H, int K, int F, int nq, int nkv, int d, int Pmax, bool own_u) {
  MtpLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += up256(bytes);
    return at;
  };
  const size_t e = sizeof(uint16_t);
  L.a = take((size_t)K * M * H * e);
  L.a2 = take((size_t)K * M * H * e);
  L.x1 = take((size_t)K * M * H * e);
  L.q = take((size_t)K * M * nq * d * e);
  L.o = take((size_t)K * M * nq * d * e);
  L.z = take((size_t)K * M * F * e);
  L.u = own_u ? take((size_t)M * (K + 1) * H * e) : 0;
  L.seq = take((size_t)K * M * sizeof(int));
  L.anc = take(sizeof(uint64_t));
  L.plan = attn_plan(K * M, 1, nq, nkv, d, Pmax, kBF16);
  L.attn = take(L.plan.ws_bytes);
  L.bytes = o;
  return L;
}

hipError_t run_mtp_draft(const MtpArgs& a, void* u_out, float* logits, void* ws, hipStream_t st) {
  const int M = a.b, H = a.H, K = a.K, F = a.F, nqd = a.nq * a.d;
  const MtpLayout L = mtp_layout(M, H, K, F, a.nq, a.nkv, a.d, a.Pmax, u_out == nullptr);
  char* w = static_cast<char*>(ws);
  uint16_t* act = reinterpret_cast<uint16_t*>(w + L.a);
  uint16_t* act2 = reinterpret_cast<uint16_t*>(w + L.a2);
  uint16_t* x1 = reinterpret_cast<uint16_t*>(w + L.x1);
  uint16_t* q = reinterpret_cast<uint16_t*>(w + L.q);
  uint16_t* o = reinterpret_cast<uint16_t*>(w + L.o);
  uint16_t* z = reinterpret_cast<uint16_t*>(w + L.z);
  uint16_t* u = u_out ? static_cast<uint16_t*>(u_out) : reinterpret_cast<uint16_t*>(w + L.u);
  int* seq = reinterpret_cast<int*>(w + L.seq);
  uint64_t* anc = reinterpret_cast<uint64_t*>(w + L.anc);
  const uint16_t* h = static_cast<const uint16_t*>(a.h);
  const int R = K + 1;
  // 1. a = RMSNorm(h; g1) per head; u slot 0 = h; seq_len per (head, sequence)
  hipLaunchKernelGGL(rmsnorm_bf16, dim3(M, K), dim3(256), 0, st, h, (int64_t)0,
                     static_cast<const uint16_t*>(a.g1), H, a.eps, M, act, u, R, a.seq_len, seq,
                     anc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 2. q -> q; k, v -> each head's cache at slot seq_len
  e = run_mtp_qkv(act, M, H, static_cast<const uint16_t*>(a.Wqkv), K, a.nq, a.nkv, a.d, q,
                  static_cast<uint16_t*>(a.Kh), static_cast<uint16_t*>(a.Vh), a.seq_len, a.Pmax,
                  st);
  if (e != hipSuccess) return e;
  // 3. attention at the current position: a one-node tree per (head, sequence)
  e = run_tree_attn(q, a.Kh, a.Vh, seq, anc, 1, K * M, 1, a.nq, a.nkv, a.d, a.Pmax,
                    1.0f / sqrtf((float)a.d), kBF16, o, w + L.attn, L.plan, st);
  if (e != hipSuccess) return e;
  // 4. x1 = h + o Wo^T
  e = run_mtp_resid(o, nqd, (int64_t)M * nqd, M, nqd, static_cast<const uint16_t*>(a.Wo), H, K,
                    x1, (int64_t)M * H, H, h, 0, H, st);
  if (e != hipSuccess) return e;
  // 5. a2 = RMSNorm(x1; g2)
  hipLaunchKernelGGL(rmsnorm_bf16, dim3(M, K), dim3(256), 0, st, x1, (int64_t)M * H,
                     static_cast<const uint16_t*>(a.g2), H, a.eps, M, act2, nullptr, 0, nullptr,
                     nullptr, nullptr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 6. z = SiLU(a2 Wg^T) * (a2 Wu^T)
  e = run_mtp_swiglu(act2, M, H, static_cast<const uint16_t*>(a.Wgu), F, K, z, st);
  if (e != hipSuccess) return e;
  // 7. y = x1 + z Wd^T -> u slot head + 1
  e = run_mtp_resid(z, F, (int64_t)M * F, M, F, static_cast<const uint16_t*>(a.Wd), H, K, u + H,
                    H, (int64_t)R * H, x1, (int64_t)M * H, H, st);
  if (e != hipSuccess) return e;
  // 8. logits of every slot through the shared LM projection (the K chunks
  //    walked backwards, as for Medusa head rows)
  return run_lm_logits(u, M * R, H, a.LM, a.V, kBF16, logits, st, true);
}

}  // namespace medusa
