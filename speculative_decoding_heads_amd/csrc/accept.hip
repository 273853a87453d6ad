// Greedy / typical / exact rejection-sampling acceptance, path choice and the
// next token.
//
// aiunderstanding.org "Medusa Decoding Heads" ("Deep Dive"): accept the longest
// prefix that matches what the model would have produced; inferensys.com
// "Medusa Heads": stop at the first rejection, roll back to the last accepted
// position, the base model supplies the next token; aicassindra.com "Medusa
// deep dive" ("Typical acceptance, not exact rejection sampling"): accept a
// token whose probability exceeds min(eps, delta * exp(-H)), H the entropy of
// the model's distribution.
//
// Conventions: greedy argmax ties go to the lower vocabulary index; typical
// uses q = softmax(x / T), natural-log entropy and a strict '>'.  A node is
// fully accepted when it and every ancestor below the root is accepted;
// L = the largest depth of a fully accepted node, the chosen node the lowest
// node index at that depth.  Next token: argmax there (greedy) or a seeded
// float64 sample from softmax(x / T) there (typical, counter draw 1).
//
// Kernels:
//   accept_stats: one 1024-thread workgroup per (sequence, node) row of base
//     logits; a single streaming pass with 16-byte loads.  Greedy: argmax key.  Typical:
//     online (m, s, t) with s = sum e^(x'-m), t = sum e^(x'-m)(x'-m),
//     x' = x / T, rescaled whenever the running max moves; then
//     H = ln s - t/s and log q(tok) = x'_tok - m - ln s.
//   accept_parts: the same statistics merged from the verify GEMM's per-tile
//     partials, one wave per node row.
//   accept_walk: one workgroup per sequence: local flags, full-path flags by
//     walking ancestors, block max/min for L and the chosen node, path and
//     accepted tokens.
//   typical mode then runs the shared float64 row sampler on the chosen node.
//
// Rejection mode (aiunderstanding.org "Medusa Decoding Heads", "Deep Dive":
// rejection sampling against the original model keeps its distribution;
// aicassindra.com "Medusa deep dive": the heads give no proposal distribution
// of their own): a node's candidates are point-mass proposals tried in node
// order; child j is taken when u_j (1 - r_j) < p(t_j) (r_j = the mass of the
// children already rejected, p the parent's tempered distribution from the
// typical statistics), so every candidate is emitted with exactly its
// probability.  The walk follows the first taken child; where every child is
// rejected the next token is drawn from the row without those children's
// tokens (the sampler's exclusion list), at a leaf from the full row.

#include "common.h"
#include "compact_dev.h"
#include "kernels.h"

namespace medusa {

constexpr int kStatThreads = 1024;

// One 1024-thread workgroup per node row; each lane issues a group of 16-byte
// loads before using any, then folds them into its argmax key (greedy: a
// float compare per value, one key per pass) or its (m, s, t) state (typical:
// the pass's max, one exponential per value, one merge); waves reduce by
// shuffles, LDS joins waves.
template <int MODE>
__global__ __launch_bounds__(kStatThreads) void accept_stats(const float* __restrict__ logits,
                                                             int V, float inv_temp,
                                                             int* __restrict__ amax,
                                                             RowStat* __restrict__ stats) {
  const int64_t row = blockIdx.x;
  const float* x = logits + row * V;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NW = kStatThreads / 64;
  constexpr int U = 8;
  uint64_t best = 0;
  float m = -INFINITY, s = 0.f, t = 0.f;
  auto take = [&](float v, int e) {
    if (MODE == kGreedy) {
      const uint64_t k = make_key(v, e);
      best = k > best ? k : best;
    } else {
      stat_add(m, s, t, v * inv_temp);
    }
  };
  if ((V & 3) == 0) {
    const int nv = V >> 2;
    for (int base = 0; base < nv; base += U * kStatThreads) {
      f32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = base + u * kStatThreads + tid;
        v[u] = e < nv ? *reinterpret_cast<const f32x4*>(x + 4 * e) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (MODE == kGreedy) {
        // this pass's largest value at its lowest index (indices rise along
        // the loop, so a strict '>' keeps the first of equal values; -0.0 and
        // +0.0 compare equal, as in the key), then one key
        float bv = -INFINITY;
        int bi = -1;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int e = base + u * kStatThreads + tid;
          if (e < nv) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const bool tk = bi < 0 || v[u][q] > bv;
              bv = tk ? v[u][q] : bv;
              bi = tk ? 4 * e + q : bi;
            }
          }
        }
        if (bi >= 0) take(bv, bi);
      } else {
        // this pass's values: their max first, then one exponential each, then
        // a single merge into the running statistics (no per-value rescale)
        float pm = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (base + u * kStatThreads + tid < nv)
#pragma unroll
            for (int q = 0; q < 4; ++q) pm = fmaxf(pm, v[u][q] * inv_temp);
        float ps = 0.f, pt = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (base + u * kStatThreads + tid < nv)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float d = v[u][q] * inv_temp - pm;
              const float ex = __expf(d);
              ps += ex;
              pt = fmaf(ex, d, pt);
            }
        if (ps > 0.f) stat_merge(m, s, t, pm, ps, pt);
      }
    }
  } else {
    for (int e = tid; e < V; e += kStatThreads) take(x[e], e);
  }
  if (MODE == kGreedy) {
    best = wave_max_u64(best);
    __shared__ uint64_t sb[NW];
    if (lane == 0) sb[wave] = best;
    __syncthreads();
    if (tid == 0) {
      uint64_t bb = sb[0];
      for (int w = 1; w < NW; ++w) bb = sb[w] > bb ? sb[w] : bb;
      amax[row] = (int)key_index(bb);
    }
  } else {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64), t2 = __shfl_xor(t, o, 64);
      stat_merge(m, s, t, m2, s2, t2);
    }
    __shared__ float sm[NW][3];
    if (lane == 0) { sm[wave][0] = m; sm[wave][1] = s; sm[wave][2] = t; }
    __syncthreads();
    if (tid == 0) {
      float M = sm[0][0], S = sm[0][1], Tt = sm[0][2];
      for (int w = 1; w < NW; ++w) stat_merge(M, S, Tt, sm[w][0], sm[w][1], sm[w][2]);
      stats[row] = RowStat{M, S, Tt, 0.f};
    }
  }
}

// The same statistics from the verify GEMM's per-tile partials: one wave per
// node row; each lane merges tiles lane, lane + 64, ... (four in flight), then
// the wave reduces its lanes.  The partials are used only when their header
// says they were made for this call (rows, vocabulary, kind of statistics and
// temperature); otherwise the wave folds the logits row itself, so a
// mismatched workspace gives the statistics of the logits, never a read past
// the partials.
template <int MODE>
__global__ __launch_bounds__(256) void accept_parts(const int* __restrict__ hdr,
                                                    const uint64_t* __restrict__ pkey,
                                                    const RowStat* __restrict__ pstat, int rows,
                                                    const float* __restrict__ logits, int V,
                                                    float inv_temp, int* __restrict__ amax,
                                                    RowStat* __restrict__ stats) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const bool typ = MODE == kTypical;
  const bool match = hdr[kHdrMagic] == kPartsMagic && hdr[kHdrRows] == rows &&
                     hdr[kHdrCols] == V && hdr[kHdrKind] == (typ ? 1 : 0) &&
                     hdr[kHdrTiles] >= 1 && (!typ || hdr[kHdrInvTemp] == __float_as_int(inv_temp));
  const int ntiles = match ? hdr[kHdrTiles] : 0;
  RowPart acc;
  part_init(acc);
  if (!match) {
    const float* x = logits + (int64_t)row * V;
    for (int e = lane; e < V; e += 64) part_add(acc, x[e], e, typ, inv_temp);
  }
  for (int j0 = 0; j0 < ntiles; j0 += 4 * 64) {
    RowPart q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * 64 + lane;
      const int64_t o = (int64_t)row * ntiles + min(j, ntiles - 1);
      const bool ok = j < ntiles;
      if (MODE == kGreedy) {
        q[u].key = ok ? pkey[o] : 0ull;
      } else {
        const RowStat st = pstat[o];
        q[u].m = st.m;
        q[u].s = ok ? st.s : 0.f;
        q[u].t = st.t;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) part_merge(acc, q[u], MODE == kTypical);
  }
  if (MODE == kGreedy) {
    acc.key = wave_max_u64(acc.key);
    if (lane == 0) amax[row] = (int)key_index(acc.key);
  } else {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part_xor(acc, o, true);
    if (lane == 0) stats[row] = RowStat{acc.m, acc.s, acc.t, 0.f};
  }
}

__device__ __forceinline__ bool full_path(int c, const int* sparent, const unsigned char* local) {
  bool full = true;
  for (int a = c; a > 0;) {
    full = full && local[a];
    const int p = sparent[a];
    if (p < 0 || p >= a) return false;
    a = p;
  }
  return full;
}

template <int MODE>
__global__ __launch_bounds__(256) void accept_walk(const float* __restrict__ logits,
                                                   const int* __restrict__ tokens,
                                                   const int* __restrict__ parent,
                                                   const int* __restrict__ depth, int T, int V,
                                                   int K, float inv_temp, float eps, float delta,
                                                   const int* __restrict__ amax,
                                                   const RowStat* __restrict__ stats,
                                                   int* __restrict__ Lout, int* __restrict__ path,
                                                   int* __restrict__ acc_tokens,
                                                   int* __restrict__ bonus, int* __restrict__ best_out,
                                                   uint8_t* __restrict__ Kc, uint8_t* __restrict__ Vc,
                                                   int* __restrict__ seq_len, int nkv, int Pmax,
                                                   int row_bytes, uint64_t seed, uint64_t step,
                                                   int* __restrict__ excl) {
  constexpr bool kStats = MODE == kTypical || MODE == kReject;   // tempered row statistics
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ int spath[kMaxHeads + 1];
  const int P = Kc ? seq_len[s] : 0;
  __shared__ unsigned char local[kMaxT];
  __shared__ int sdepth[kMaxT], sparent[kMaxT];
  __shared__ int samax[kMaxT];
  __shared__ RowStat sstat[kMaxT];
  __shared__ int stok[kMaxT];
  __shared__ int bestL, bestNode;
  if (tid == 0) { bestL = 0; bestNode = 0x7fffffff; }
  // Node c (thread c; T <= kMaxT <= blockDim.x): its parent, depth, token and
  // (typical) the logit of its token in the parent's row are loaded before the
  // statistics below, so their latency overlaps that work.
  int my_parent = -1, my_tok = -1;
  bool my_valid = false;
  float my_logit = 0.f;
  if (tid < T) {
    my_parent = parent[tid];
    my_tok = tokens[(int64_t)s * T + tid];
    sparent[tid] = my_parent;
    sdepth[tid] = depth[tid];
    stok[tid] = my_tok;
    my_valid = tid > 0 && my_tok >= 0 && my_tok < V && my_parent >= 0 && my_parent < tid;
    if (kStats && my_valid)
      my_logit = logits[((int64_t)s * T + my_parent) * V + my_tok];
  }
  // per-node statistics of this sequence
  for (int p = tid; p < T; p += blockDim.x) {
    const int64_t row = (int64_t)s * T + p;
    if (MODE == kGreedy) samax[p] = amax[row];
    else sstat[p] = stats[row];
  }
  __syncthreads();
  if constexpr (MODE == kReject) {
    // Exact rejection sampling: p = the node's token under its parent's
    // tempered distribution; child j (node order) of a depth-d node is
    // accepted when u * (1 - r) < p, r = the p of its earlier siblings, u =
    // draw 16 d + j keyed by splitmix64(seed); the walk takes the first
    // accepted child at every node.
    __shared__ double sp[kMaxT];
    __shared__ int first_acc[kMaxT], first_kid[kMaxT], sj[kMaxT];
    if (tid < T) {
      double pc = 0.0;
      if (my_valid) {
        const RowStat st = sstat[my_parent];
        pc = exp((double)(my_logit * inv_temp) - (double)st.m - log((double)st.s));
      }
      sp[tid] = pc;
      first_acc[tid] = T;
      first_kid[tid] = T;
    }
    __syncthreads();
    if (tid > 0 && tid < T && my_parent >= 0 && my_parent < tid) atomicMin(&first_kid[my_parent], tid);
    __syncthreads();
    if (tid < T) sj[tid] = 0;
    if (tid < T && my_valid) {
      // the earlier siblings: from the parent's first child (siblings follow
      // one another in node order, so this is at most kmax - 1 steps)
      double r = 0.0;
      int j = 0;
      for (int c = first_kid[my_parent]; c < tid; ++c)
        if (sparent[c] == my_parent) {
          r += sp[c];
          ++j;
        }
      sj[tid] = j;
      const uint64_t draw = (uint64_t)(16 * sdepth[my_parent] + j);
      const double u = counter_uniform(splitmix64(seed), step, (uint64_t)s, draw);
      if (u * (1.0 - r) < sp[tid]) atomicMin(&first_acc[my_parent], tid);
    }
    __syncthreads();
    if (tid == 0) {
      int n = 0, d = 0;
      while (d < K && first_acc[n] < T) {   // children follow their parent: the walk ends
        n = first_acc[n];
        ++d;
      }
      bestL = d;
      bestNode = n;
    }
    __syncthreads();
    // the stop node's children were all rejected: the next token is drawn
    // without their tokens (none when it has no children)
    if (tid < kSampExcl) excl[(int64_t)s * kSampExcl + tid] = -1;
    __syncthreads();
    if (my_valid && my_parent == bestNode && sj[tid] < kSampExcl)
      excl[(int64_t)s * kSampExcl + sj[tid]] = stok[tid];
  } else {
    if (tid < T) {
      bool ok = tid == 0;
      if (my_valid) {
        if (MODE == kGreedy) {
          ok = my_tok == samax[my_parent];
        } else {
          const RowStat st = sstat[my_parent];
          const double lns = log((double)st.s);
          const double H = lns - (double)st.t / (double)st.s;
          const double logq = (double)(my_logit * inv_temp) - (double)st.m - lns;
          const double thr = fmin((double)eps, (double)delta * exp(-H));
          ok = exp(logq) > thr;
        }
      }
      local[tid] = ok;
    }
    __syncthreads();
    // A parent table is valid when 0 <= parent[c] < c; anything else is
    // treated as a rejected node, so the walks below always end.
    for (int c = tid; c < T; c += blockDim.x) {
      if (full_path(c, sparent, local)) atomicMax(&bestL, sdepth[c]);
    }
    __syncthreads();
    for (int c = tid; c < T; c += blockDim.x) {
      if (full_path(c, sparent, local) && sdepth[c] == bestL) atomicMin(&bestNode, c);
    }
  }
  __syncthreads();
  if (tid == 0) {
    const int L = bestL, best = bestNode;
    Lout[s] = L;
    for (int d = L + 1; d <= K; ++d) {
      path[(int64_t)s * (K + 1) + d] = -1;
      acc_tokens[(int64_t)s * (K + 1) + d] = -1;
    }
    int a = best;
    for (int d = L; d >= 0; --d) {
      path[(int64_t)s * (K + 1) + d] = a;
      spath[d] = a;
      acc_tokens[(int64_t)s * (K + 1) + d] = stok[a];
      a = a > 0 ? sparent[a] : 0;
    }
    if (MODE == kGreedy) bonus[s] = samax[best];
    best_out[s] = best;
  }
  if (!Kc) return;
  // fused rollback of the accepted path's K/V (the same moves as medusa_kv_compact)
  __syncthreads();
  const int L = bestL;
  const bool ok = P >= 0 && L >= 0 && L <= K;
  if (ok) compact_columns(Kc, Vc, s, P, L, spath, nkv, Pmax, row_bytes);
  __syncthreads();
  if (tid == 0 && ok) seq_len[s] = P + L + 1;
}

// Workspace: stats per node row, amax per node row, the chosen node per
// sequence, the excluded tokens per sequence (rejection mode), then (16-byte
// aligned) the sampler's slice partials.
static size_t samp_offset(int b, int T) {
  const size_t rows = (size_t)b * T;
  return (rows * sizeof(RowStat) + rows * sizeof(int) + (size_t)b * sizeof(int) +
          (size_t)b * kSampExcl * sizeof(int) + 15) & ~(size_t)15;
}

size_t accept_workspace(int b, int T) { return samp_offset(b, T) + sample_workspace(b); }

hipError_t run_accept(const float* base_logits, const int* tokens, const int* parent,
                      const int* depth, int b, int T, int V, int K, int mode, float temperature,
                      float eps, float delta, uint64_t seed, uint64_t step, int* L, int* path,
                      int* acc_tokens, int* bonus, void* ws, hipStream_t st, const KvRollback* kv,
                      const void* parts) {
  const size_t rows = (size_t)b * T;
  RowStat* stats = static_cast<RowStat*>(ws);
  int* amax = reinterpret_cast<int*>(stats + rows);
  int* best = amax + rows;
  int* excl = best + b;
  const float inv_temp = 1.0f / temperature;
  uint8_t* Kc = kv ? static_cast<uint8_t*>(kv->Kc) : nullptr;
  uint8_t* Vc = kv ? static_cast<uint8_t*>(kv->Vc) : nullptr;
  int* seq_len = kv ? kv->seq_len : nullptr;
  const int nkv = kv ? kv->nkv : 0, Pmax = kv ? kv->Pmax : 0;
  const int row_bytes = kv ? kv->d * (kv->dtype == kBF16 ? 2 : 4) : 0;
  const int* hdr = static_cast<const int*>(parts);
  const uint64_t* pkey =
      parts ? reinterpret_cast<const uint64_t*>(static_cast<const char*>(parts) + kPartsHeader) : nullptr;
  const RowStat* pstat =
      parts ? reinterpret_cast<const RowStat*>(static_cast<const char*>(parts) + kPartsHeader) : nullptr;
  const unsigned pgrid = (unsigned)((rows + 3) / 4);
  if (mode == kGreedy) {
    if (parts)
      hipLaunchKernelGGL(accept_parts<kGreedy>, dim3(pgrid), dim3(256), 0, st, hdr, pkey, pstat,
                         (int)rows, base_logits, V, inv_temp, amax, stats);
    else
      hipLaunchKernelGGL(accept_stats<kGreedy>, dim3((unsigned)rows), dim3(kStatThreads), 0, st,
                         base_logits, V, inv_temp, amax, stats);
    hipLaunchKernelGGL(accept_walk<kGreedy>, dim3(b), dim3(256), 0, st, base_logits, tokens,
                       parent, depth, T, V, K, inv_temp, eps, delta, amax, stats, L, path,
                       acc_tokens, bonus, best, Kc, Vc, seq_len, nkv, Pmax, row_bytes, seed, step,
                       excl);
    return hipGetLastError();
  }
  // typical and rejection modes: tempered statistics of every node row
  if (parts)
    hipLaunchKernelGGL(accept_parts<kTypical>, dim3(pgrid), dim3(256), 0, st, hdr, pkey, pstat,
                       (int)rows, base_logits, V, inv_temp, amax, stats);
  else
    hipLaunchKernelGGL(accept_stats<kTypical>, dim3((unsigned)rows), dim3(kStatThreads), 0, st,
                       base_logits, V, inv_temp, amax, stats);
  if (mode == kReject)
    hipLaunchKernelGGL(accept_walk<kReject>, dim3(b), dim3(256), 0, st, base_logits, tokens,
                       parent, depth, T, V, K, inv_temp, eps, delta, amax, stats, L, path,
                       acc_tokens, bonus, best, Kc, Vc, seq_len, nkv, Pmax, row_bytes, seed, step,
                       excl);
  else
    hipLaunchKernelGGL(accept_walk<kTypical>, dim3(b), dim3(256), 0, st, base_logits, tokens,
                       parent, depth, T, V, K, inv_temp, eps, delta, amax, stats, L, path,
                       acc_tokens, bonus, best, Kc, Vc, seq_len, nkv, Pmax, row_bytes, seed, step,
                       excl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return run_sample_rows(base_logits, (int64_t)T * V, best, b, V, temperature, seed, step, 1, bonus,
                         static_cast<char*>(ws) + samp_offset(b, T), st, nullptr, 0,
                         mode == kReject ? excl : nullptr);
}

}  // namespace medusa
