// Per-head top-k shortlists, greedy root and float64 row sampling.
//
// aicassindra.com "Medusa deep dive", "From top-k heads to a sparse candidate
// tree": keep the top k_i tokens of head i.  Order: logit descending, equal
// logits by lower vocabulary index (a 64-bit key, see common.h).
//
// Selection is one launch, one workgroup per row (see topk_rows).
// The root row (head 0) takes k = 1 in greedy mode; in typical mode the root
// is drawn by the row sampler instead, and with a given root (the previous
// step's next token) root[] is an input.
//
// The row sampler (run_sample_rows) draws from softmax(x / T) in float64:
// e_i = exp((x_i - max)/T), the smallest i whose running sum (vocabulary
// order) exceeds u * sum e, with u from the SplitMix64 counter.  Slice sums
// come from many workgroups (sample_part); one workgroup per row then finds
// the slice holding the crossing and rescans it (sample_pick).

#include "common.h"
#include "kernels.h"

namespace medusa {


__device__ __forceinline__ int row_k(const TopkArgs& a, int i) {
  if (i == 0) return a.root_mode == kGreedy ? 1 : 0;
  return a.k[i - 1];
}

// One workgroup (1024 threads) per row, threshold selection:
//   A. lanes stream their slice of the row (16-byte loads issued before use;
//      rows up to 32768 entries stay in registers, longer rows are re-read
//      from L2 in step C) and keep their largest value with its lowest index;
//   B. each wave reduces its lanes' (value, index) keys to the wave maximum;
//      tau = the k-th largest of the 16 wave maxima.  Those k wave maxima are
//      k distinct entries of the row, so the row's k-th largest key is >= tau
//      and every top-k entry has key >= tau.  (With fewer than k non-empty
//      waves tau is 0 and every entry is a candidate.)
//   C. lanes append the keys >= tau of their entries to an LDS candidate list
//      (a float compare against tau's value filters first; about k to 3k
//      entries for continuous data);
//   D. each candidate's rank is the number of larger candidates (keys are
//      distinct), and candidates of rank < k write output slot rank.
// If ties make the candidate list overflow its LDS capacity (or it is long),
// step D instead runs k rounds of "largest key below the previous pick".
constexpr int kTopkThreads = 1024;
constexpr int kTopkKPT = 32;          // entries kept per lane (rows up to 32768 entries)
constexpr int kTopkCand = 2048;       // LDS candidate capacity
constexpr int kTopkRankMax = 1024;    // rank selection for up to this many candidates
static_assert(kTopkThreads >= kMaxT, "one thread per tree node");

__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NW = kTopkThreads / 64;
  v = wave_max_u64(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint64_t r = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = red[w] > r ? red[w] : r;
  return r;
}

// Tree tables of one sequence (fused with the shortlists, see topk_tree in
// run_topk): position ids for every node and, from sequence 0, the static
// parent / depth / ancestor tables.  Thread j handles node j (T <= the
// workgroup size); the parents were staged in LDS (tpar) and node j's depth
// in a register at the start of the kernel, so the ancestor walks read LDS.
__device__ void tree_common(const TreeDev& t, const TreeOut& o, int s, const int16_t* tpar,
                            int my_depth) {
  const int P = o.seq_len[s];
  const int j = threadIdx.x;
  if (j < t.T) {
    o.pos[(int64_t)s * t.T + j] = P + my_depth;
    if (s == 0) {
      o.parent[j] = tpar[j];
      o.depth[j] = my_depth;
      uint64_t w[kMaxAncWords] = {0, 0, 0, 0};
      for (int a = j; a >= 0; a = tpar[a]) w[a >> 6] |= 1ull << (a & 63);
      for (int q = 0; q < t.anc_words; ++q)
        o.anc[(int64_t)j * t.anc_words + q] = q < kMaxAncWords ? w[q] : 0;
    }
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_rows(const float* __restrict__ logits,
                                                          TopkArgs a, int* __restrict__ root,
                                                          int* __restrict__ idx,
                                                          float* __restrict__ val, TreeDev t,
                                                          TreeOut to) {
  constexpr int NW = kTopkThreads / 64;
  const int row = blockIdx.x;                 // s*(K+1) + i
  const int s = row / (a.K + 1), i = row % (a.K + 1);
  const int k = row_k(a, i);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ uint64_t red[NW];
  __shared__ uint64_t cand[kTopkCand];
  __shared__ int ncand;
  __shared__ uint64_t tau_s;
  if (i > 0) {
    for (int r = k + tid; r < a.kmax; r += kTopkThreads) {
      const int64_t o = ((int64_t)s * a.K + (i - 1)) * a.kmax + r;
      idx[o] = -1;
      val[o] = -INFINITY;
    }
  }
  const bool tree = to.tokens != nullptr;
  // this row's tree tables, read before the logits so that they arrive while
  // the row streams in: node tid's depth and rank, and the parents in LDS
  __shared__ int16_t tpar[kMaxT];
  int my_depth = -1, my_rank = 0;
  if (tree && tid < t.T) {
    tpar[tid] = t.parent[tid];
    my_depth = t.depth[tid];
    my_rank = t.rank[tid];
  }
  if (k == 0) {            // root row: drawn by the sampler (typical) or given
    if (tree && i == 0) {
      __syncthreads();     // tpar
      tree_common(t, to, s, tpar, my_depth);
      if (a.root_mode == kRootGiven && tid == 0) to.tokens[(int64_t)s * t.T] = root[s];
    }
    return;
  }
  if (tid == 0) ncand = 0;
  const float* x = logits + (int64_t)row * a.V;
  const bool vec = (a.V & 3) == 0;
  const bool in_regs = vec && a.V <= kTopkKPT * kTopkThreads;
  const int nv = a.V >> 2;

  // ---- A: the lane's largest value, lowest index among equals (entries in
  // index order: 16-byte group u*1024 + tid, then its 4 entries)
  f32x4 v[kTopkKPT / 4];
  float lv = -INFINITY;
  int li = -1;
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < kTopkKPT / 4; ++u) {
      const int e = u * kTopkThreads + tid;
      v[u] = e < nv ? *reinterpret_cast<const f32x4*>(x + 4 * e) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kTopkKPT / 4; ++u) {
      const int e = u * kTopkThreads + tid;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool take = e < nv && (li < 0 || v[u][q] > lv);
        lv = take ? v[u][q] : lv;
        li = take ? 4 * e + q : li;
      }
    }
  } else if (vec) {
    for (int e0 = tid; e0 < nv; e0 += 4 * kTopkThreads) {
      f32x4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * kTopkThreads;
        w[u] = e < nv ? *reinterpret_cast<const f32x4*>(x + 4 * e) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * kTopkThreads;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool take = e < nv && (li < 0 || w[u][q] > lv);
          lv = take ? w[u][q] : lv;
          li = take ? 4 * e + q : li;
        }
      }
    }
  } else {
    for (int e = tid; e < a.V; e += kTopkThreads) {
      const float y = x[e];
      const bool take = li < 0 || y > lv;
      lv = take ? y : lv;
      li = take ? e : li;
    }
  }

  // ---- B: tau = k-th largest wave maximum
  const uint64_t wm = wave_max_u64(li >= 0 ? make_key(lv, (uint32_t)li) : 0ull);
  if (lane == 0) red[wave] = wm;
  __syncthreads();
  if (tid < NW) {
    const uint64_t mine = red[tid];
    int rank = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) rank += red[w] > mine ? 1 : 0;
    // nonzero keys are distinct: exactly one wave maximum has rank k-1 when at
    // least k waves hold entries; otherwise tau = 0 (every entry a candidate)
    if (rank == k - 1 && mine != 0) tau_s = mine;
    if (tid == 0) {
      int nz = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) nz += red[w] != 0 ? 1 : 0;
      if (nz < k) tau_s = 0;
    }
  }
  __syncthreads();
  const uint64_t tau = tau_s;
  const float tv = tau ? key_value(tau) : -INFINITY;

  // ---- C: candidates (key >= tau implies value >= tau's value)
  auto offer = [&](float y, int e) {
    if (y >= tv) {
      const uint64_t kk = make_key(y, (uint32_t)e);
      if (kk >= tau) {
        const int slot = atomicAdd(&ncand, 1);
        if (slot < kTopkCand) cand[slot] = kk;
      }
    }
  };
  // Only a lane whose own largest value reaches tau's value can hold a
  // candidate (a handful of lanes for continuous data): the others skip the
  // pass, and with it the re-read of long rows.
  if (li >= 0 && lv >= tv) {
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < kTopkKPT / 4; ++u) {
        const int e = u * kTopkThreads + tid;
        if (e < nv) {
#pragma unroll
          for (int q = 0; q < 4; ++q) offer(v[u][q], 4 * e + q);
        }
      }
    } else if (vec) {
      for (int e = tid; e < nv; e += kTopkThreads) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(x + 4 * e);
#pragma unroll
        for (int q = 0; q < 4; ++q) offer(w[q], 4 * e + q);
      }
    } else {
      for (int e = tid; e < a.V; e += kTopkThreads) offer(x[e], e);
    }
  }
  __syncthreads();
  const int nc = ncand;

  __shared__ int res[kMaxK];
  auto emit = [&](int r, uint64_t key) {
    res[r] = (int)key_index(key);
    if (i == 0) {
      root[s] = (int)key_index(key);
    } else {
      const int64_t o = ((int64_t)s * a.K + (i - 1)) * a.kmax + r;
      idx[o] = (int)key_index(key);
      val[o] = key_value(key);
    }
  };
  // ---- D: rank of each candidate among the candidates
  if (nc <= kTopkRankMax) {
    if (tid < nc) {
      const uint64_t mine = cand[tid];
      int rank = 0;
      for (int j = 0; j < nc; ++j) rank += cand[j] > mine ? 1 : 0;
      if (rank < k) emit(rank, mine);
    }
  } else if (nc <= kTopkCand) {
    if (tid < 64) {
      uint64_t p = ~0ull;
      for (int r = 0; r < k; ++r) {
        uint64_t best = 0;
        for (int j = lane; j < nc; j += 64) {
          const uint64_t c = cand[j];
          if (c < p && c > best) best = c;
        }
        best = wave_max_u64(best);
        p = best;
        if (lane == 0) emit(r, best);
      }
    }
  } else {
    // overflow (heavy ties): k rounds over the whole row
    uint64_t p = ~0ull;
    for (int r = 0; r < k; ++r) {
      uint64_t best = 0;
      if (in_regs) {
#pragma unroll
        for (int u = 0; u < kTopkKPT / 4; ++u) {
          const int e = u * kTopkThreads + tid;
          if (e < nv) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint64_t kk = make_key(v[u][q], (uint32_t)(4 * e + q));
              if (kk < p && kk > best) best = kk;
            }
          }
        }
      } else {
        for (int e = tid; e < a.V; e += kTopkThreads) {
          const uint64_t kk = make_key(x[e], (uint32_t)e);
          if (kk < p && kk > best) best = kk;
        }
      }
      best = block_max_u64(best, red);
      p = best;
      if (tid == 0) emit(r, best);
    }
  }
  if (!tree) return;
  // ---- tree tokens: the nodes whose last rank lies in this head's shortlist
  __syncthreads();
  if (i == 0) {
    tree_common(t, to, s, tpar, my_depth);
    if (tid == 0) to.tokens[(int64_t)s * t.T] = res[0];
  } else if (my_depth == i) {
    to.tokens[(int64_t)s * t.T + tid] = res[my_rank];
  }
}

// The float64 sampler's slice partials (typical root draws).
size_t topk_workspace(int b, int K, int V, int kmax) {
  (void)K; (void)V; (void)kmax;
  return sample_workspace(b);
}

hipError_t run_topk(const float* logits, const TopkArgs& a, int* root, int* idx, float* val,
                    void* ws, hipStream_t st, const TreeDev* tree, const TreeOut* tree_out) {
  const int rows = a.b * (a.K + 1);
  TreeDev t{};
  TreeOut o{};
  if (tree) {
    t = *tree;
    o = *tree_out;
  }
  hipLaunchKernelGGL(topk_rows, dim3(rows), dim3(kTopkThreads), 0, st, logits, a, root, idx, val, t,
                     o);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.root_mode == kTypical)
    return run_sample_rows(logits, (int64_t)(a.K + 1) * a.V, nullptr, a.b, a.V, a.temperature,
                           a.seed, a.step, 0, root, ws, st, tree ? o.tokens : nullptr,
                           tree ? t.T : 0);
  return hipSuccess;
}

// ---------------------------------------------------------------- sampling
// Two launches per draw, so that a row's float64 exponentials spread over many
// CUs:
//   sample_part  - one workgroup per (row, slice): the row is cut into
//                  kSampSlices contiguous slices; slice j yields its float
//                  max m_j and s_j = sum exp((x_i - m_j) / T) in float64
//                  (the division taken as a product with 1/T).
//   sample_pick  - one workgroup per row: M = max m_j, c_j = s_j
//                  exp((m_j - M) / T) (the slice's share of the row's sum
//                  exp((x_i - M) / T)); the first slice whose running sum of
//                  c exceeds u * sum c is rescanned element by element with
//                  e_i = exp((x_i - M) / T), starting from the sum of the
//                  slices before it.  The pick is the first element whose
//                  running sum exceeds u * sum c; if rounding leaves none, the
//                  slice's last element.
// The running sums differ from a serial float64 sum only by rounding, so a
// sample can differ from the serial rule only when u * sum lies within a few
// ulps of a running sum.
// With an exclusion list (up to kSampExcl tokens per row, -1 padded) the draw
// is from the row with those tokens removed: their e_i leave their slices'
// shares and the total, and the rescan skips them.
constexpr int kSampThreads = 256;

struct SampPart {
  double m;   // slice max (a float value), -inf for an empty slice
  double s;   // sum of exp((x - m) / T) over the slice
};

__device__ __forceinline__ const float* samp_row(const float* base, int64_t seq_stride,
                                                 const int* row_sel, int V, int s) {
  const int rsel = row_sel ? row_sel[s] : 0;
  return base + (int64_t)s * seq_stride + (int64_t)rsel * V;
}

__global__ __launch_bounds__(kSampThreads) void sample_part(const float* __restrict__ base,
                                                            int64_t seq_stride,
                                                            const int* __restrict__ row_sel,
                                                            int V, float temperature,
                                                            SampPart* __restrict__ parts) {
  constexpr int NW = kSampThreads / 64;
  const int j = blockIdx.x % kSampSlices, s = blockIdx.x / kSampSlices;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Ls = (V + kSampSlices - 1) / kSampSlices;
  const int lo = min(V, j * Ls), hi = min(V, lo + Ls);
  const float* x = samp_row(base, seq_stride, row_sel, V, s);
  __shared__ float smax[NW];
  __shared__ double ssum[NW];

  float m = -INFINITY;
  for (int e = lo + tid; e < hi; e += kSampThreads) m = fmaxf(m, x[e]);
  m = wave_max(m);
  if (lane == 0) smax[wave] = m;
  __syncthreads();
  m = smax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) m = fmaxf(m, smax[w]);
  const double md = (double)m, rt = 1.0 / (double)temperature;
  double part = 0.0;
  for (int e = lo + tid; e < hi; e += kSampThreads) part += exp(((double)x[e] - md) * rt);
  part = wave_sum_d(part);
  if (lane == 0) ssum[wave] = part;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += ssum[w];
    parts[(int64_t)s * kSampSlices + j] = SampPart{lo < hi ? md : -(double)INFINITY, t};
  }
}

__global__ __launch_bounds__(kSampThreads) void sample_pick(const float* __restrict__ base,
                                                            int64_t seq_stride,
                                                            const int* __restrict__ row_sel,
                                                            int V, float temperature,
                                                            uint64_t seed, uint64_t step,
                                                            uint64_t draw,
                                                            const SampPart* __restrict__ parts,
                                                            const int* __restrict__ excl,
                                                            int* __restrict__ out,
                                                            int* __restrict__ out2,
                                                            int out2_stride) {
  static_assert(kSampSlices == 64, "one lane per slice");
  static_assert(kSampExcl <= 64, "one lane per excluded token");
  constexpr int NW = kSampThreads / 64;
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Ls = (V + kSampSlices - 1) / kSampSlices;
  const float* x = samp_row(base, seq_stride, row_sel, V, s);
  const double rt = 1.0 / (double)temperature;
  __shared__ int sh_j, found;
  __shared__ double sh_base, sh_target, sh_max;
  __shared__ double wsum[NW];
  __shared__ int sx[kSampExcl];

  if (tid < kSampExcl) {
    const int t = excl ? excl[(int64_t)s * kSampExcl + tid] : -1;
    sx[tid] = t >= 0 && t < V ? t : -1;
  }
  __syncthreads();
  auto excluded = [&](int e) {
    bool hit = false;
#pragma unroll
    for (int q = 0; q < kSampExcl; ++q) hit |= sx[q] == e;
    return hit;
  };
  if (wave == 0) {
    const SampPart p = parts[(int64_t)s * kSampSlices + lane];
    const double M = (double)wave_max((float)p.m);
    double c = p.m == -(double)INFINITY ? 0.0 : p.s * exp((p.m - M) * rt);
    if (excl) {
      // each excluded token's share leaves its slice (lane q holds token q)
      const int tq = lane < kSampExcl ? sx[lane] : -1;
      const double eq = tq >= 0 ? exp(((double)x[tq] - M) * rt) : 0.0;
#pragma unroll
      for (int q = 0; q < kSampExcl; ++q) {
        const int t = __shfl(tq, q, 64);
        const double e = __shfl(eq, q, 64);
        if (t >= 0 && lane == t / Ls) c -= e;
      }
      c = fmax(c, 0.0);
    }
    double incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    const double total = __shfl(incl, 63, 64);
    const double prev = __shfl_up(incl, 1, 64);
    const double excl = lane > 0 ? prev : 0.0;
    const double target = counter_uniform(seed, step, (uint64_t)s, draw) * total;
    const uint64_t over = __ballot(incl > target);
    const uint64_t live = __ballot(c > 0.0);
    // the first slice whose running sum passes the target; if rounding
    // leaves none, the last slice with any mass
    const int js = over ? __ffsll((long long)over) - 1
                        : (live ? 63 - __clzll((long long)live) : 0);
    if (lane == js) {
      sh_j = js;
      sh_base = excl;
      sh_target = target;
      sh_max = M;
    }
    if (lane == 0) found = -1;
  }
  __syncthreads();
  const int j = sh_j;
  const double b0 = sh_base, target = sh_target, md = sh_max;
  const int lo = min(V, j * Ls), hi = min(V, lo + Ls);
  // contiguous pieces of the slice in thread order = vocabulary order
  const int per = (hi - lo + kSampThreads - 1) / kSampThreads;
  const int tlo = min(hi, lo + tid * per), thi = min(hi, tlo + per);
  double part = 0.0;
  for (int e = tlo; e < thi; ++e)
    if (!excl || !excluded(e)) part += exp(((double)x[e] - md) * rt);
  double incl = part;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  // thread t's end and thread t+1's start come from the same additions, so
  // they are equal bit for bit and at most one thread brackets the target
  double wpre = 0.0;
  for (int w = 0; w < wave; ++w) wpre = wpre + wsum[w];
  const double prev = __shfl_up(incl, 1, 64);
  const double start = b0 + (wpre + (lane > 0 ? prev : 0.0));
  const double end = b0 + (wpre + incl);
  if (tlo < thi && start <= target && end > target) {
    double run = start;
    int pick = -1;
    for (int e = tlo; e < thi; ++e) {
      if (excl && excluded(e)) continue;
      run += exp(((double)x[e] - md) * rt);
      pick = e;
      if (run > target) break;
    }
    if (pick >= 0) found = pick;
  }
  __syncthreads();
  if (tid == 0) {
    int pick = found;
    if (pick < 0) {   // rounding left no bracket: the slice's last token still in play
      pick = max(lo, hi - 1);
      for (int e = hi - 1; e >= lo; --e)
        if (!excl || !excluded(e)) {
          pick = e;
          break;
        }
    }
    out[s] = pick;
    if (out2) out2[(int64_t)s * out2_stride] = pick;
  }
}

size_t sample_workspace(int b) { return (size_t)b * kSampSlices * sizeof(SampPart); }

hipError_t run_sample_rows(const float* base, int64_t seq_stride, const int* row_sel, int b, int V,
                           float temperature, uint64_t seed, uint64_t step, uint64_t draw, int* out,
                           void* ws, hipStream_t st, int* out2, int out2_stride, const int* excl) {
  SampPart* parts = static_cast<SampPart*>(ws);
  hipLaunchKernelGGL(sample_part, dim3((unsigned)b * kSampSlices), dim3(kSampThreads), 0, st, base,
                     seq_stride, row_sel, V, temperature, parts);
  hipLaunchKernelGGL(sample_pick, dim3(b), dim3(kSampThreads), 0, st, base, seq_stride, row_sel, V,
                     temperature, seed, step, draw, parts, excl, out, out2, out2_stride);
  return hipGetLastError();
}

}  // namespace medusa
