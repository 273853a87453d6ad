// Per-head top-k shortlists, greedy root and float64 row sampling.
//
// aicassindra.com "Medusa deep dive", "From top-k heads to a sparse candidate
// tree": keep the top k_i tokens of head i.  Order: logit descending, equal
// logits by lower vocabulary index (a 64-bit key, see common.h).
//
// Selection is one launch, one workgroup per row (see topk_rows).
// The root row (head 0) takes k = 1 in greedy mode; in typical mode the root
// is drawn by sample_rows instead.
//
// sample_rows draws from softmax(x / T) in float64: e_i = exp((x_i - max)/T),
// the smallest i whose running sum (vocabulary order) exceeds u * sum e, with
// u from the SplitMix64 counter.  Each thread owns one contiguous slice; slice
// sums are scanned across the block, and the slice holding the crossing is
// rescanned serially.

#include "common.h"
#include "kernels.h"

namespace medusa {


__device__ __forceinline__ int row_k(const TopkArgs& a, int i) {
  if (i == 0) return a.root_mode == kGreedy ? 1 : 0;
  return a.k[i - 1];
}

// One workgroup (1024 threads) per row, threshold selection:
//   A. lanes stream their slice of the row (16-byte loads, a group issued
//      before use), form the 64-bit keys and keep them in registers (rows up
//      to 32768 entries; longer rows are re-read from L2 in step C) with the
//      lane's largest key;
//   B. tau = the k-th largest of the 1024 lane maxima: each wave takes its k
//      largest lane maxima (k rounds of a wave max below the previous pick,
//      shuffle butterflies, no barrier), wave 0 takes the k-th largest of the
//      16 x k results.  The k largest lane maxima are k distinct entries, so
//      the row's k-th largest key is >= tau: every top-k entry has key >= tau;
//   C. lanes append their keys >= tau to an LDS candidate list (about k
//      entries for continuous data);
//   D. wave 0 takes the k largest candidates, in order.
// If ties make the candidate list overflow its LDS capacity, step D instead
// runs k rounds of "largest key below the previous pick" over the whole row.
constexpr int kTopkThreads = 1024;
constexpr int kTopkKPT = 32;          // keys kept per lane (rows up to 32768 entries)
constexpr int kTopkCand = 2048;       // LDS candidate capacity

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

__global__ __launch_bounds__(kTopkThreads) void topk_rows(const float* __restrict__ logits,
                                                          TopkArgs a, int* __restrict__ root,
                                                          int* __restrict__ idx,
                                                          float* __restrict__ val) {
  const int row = blockIdx.x;                 // s*(K+1) + i
  const int s = row / (a.K + 1), i = row % (a.K + 1);
  const int k = row_k(a, i);
  const int tid = threadIdx.x, lane = tid & 63;
  __shared__ uint64_t red[kTopkThreads / 64];
  __shared__ uint64_t cand[kTopkCand];
  __shared__ int ncand;
  if (i > 0) {
    for (int r = k + tid; r < a.kmax; r += kTopkThreads) {
      const int64_t o = ((int64_t)s * a.K + (i - 1)) * a.kmax + r;
      idx[o] = -1;
      val[o] = -INFINITY;
    }
  }
  if (k == 0) return;
  const float* x = logits + (int64_t)row * a.V;
  const bool in_regs = (a.V & 3) == 0 && a.V <= kTopkKPT * kTopkThreads;

  // ---- A: keys (in registers when the row fits) and the lane maximum
  uint64_t keys[kTopkKPT];
  uint64_t lmax = 0;
  if (in_regs) {
    const int nv = a.V >> 2;
    f32x4 v[kTopkKPT / 4];
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
        const uint64_t kk = e < nv ? make_key(v[u][q], 4 * e + q) : 0ull;
        keys[4 * u + q] = kk;
        lmax = kk > lmax ? kk : lmax;
      }
    }
  } else {
    for (int e = tid; e < a.V; e += kTopkThreads) {
      const uint64_t kk = make_key(x[e], e);
      lmax = kk > lmax ? kk : lmax;
    }
  }
  // ---- B: tau = k-th largest lane maximum: each wave finds its k largest
  // lane maxima (wave-local rounds), wave 0 takes the k-th largest of those
  __shared__ uint64_t wtop[kTopkThreads / 64][kMaxK];
  __shared__ uint64_t tau_s;
  {
    const int wave = tid >> 6;
    uint64_t p = ~0ull;
    for (int r = 0; r < k; ++r) {
      const uint64_t b_ = wave_max_u64(lmax < p ? lmax : 0ull);
      p = b_;
      if (lane == 0) wtop[wave][r] = b_;
    }
  }
  __syncthreads();
  if (tid < 64) {
    constexpr int NW = kTopkThreads / 64;
    uint64_t p = ~0ull;
    for (int r = 0; r < k; ++r) {
      uint64_t b_ = 0;
      for (int j = lane; j < NW * k; j += 64) {
        const uint64_t v = wtop[j / k][j % k];
        if (v < p && v > b_) b_ = v;
      }
      p = wave_max_u64(b_);
    }
    if (lane == 0) tau_s = p;
  }
  __syncthreads();
  const uint64_t tau = tau_s;
  // ---- C: candidates >= tau
  if (tid == 0) ncand = 0;
  __syncthreads();
  if (in_regs) {
#pragma unroll
    for (int j = 0; j < kTopkKPT; ++j) {
      if (keys[j] >= tau && keys[j] != 0) {
        const int slot = atomicAdd(&ncand, 1);
        if (slot < kTopkCand) cand[slot] = keys[j];
      }
    }
  } else {
    for (int e = tid; e < a.V; e += kTopkThreads) {
      const uint64_t kk = make_key(x[e], e);
      if (kk >= tau) {
        const int slot = atomicAdd(&ncand, 1);
        if (slot < kTopkCand) cand[slot] = kk;
      }
    }
  }
  __syncthreads();
  const int nc = ncand;
  // ---- D: the k largest candidates in order
  if (nc <= kTopkCand) {
    if (threadIdx.x < 64) {
      uint64_t p = ~0ull;
      for (int r = 0; r < k; ++r) {
        uint64_t best = 0;
        for (int j = lane; j < nc; j += 64) {
          const uint64_t v = cand[j];
          if (v < p && v > best) best = v;
        }
        best = wave_max_u64(best);
        p = best;
        if (lane == 0) {
          if (i == 0) {
            root[s] = (int)key_index(best);
          } else {
            const int64_t o = ((int64_t)s * a.K + (i - 1)) * a.kmax + r;
            idx[o] = (int)key_index(best);
            val[o] = key_value(best);
          }
        }
      }
    }
  } else {
    // overflow (heavy ties): k rounds over the whole row
    uint64_t p = ~0ull;
    for (int r = 0; r < k; ++r) {
      uint64_t best = 0;
      if (in_regs) {
#pragma unroll
        for (int j = 0; j < kTopkKPT; ++j)
          if (keys[j] < p && keys[j] > best) best = keys[j];
      } else {
        for (int e = tid; e < a.V; e += kTopkThreads) {
          const uint64_t kk = make_key(x[e], e);
          if (kk < p && kk > best) best = kk;
        }
      }
      best = block_max_u64(best, red);
      p = best;
      if (tid == 0) {
        if (i == 0) {
          root[s] = (int)key_index(best);
        } else {
          const int64_t o = ((int64_t)s * a.K + (i - 1)) * a.kmax + r;
          idx[o] = (int)key_index(best);
          val[o] = key_value(best);
        }
      }
    }
  }
}

size_t topk_workspace(int b, int K, int V, int kmax) {
  (void)b; (void)K; (void)V; (void)kmax;
  return 0;
}

hipError_t run_topk(const float* logits, const TopkArgs& a, int* root, int* idx, float* val,
                    void* ws, hipStream_t st) {
  (void)ws;
  const int rows = a.b * (a.K + 1);
  hipLaunchKernelGGL(topk_rows, dim3(rows), dim3(kTopkThreads), 0, st, logits, a, root, idx, val);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.root_mode == kTypical)
    return run_sample_rows(logits, (int64_t)(a.K + 1) * a.V, nullptr, a.b, a.V, a.temperature,
                           a.seed, a.step, 0, root, st);
  return hipSuccess;
}

// ---------------------------------------------------------------- sampling
constexpr int kSampThreads = 1024;

__global__ __launch_bounds__(kSampThreads) void sample_rows(const float* __restrict__ base,
                                                            int64_t seq_stride,
                                                            const int* __restrict__ row_sel, int V,
                                                            float temperature, uint64_t seed,
                                                            uint64_t step, uint64_t draw,
                                                            int* __restrict__ out) {
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NW = kSampThreads / 64;
  const int rsel = row_sel ? row_sel[s] : 0;
  const float* x = base + (int64_t)s * seq_stride + (int64_t)rsel * V;
  __shared__ float smax[NW];
  __shared__ double ssum[NW];
  __shared__ int found;

  float m = -INFINITY;
  for (int e = tid; e < V; e += kSampThreads) m = fmaxf(m, x[e]);
  m = wave_max(m);
  if (lane == 0) smax[wave] = m;
  if (tid == 0) found = V - 1;
  __syncthreads();
  m = smax[0];
  for (int w = 1; w < NW; ++w) m = fmaxf(m, smax[w]);

  const double md = (double)m, td = (double)temperature;
  const int chunk = (V + kSampThreads - 1) / kSampThreads;
  const int lo = min(V, tid * chunk), hi = min(V, lo + chunk);
  double part = 0.0;
  for (int e = lo; e < hi; ++e) part += exp(((double)x[e] - md) / td);

  // block exclusive scan of the slice sums (thread order = vocabulary order)
  double incl = part;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    double y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) ssum[wave] = incl;
  __syncthreads();
  // Slice bounds are built so that thread t's end equals thread t+1's start
  // bit for bit (same additions in the same order); exactly one slice holds
  // the crossing.
  double wpre = 0.0, total = 0.0;
  for (int w = 0; w < NW; ++w) {
    if (w < wave) wpre = wpre + ssum[w];
    total = total + ssum[w];
  }
  const double prev_incl = __shfl_up(incl, 1, 64);
  const double excl = wpre + (lane > 0 ? prev_incl : 0.0);
  const double end = wpre + incl;
  const double u = counter_uniform(seed, step, (uint64_t)s, draw);
  const double target = u * total;
  if (excl <= target && end > target) {
    double run = 0.0;
    int pick = hi - 1;
    for (int e = lo; e < hi; ++e) {
      run += exp(((double)x[e] - md) / td);
      if (excl + run > target) {
        pick = e;
        break;
      }
    }
    found = pick;
  }
  __syncthreads();
  if (tid == 0) out[s] = found;
}

hipError_t run_sample_rows(const float* base, int64_t seq_stride, const int* row_sel, int b, int V,
                           float temperature, uint64_t seed, uint64_t step, uint64_t draw,
                           int* out, hipStream_t st) {
  hipLaunchKernelGGL(sample_rows, dim3(b), dim3(kSampThreads), 0, st, base, seq_stride, row_sel, V,
                     temperature, seed, step, draw, out);
  return hipGetLastError();
}

}  // namespace medusa
