// Per-head top-k shortlists, greedy root and float64 row sampling.
//
// aicassindra.com "Medusa deep dive", "From top-k heads to a sparse candidate
// tree": keep the top k_i tokens of head i.  Order: logit descending, equal
// logits by lower vocabulary index (a 64-bit key, see common.h).
//
// Selection is two launches:
//   1. topk_chunk: grid (chunks, rows).  Each lane streams its slice of a
//      vocabulary chunk with 16-byte loads and keeps a sorted register list of
//      its KM best keys (a new key is compared with the list's last entry and
//      usually rejected).  The 64 lists of a wave are merged by k rounds of a
//      wave-wide max (shuffle butterfly) in which the lane holding the winner
//      (found by ballot) pops its head; the 4 wave results are staged in LDS
//      and merged by one wave the same way.
//   2. topk_merge: one wave per row merges the chunk results (k rounds of
//      "largest key below the previous pick") and writes indices and values.
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

constexpr int kTopkChunk = 4096;   // vocabulary entries per workgroup in phase 1

template <int KM>
__device__ __forceinline__ void list_insert(uint64_t (&lst)[KM], uint64_t key) {
  if (key <= lst[KM - 1]) return;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    uint64_t hi = key > lst[j] ? key : lst[j];
    uint64_t lo = key > lst[j] ? lst[j] : key;
    lst[j] = hi;
    key = lo;
  }
}

// k rounds of wave max over the lanes' list heads; results in out[0..k).
template <int KM>
__device__ __forceinline__ void wave_merge_lists(uint64_t (&lst)[KM], int k, uint64_t* out) {
  const int lane = threadIdx.x & 63;
  for (int r = 0; r < k; ++r) {
    uint64_t head = lst[0];
    uint64_t best = wave_max_u64(head);
    uint64_t mask = __ballot(head == best && best != 0);
    int winner = mask ? (__ffsll((unsigned long long)mask) - 1) : -1;
    if (lane == winner) {
#pragma unroll
      for (int j = 0; j < KM - 1; ++j) lst[j] = lst[j + 1];
      lst[KM - 1] = 0;
    }
    if (lane == 0) out[r] = best;
  }
}

__device__ __forceinline__ int row_k(const TopkArgs& a, int i) {
  if (i == 0) return a.root_mode == kGreedy ? 1 : 0;
  return a.k[i - 1];
}

template <int KM>
__global__ __launch_bounds__(256) void topk_chunk(const float* __restrict__ logits, TopkArgs a,
                                                  uint64_t* __restrict__ ws, int nchunks) {
  const int row = blockIdx.y;                 // s*(K+1) + i
  const int i = row % (a.K + 1);
  const int k = row_k(a, i);
  const int c = blockIdx.x;
  uint64_t* out = ws + ((int64_t)row * nchunks + c) * KM;
  if (k == 0) return;
  const float* x = logits + (int64_t)row * a.V;
  const int lo = c * kTopkChunk, hi = min(a.V, lo + kTopkChunk);

  uint64_t lst[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) lst[j] = 0;
  if ((a.V & 3) == 0) {
    for (int e = lo + 4 * threadIdx.x; e < hi; e += 4 * 256) {
      f32x4 v = *reinterpret_cast<const f32x4*>(x + e);
      list_insert<KM>(lst, make_key(v[0], e));
      list_insert<KM>(lst, make_key(v[1], e + 1));
      list_insert<KM>(lst, make_key(v[2], e + 2));
      list_insert<KM>(lst, make_key(v[3], e + 3));
    }
  } else {
    for (int e = lo + threadIdx.x; e < hi; e += 256) list_insert<KM>(lst, make_key(x[e], e));
  }
  __shared__ uint64_t wres[4][KM];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  wave_merge_lists<KM>(lst, k, wres[wave]);
  __syncthreads();
  if (wave == 0) {
    // lanes 0..4k-1 hold one candidate each
    uint64_t one[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) one[j] = 0;
    if (lane < 4 * k) one[0] = wres[lane / k][lane % k];
    uint64_t res[KM];
    wave_merge_lists<KM>(one, k, res);
    if (lane == 0)
      for (int r = 0; r < KM; ++r) out[r] = r < k ? res[r] : 0;
  }
}

template <int KM>
__global__ __launch_bounds__(64) void topk_merge(const uint64_t* __restrict__ ws, TopkArgs a,
                                                 int nchunks, int* __restrict__ root,
                                                 int* __restrict__ idx, float* __restrict__ val) {
  const int row = blockIdx.x;
  const int s = row / (a.K + 1), i = row % (a.K + 1);
  const int k = row_k(a, i);
  const int lane = threadIdx.x;
  const uint64_t* cand = ws + (int64_t)row * nchunks * KM;
  const int ncand = nchunks * KM;
  uint64_t prev = ~0ull;
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
    for (int j = lane; j < ncand; j += 64) {
      uint64_t v = cand[j];
      if (v < prev && v > best) best = v;
    }
    best = wave_max_u64(best);
    prev = best;
    if (lane == 0) {
      if (i == 0) {
        root[s] = (int)key_index(best);
      } else {
        int64_t o = ((int64_t)s * a.K + (i - 1)) * a.kmax + r;
        idx[o] = (int)key_index(best);
        val[o] = key_value(best);
      }
    }
  }
  if (i > 0) {
    for (int r = k + lane; r < a.kmax; r += 64) {
      int64_t o = ((int64_t)s * a.K + (i - 1)) * a.kmax + r;
      idx[o] = -1;
      val[o] = -INFINITY;
    }
  }
}

static int km_for(int kmax) { return kmax <= 4 ? 4 : (kmax <= 8 ? 8 : 16); }

size_t topk_workspace(int b, int K, int V, int kmax) {
  const int nchunks = (V + kTopkChunk - 1) / kTopkChunk;
  return (size_t)b * (K + 1) * nchunks * km_for(kmax) * sizeof(uint64_t);
}

hipError_t run_topk(const float* logits, const TopkArgs& a, int* root, int* idx, float* val,
                    void* ws, hipStream_t st) {
  const int nchunks = (a.V + kTopkChunk - 1) / kTopkChunk;
  const int rows = a.b * (a.K + 1);
  uint64_t* w = static_cast<uint64_t*>(ws);
  dim3 g1(nchunks, rows);
  switch (km_for(a.kmax)) {
    case 4:
      hipLaunchKernelGGL(topk_chunk<4>, g1, dim3(256), 0, st, logits, a, w, nchunks);
      hipLaunchKernelGGL(topk_merge<4>, dim3(rows), dim3(64), 0, st, w, a, nchunks, root, idx, val);
      break;
    case 8:
      hipLaunchKernelGGL(topk_chunk<8>, g1, dim3(256), 0, st, logits, a, w, nchunks);
      hipLaunchKernelGGL(topk_merge<8>, dim3(rows), dim3(64), 0, st, w, a, nchunks, root, idx, val);
      break;
    default:
      hipLaunchKernelGGL(topk_chunk<16>, g1, dim3(256), 0, st, logits, a, w, nchunks);
      hipLaunchKernelGGL(topk_merge<16>, dim3(rows), dim3(64), 0, st, w, a, nchunks, root, idx,
                         val);
      break;
  }
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
