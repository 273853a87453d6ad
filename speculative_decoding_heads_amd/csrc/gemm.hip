// Medusa heads and LM projection: C[m, n] = sum_k X[m, k] * W[n, k].
//
// Head formula (aicassindra.com "Medusa deep dive", "The heads are residual
// blocks, not linear layers"): head_i(h) = LMproj(h + SiLU(W_i h)); the heads
// run off one hidden state as a few small matmuls.  Both products here are
// "NT" GEMMs: activations X [M, K] and weights W [N, K] are row-major with the
// contraction dimension contiguous.
//
//   * W_i stage: X = h [b, H], W = all heads stacked [K*H, H]; epilogue
//     u = h + SiLU(z) stored in bf16 (or f32).
//   * LM stage: X = u [b*(K+1), H] (or the attention output on the verify
//     pass), W = LMproj [V, H]; fp32 logits.
//
// bf16 kernels use v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  W rows
// are the MFMA "A" rows, X rows the "B" columns, so each lane ends up with 4
// consecutive n of one output row (one 16-byte store of logits).
//
// bf16 kernels:
//   gemm_skinny : M <= 16 with fewer than 30720 weight rows (M <= 32 for a
//                 single head, N = H).  HBM-bound weight stream.  A workgroup
//                 owns 16*NB weight rows; its 4 waves split K and reduce
//                 through LDS.  With 32 rows and K > 4096 both operands go
//                 global -> registers (X is tiny and stays in L2; each lane
//                 loads 64 contiguous bytes per row per step); with K <= 4096
//                 the weights stream by LDS DMA and X sits in registers
//                 (gemm_skinny_dma); with 16 rows both operands stream by LDS
//                 DMA (gemm_skinny1_dma).
//   gemm_tiled  : the other M <= 80 cases (and heads with larger M).  A
//                 workgroup of 8 waves (4 when there are too few weight rows to
//                 give every CU a 128-row tile) owns BM = 16*MB activation rows
//                 (staged in LDS once per K chunk and shared by all waves:
//                 re-reading X per wave from L2 costs more than the weights) and
//                 16*NBW weight rows per wave (direct loads).  Each workgroup
//                 starts its K walk at its own chunk, so the workgroups do not
//                 all read the same slice of X at once.  Tiles are mapped to
//                 XCDs so that the M-tiles of one weight tile run on one XCD.
//   gemm_dma    : gemm_tiled's 8-wave logits shapes (at most 80 rows over a
//                 wide vocabulary: the heads' LM pass, the batch-1 verify
//                 rows) and its 8/10-wave heads shapes of at most 16 rows: the
//                 same tile and MFMA order, with both operands streamed global
//                 -> LDS by DMA (see below).
//   gemm_ring   : M > 80, MFMA-bound (see below).
// One f32 kernel (tiny fp32 workload): one wave per weight row.

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace medusa {

// ---------------------------------------------------------------- epilogues
struct EpiLogits {
  float* C;
  int64_t ldc;
  int M, N;
  __device__ __forceinline__ void store4(int m, int n, f32x4 v) const {
    if (m >= M || n >= N) return;
    float* p = C + (int64_t)m * ldc + n;
    if (n + 3 < N && ((((uintptr_t)p) & 15) == 0)) {
      *reinterpret_cast<f32x4*>(p) = v;
    } else {
      for (int i = 0; i < 4 && n + i < N; ++i) p[i] = v[i];
    }
  }
  __device__ __forceinline__ void store1(int m, int n, float v) const {
    if (m < M && n < N) C[(int64_t)m * ldc + n] = v;
  }
  __device__ __forceinline__ void copy_base(int, int) const {}
};

// Logits plus the acceptance partial of every (row, weight tile): the argmax
// key (greedy) or the online softmax statistics of logits / temperature
// (typical), so acceptance never re-reads the logits for them.  Partials are
// [rows][ntiles]; header = {ntiles, typical, rows}, written by workgroup 0.
struct EpiLogitsStats : EpiLogits {
  bool typical;
  float inv_temp;
  int ntiles;
  int* header;
  uint64_t* pkey;
  RowStat* pstat;
  // These logits are large (133 MB at 1040 x 32000) and acceptance reads only
  // a few values of each row (the statistics come from the partials), so they
  // are stored non-temporally: as ordinary stores they stay in the caches as
  // dirty lines whose write-back then competes with the next step's weight
  // streams (measured at 7B batch 16: heads 37 -> 33 us, heads' LM pass
  // 67 -> 58 us, this GEMM level; level at the 128k workload).
  __device__ __forceinline__ void store4(int m, int n, f32x4 v) const {
    if (m >= M || n >= N) return;
    float* p = C + (int64_t)m * ldc + n;
    if (n + 3 < N && ((((uintptr_t)p) & 15) == 0)) {
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
    } else {
      for (int i = 0; i < 4 && n + i < N; ++i) __builtin_nontemporal_store(v[i], p + i);
    }
  }
  __device__ __forceinline__ void write_part(int row, int tile, const RowPart& p) const {
    const int64_t o = (int64_t)row * ntiles + tile;
    if (typical) pstat[o] = RowStat{p.m, p.s, p.t, 0.f};
    else pkey[o] = p.key;
  }
  __device__ __forceinline__ void write_header() const {
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      header[kHdrTiles] = ntiles;
      header[kHdrKind] = typical ? 1 : 0;
      header[kHdrRows] = M;
      header[kHdrCols] = N;
      header[kHdrInvTemp] = __float_as_int(inv_temp);
      header[kHdrMagic] = kPartsMagic;
    }
  }
};
template <class Epi> struct HasParts : std::false_type {};
template <> struct HasParts<EpiLogitsStats> : std::true_type {};
template <class Epi> struct IsLogits : std::is_base_of<EpiLogits, Epi> {};

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

// u[m, base + i, o] = x[m, o] + SiLU(z[m, i*H + o])   (n = i*H + o)
template <typename T>
struct EpiHeads {
  T* U;                 // [M, R, H]
  const T* X;           // [M, ldx]
  int64_t ldx;
  int H, R, base, M, N;
  __device__ __forceinline__ void store1(int m, int n, float z) const {
    if (m >= M || n >= N) return;
    int i = n / H, o = n - i * H;
    float x;
    if constexpr (sizeof(T) == 2) x = bf16_to_f32(X[(int64_t)m * ldx + o]);
    else x = X[(int64_t)m * ldx + o];
    float u = x + silu_f(z);
    T* p = U + ((int64_t)m * R + base + i) * H + o;
    if constexpr (sizeof(T) == 2) *p = f32_to_bf16(u);
    else *p = u;
  }
  __device__ __forceinline__ void store4(int m, int n, f32x4 v) const {
    if (m >= M || n >= N) return;
    if constexpr (sizeof(T) == 2) {
      if (n + 3 < N && (H & 3) == 0) {       // 4 consecutive o inside one head
        int i = n / H, o = n - i * H;
        uint2 xw = *reinterpret_cast<const uint2*>(X + (int64_t)m * ldx + o);
        float u0 = bf16_lo(xw.x) + silu_f(v[0]);
        float u1 = bf16_hi(xw.x) + silu_f(v[1]);
        float u2 = bf16_lo(xw.y) + silu_f(v[2]);
        float u3 = bf16_hi(xw.y) + silu_f(v[3]);
        uint2 out;
        out.x = pack_bf16x2(u0, u1);
        out.y = pack_bf16x2(u2, u3);
        *reinterpret_cast<uint2*>(U + ((int64_t)m * R + base + i) * H + o) = out;
        return;
      }
    }
    for (int j = 0; j < 4; ++j) store1(m, n + j, v[j]);
  }
  // slot 0 of u is x itself (the base head): the workgroups whose weight rows
  // fall in [0, H) also copy x[:, n_begin .. n_end) there.
  __device__ __forceinline__ void copy_base(int n_begin, int n_end) const {
    if (!base || n_begin >= H) return;
    const int w = min(n_end, H) - n_begin;
    for (int e = threadIdx.x; e < M * w; e += blockDim.x) {
      const int m = e / w, o = n_begin + e - m * w;
      U[(int64_t)m * R * H + o] = X[(int64_t)m * ldx + o];
    }
  }
};

// ---------------------------------------------------------------- MTP layer epilogues
// One transformer layer per MTP head, its GEMMs batched over the heads
// (blockIdx.y = head).  Columns arrive four at a time (n % 4 == 0, N % 4 == 0).
// q | k | v of the current position: q -> Q [heads, M, nqd]; k, v -> the
// head's cache [heads, M, nkv, Pmax, d] at slot seq_len[m] (nothing is
// written for a sequence whose slot lies outside the cache).
struct EpiQKV {
  uint16_t* Q;
  uint16_t* Kc;
  uint16_t* Vc;
  const int* seq_len;
  int nqd, nkvd, d, Pmax, M, N;
  __device__ __forceinline__ void store4(int m, int n, f32x4 v) const {
    if (m >= M || n >= N) return;
    const int hd = blockIdx.y;
    uint2 w;
    w.x = pack_bf16x2(v[0], v[1]);
    w.y = pack_bf16x2(v[2], v[3]);
    if (n < nqd) {
      *reinterpret_cast<uint2*>(Q + ((int64_t)hd * M + m) * nqd + n) = w;
      return;
    }
    int c = n - nqd;
    uint16_t* C = Kc;
    if (c >= nkvd) {
      c -= nkvd;
      C = Vc;
    }
    const int P = seq_len[m];
    if (P < 0 || P >= Pmax) return;
    const int g = c / d, e = c - g * d;
    const int nkv = nkvd / d;
    *reinterpret_cast<uint2*>(C + ((((int64_t)hd * M + m) * nkv + g) * Pmax + P) * d + e) = w;
  }
  __device__ __forceinline__ void copy_base(int, int) const {}
};
// out = bf16(R + z): O at O + head * so + m * ldo + n, R likewise (sr = 0: one
// residual for every head).
struct EpiResid {
  uint16_t* O;
  const uint16_t* R;
  int64_t so, ldo, sr, ldr;
  int M, N;
  __device__ __forceinline__ void store4(int m, int n, f32x4 v) const {
    if (m >= M || n >= N) return;
    const int hd = blockIdx.y;
    const uint2 r = *reinterpret_cast<const uint2*>(R + hd * sr + (int64_t)m * ldr + n);
    uint2 w;
    w.x = pack_bf16x2(bf16_lo(r.x) + v[0], bf16_hi(r.x) + v[1]);
    w.y = pack_bf16x2(bf16_lo(r.y) + v[2], bf16_hi(r.y) + v[3]);
    *reinterpret_cast<uint2*>(O + hd * so + (int64_t)m * ldo + n) = w;
  }
  __device__ __forceinline__ void copy_base(int, int) const {}
};
// SwiGLU on weight rows interleaved (gate_j, up_j) = rows (2j, 2j + 1):
// out[j] = bf16(SiLU(gate_j) * up_j) at O + head * so + m * ldo.
struct EpiSwiGLU {
  uint16_t* O;
  int64_t so, ldo;
  int M, N;
  __device__ __forceinline__ void store4(int m, int n, f32x4 v) const {
    if (m >= M || n >= N) return;
    const int hd = blockIdx.y;
    const float a = v[0] / (1.0f + expf(-v[0])) * v[1];
    const float b = v[2] / (1.0f + expf(-v[2])) * v[3];
    *reinterpret_cast<uint32_t*>(O + hd * so + (int64_t)m * ldo + (n >> 1)) = pack_bf16x2(a, b);
  }
  __device__ __forceinline__ void copy_base(int, int) const {}
};

// ---------------------------------------------------------------- skinny bf16
// grid.x = ceil(N / (16*NB)); block = 256 (4 waves splitting K in 128-chunks).
// grid.y = independent problems of the same shape (X, W advanced by bsx, bsw
// elements per problem; the epilogue reads blockIdx.y for its outputs).
template <int NB, int MB, class Epi>
__global__ __launch_bounds__(256) void gemm_skinny_bf16(const uint16_t* __restrict__ X,
                                                        int64_t ldx, int M,
                                                        const uint16_t* __restrict__ W,
                                                        int N, int Kd, Epi epi, int64_t bsx,
                                                        int64_t bsw) {
  X += blockIdx.y * bsx;
  W += blockIdx.y * bsw;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int n0 = blockIdx.x * 16 * NB;
  const int nchunks = Kd >> 7;

  const uint16_t* wp[NB];
  const uint16_t* xp[MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int n = min(n0 + 16 * nb + r16, N - 1);
    wp[nb] = W + (int64_t)n * Kd + 32 * g4;
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    int m = min(16 * mb + r16, M - 1);
    xp[mb] = X + (int64_t)m * ldx + 32 * g4;
  }

  f32x4 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Two register stages used alternately (no copies between them), so the
  // next chunk's loads stay in flight while the current chunk is multiplied.
  uint4 wa[NB][4], xa[MB][4], wb[NB][4], xb[MB][4];
  auto load = [&](int c, uint4 (&w)[NB][4], uint4 (&xv)[MB][4]) {
    const int k0 = c << 7;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int s = 0; s < 4; ++s) w[nb][s] = ldg16(wp[nb] + k0 + 8 * s);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int s = 0; s < 4; ++s) xv[mb][s] = ldg16(xp[mb] + k0 + 8 * s);
  };
  auto mma = [&](const uint4 (&w)[NB][4], const uint4 (&xv)[MB][4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = mfma16x16x32(w[nb][s], xv[mb][s], acc[nb][mb]);
  };
  // Waves take whole pairs of 128-wide chunks, so the two-stage body below has
  // no branch: a load under a branch would make the compiler wait for every
  // outstanding load before the next multiply (and it would sink the second
  // stage's loads into that branch).  The next pair's first chunk is always
  // prefetched (clamped at the end; a repeated chunk hits L2).  An odd last
  // chunk is done on its own by wave 0.
  const int npairs = nchunks >> 1;
  const int p_begin = (npairs * wave) >> 2, p_end = (npairs * (wave + 1)) >> 2;
  if (p_begin < p_end) {
    const int c_last = 2 * p_end - 1;
    load(2 * p_begin, wa, xa);
    for (int c = 2 * p_begin; c < 2 * p_end; c += 2) {
      // scheduling barriers keep each stage's loads issued before the other
      // stage's multiplies (issue is in order: a load placed after a
      // dependent MFMA chain would leave the memory pipe idle meanwhile)
      load(c + 1, wb, xb);
      __builtin_amdgcn_sched_barrier(0);
      mma(wa, xa);
      __builtin_amdgcn_sched_barrier(0);
      load(min(c + 2, c_last), wa, xa);
      __builtin_amdgcn_sched_barrier(0);
      mma(wb, xb);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if ((nchunks & 1) && wave == 0) {
    load(nchunks - 1, wb, xb);
    mma(wb, xb);
  }

  // cross-wave reduction of the 4 K-partials
  __shared__ f32x4 red[4][NB * MB][64];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[wave][nb * MB + mb][lane] = acc[nb][mb];
  __syncthreads();
  for (int p = wave; p < NB * MB; p += 4) {
    f32x4 v = red[0][p][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      f32x4 t = red[w][p][lane];
      v[0] += t[0]; v[1] += t[1]; v[2] += t[2]; v[3] += t[3];
    }
    const int nb = p / MB, mb = p - nb * MB;
    epi.store4(16 * mb + r16, n0 + 16 * nb + 4 * g4, v);
  }
  epi.copy_base(n0, n0 + 16 * NB);
}

// ---------------------------------------------------------------- skinny bf16 by LDS DMA
// gemm_skinny_bf16<2, 1> (32 weight rows per workgroup, 4 waves splitting K
// in whole pairs of 128-wide chunks, the same chunk order and LDS reduction,
// so the same outputs bit for bit) with the weights streamed global -> LDS by
// DMA with the non-temporal hint (read once per step) into a 2-deep ring per
// wave, and each wave's activation rows (at most 8 chunks: K <= 4096) held in
// registers for the whole call.  The waves never wait on each other before
// the reduction.  A ring slot holds the 32 rows of one chunk, row-major with
// 16-byte pieces XOR-swizzled by row; each DMA issue covers four whole rows.
template <class Epi>
__global__ __launch_bounds__(256) void gemm_skinny_dma_bf16(const uint16_t* __restrict__ X,
                                                            int64_t ldx, int M,
                                                            const uint16_t* __restrict__ W,
                                                            int N, int Kd, Epi epi, int64_t bsx,
                                                            int64_t bsw) {
  constexpr int NB = 2, LDSROW = 128, MAXC = 8;
  X += blockIdx.y * bsx;
  W += blockIdx.y * bsw;
  auto xsw = [](int r) { return (r & 3) | ((r & 4) << 1); };
  __shared__ __attribute__((aligned(16))) uint16_t wring[4][2][16 * NB * LDSROW];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int n0 = blockIdx.x * 16 * NB;
  const int nchunks = Kd >> 7;
  const int npairs = nchunks >> 1;
  const int p_begin = (npairs * wave) >> 2, p_end = (npairs * (wave + 1)) >> 2;
  const int c0 = 2 * p_begin, nc = 2 * (p_end - p_begin);   // this wave's chunks, nc <= MAXC

  // the activation fragments of all of this wave's chunks (indices clamped,
  // so no load sits under a branch)
  uint4 xr[MAXC][4];
  const uint16_t* xp = X + (int64_t)min(r16, M - 1) * ldx + 32 * g4;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int c = min(c0 + min(j, max(nc - 1, 0)), nchunks - 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) xr[j][s] = ldg16(xp + (c << 7) + 8 * s);
  }
  const uint16_t* wsrc[4 * NB];
#pragma unroll
  for (int u = 0; u < 4 * NB; ++u) {
    const int row = 4 * u + (lane >> 4);
    wsrc[u] = W + (int64_t)min(n0 + row, N - 1) * Kd + 8 * ((lane & 15) ^ xsw(row));
  }
  const uint32_t rl = lds_u32(&wring[wave][0][0]);
  auto issue = [&](int c, int slot) {
    const uint32_t base = rl + (uint32_t)(slot * 16 * NB * LDSROW * 2);
#pragma unroll
    for (int u = 0; u < 4 * NB; ++u)
      dma16_nt(wsrc[u] + (c << 7), __builtin_amdgcn_readfirstlane(base + (uint32_t)(u * 1024)));
  };

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int sw = xsw(r16);
  if (nc > 0) issue(c0, 0);
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    if (j < nc) {                                   // uniform
      if (j + 1 < nc) {
        // the slot chunk j+1 fills was read by chunk j-1: those LDS reads are done
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue(c0 + j + 1, (j + 1) & 1);
        vm_wait<4 * NB>();                          // chunk j landed (j+1 may be in flight)
      } else {
        vm_wait<0>();
      }
      const uint16_t* wb = &wring[wave][j & 1][0];
      uint4 w[NB][4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int row = 16 * nb + r16;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          w[nb][s] = *reinterpret_cast<const uint4*>(wb + row * LDSROW + 8 * ((4 * g4 + s) ^ sw));
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma16x16x32(w[nb][s], xr[j][s], acc[nb]);
    }
  }

  // cross-wave reduction of the 4 K-partials, as in gemm_skinny_bf16
  __shared__ f32x4 red[4][NB][64];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) red[wave][nb][lane] = acc[nb];
  __syncthreads();
  for (int p = wave; p < NB; p += 4) {
    f32x4 v = red[0][p][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      f32x4 t = red[w][p][lane];
      v[0] += t[0]; v[1] += t[1]; v[2] += t[2]; v[3] += t[3];
    }
    epi.store4(r16, n0 + 16 * p + 4 * g4, v);
  }
  epi.copy_base(n0, n0 + 16 * NB);
}

// gemm_skinny_bf16<1, MB> (16 weight rows per workgroup: the single-head
// GEMMs, N = H) with both operands streamed global -> LDS by DMA through a
// 2-deep ring per wave: K may be long (11008), so the activation rows are
// not held in registers.  The waves split K in whole pairs of 128-wide chunks
// (wave 0 also takes an odd last chunk), in the same order as the register
// kernel, with the same MFMA order and reduction: the same outputs bit for
// bit.  A slot holds the chunk's 16 weight rows and then its 16 MB activation
// rows (clamped to M - 1), row-major, 16-byte pieces XOR-swizzled by row;
// weights with the non-temporal hint (read once), activations without.
template <int MB, class Epi>
__global__ __launch_bounds__(256) void gemm_skinny1_dma_bf16(const uint16_t* __restrict__ X,
                                                             int64_t ldx, int M,
                                                             const uint16_t* __restrict__ W,
                                                             int N, int Kd, Epi epi, int64_t bsx,
                                                             int64_t bsw) {
  constexpr int LDSROW = 128, ROWS = 16 + 16 * MB, NU = ROWS / 4;   // 1 KB units per chunk
  X += blockIdx.y * bsx;
  W += blockIdx.y * bsw;
  auto xsw = [](int r) { return (r & 3) | ((r & 4) << 1); };
  __shared__ __attribute__((aligned(16))) uint16_t wring[4][2][ROWS * LDSROW];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int nchunks = Kd >> 7;
  const int npairs = nchunks >> 1;
  const int p_begin = (npairs * wave) >> 2, p_end = (npairs * (wave + 1)) >> 2;
  const int c0 = 2 * p_begin;
  const bool odd = (nchunks & 1) && wave == 0;
  const int nc = 2 * (p_end - p_begin) + (odd ? 1 : 0);   // this wave's chunks
  auto chunk = [&](int j) { return j < 2 * (p_end - p_begin) ? c0 + j : nchunks - 1; };

  // unit u: rows 4u..4u+3 of the slot (weights first, then activations)
  const uint16_t* src[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int row = 4 * u + (lane >> 4);
    const int part = (lane & 15) ^ xsw(row);
    src[u] = row < 16 ? W + (int64_t)min(n0 + row, N - 1) * Kd + 8 * part
                      : X + (int64_t)min(row - 16, M - 1) * ldx + 8 * part;
  }
  const uint32_t rl = lds_u32(&wring[wave][0][0]);
  auto issue = [&](int c, int slot) {
    const uint32_t base = rl + (uint32_t)(slot * ROWS * LDSROW * 2);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const uint32_t l = __builtin_amdgcn_readfirstlane(base + (uint32_t)(u * 1024));
      if (u < 4) dma16_nt(src[u] + (c << 7), l);
      else dma16(src[u] + (c << 7), l);
    }
  };

  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int sw = xsw(r16);
  if (nc > 0) issue(chunk(0), 0);
  for (int j = 0; j < nc; ++j) {
    if (j + 1 < nc) {
      // the slot chunk j+1 fills was read by chunk j-1: those LDS reads are done
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(chunk(j + 1), (j + 1) & 1);
      vm_wait<NU>();                                 // chunk j landed (j+1 may be in flight)
    } else {
      vm_wait<0>();
    }
    const uint16_t* sb = &wring[wave][j & 1][0];
    uint4 w[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      w[s] = *reinterpret_cast<const uint4*>(sb + r16 * LDSROW + 8 * ((4 * g4 + s) ^ sw));
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint4 xv = *reinterpret_cast<const uint4*>(
            sb + (16 + 16 * mb + r16) * LDSROW + 8 * ((4 * g4 + s) ^ sw));
        acc[mb] = mfma16x16x32(w[s], xv, acc[mb]);
      }
  }

  // cross-wave reduction of the 4 K-partials, as in gemm_skinny_bf16
  __shared__ f32x4 red[4][MB][64];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
  __syncthreads();
  for (int p = wave; p < MB; p += 4) {
    f32x4 v = red[0][p][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      f32x4 t = red[w][p][lane];
      v[0] += t[0]; v[1] += t[1]; v[2] += t[2]; v[3] += t[3];
    }
    epi.store4(16 * p + r16, n0 + 4 * g4, v);
  }
  epi.copy_base(n0, n0 + 16);
}

// ---------------------------------------------------------------- tiled bf16
// Tile index t -> (n tile, m tile) with all m tiles of one n tile adjacent on
// one XCD (workgroups are dispatched round-robin over the 8 XCDs).
__device__ __forceinline__ int xcd_tile(int b, int total) {
  const int x = b & 7, j = b >> 3;
  const int q = total >> 3, r = total & 7;
  return x * q + min(x, r) + j;
}

template <int MB, int NBW, class Epi, int NWAVES = 4>
__global__ __launch_bounds__(64 * NWAVES) void gemm_tiled_bf16(const uint16_t* __restrict__ X,
                                                               int64_t ldx, int M,
                                                               const uint16_t* __restrict__ W,
                                                               int N, int Kd, int ntm, Epi epi,
                                                               bool rev, int64_t bsx,
                                                               int64_t bsw) {
  X += blockIdx.y * bsx;                       // grid.y: independent problems, as skinny
  W += blockIdx.y * bsw;
  constexpr int NT = 64 * NWAVES;
  constexpr int BM = 16 * MB;
  constexpr int BN = 16 * NBW * NWAVES;
  constexpr int LDSROW = 128;                  // bf16 elements per LDS row
  // The 16 chunks (16 B) of an activation row are XOR-swizzled by
  // (r & 3) | ((r & 4) << 1): a fragment read has lanes 16 apart read chunks 4
  // apart of the same rows, and this keeps what the LDS serves together on
  // distinct banks (a 16-byte row pad left conflict stalls).
  auto xsw = [](int r) { return (r & 3) | ((r & 4) << 1); };
  constexpr int XP = (BM * 16 + NT - 1) / NT;  // 16-byte X pieces per thread per chunk
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * LDSROW];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int t = xcd_tile(blockIdx.x, gridDim.x);
  const int tm = t % ntm, tn = t / ntm;
  const int m0 = tm * BM, n0 = tn * BN + wave * 16 * NBW;
  const int nchunks = Kd >> 7;

  const uint16_t* wp[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    int n = min(n0 + 16 * nb + r16, N - 1);
    wp[nb] = W + (int64_t)n * Kd + 32 * g4;
  }
  const uint16_t* xsrc[XP];
  int xdst[XP];
#pragma unroll
  for (int i = 0; i < XP; ++i) {
    const int piece = min(threadIdx.x + NT * i, BM * 16 - 1);   // BM rows x 16 pieces
    const int row = piece >> 4, part = piece & 15;
    xsrc[i] = X + (int64_t)min(m0 + row, M - 1) * ldx + part * 8;
    xdst[i] = row * LDSROW + (part ^ xsw(row)) * 8;
  }

  f32x4 acc[NBW][MB];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Each workgroup walks the K chunks from its own starting chunk: every
  // workgroup reads the same activation rows, and in lockstep they would all
  // hit the same few L2 channels at once.
  // With rev the walk runs backwards (rot-1, rot-2, ..., rot): the same grid
  // over the same weights then reads, first, what the forward walk read last.
  const int rot = (int)(blockIdx.x % (unsigned)nchunks);
  auto rc = [&](int c) {
    if (rev) { const int q = rot - 1 - c; return q < 0 ? q + nchunks : q; }
    const int q = c + rot;
    return q >= nchunks ? q - nchunks : q;
  };
  uint4 wa[NBW][4], wb[NBW][4], xr[XP];
  auto loadW = [&](int c, uint4 (&w)[NBW][4]) {
    const int k0 = rc(c) << 7;
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int s = 0; s < 4; ++s) w[nb][s] = ldg16(wp[nb] + k0 + 8 * s);
  };
  auto loadX = [&](int c) {
#pragma unroll
    for (int i = 0; i < XP; ++i) xr[i] = ldg16(xsrc[i] + (rc(c) << 7));
  };
  auto storeX = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XP; ++i) *reinterpret_cast<uint4*>(&xs[buf][xdst[i]]) = xr[i];
  };
  auto mma = [&](const uint4 (&w)[NBW][4], int buf) {
    const uint16_t* xb = &xs[buf][r16 * LDSROW];
    const int sw = xsw(r16);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint4 b = *reinterpret_cast<const uint4*>(xb + mb * 16 * LDSROW + 8 * ((4 * g4 + s) ^ sw));
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[nb][mb] = mfma16x16x32(w[nb][s], b, acc[nb][mb]);
      }
    }
  };

  // Chunk c uses LDS buffer c & 1.  Weights: two register stages used
  // alternately (loads never under a branch, indices clamped); X: one chunk
  // ahead in registers, written to the free LDS buffer after the multiply.
  const int cl = nchunks - 1;
  loadX(0);
  loadW(0, wa);
  storeX(0);
  __syncthreads();
  loadX(min(1, cl));
  loadW(min(1, cl), wb);
  for (int c = 0; c + 1 < nchunks; c += 2) {
    __builtin_amdgcn_sched_barrier(0);
    mma(wa, 0);
    storeX(1);
    loadX(min(c + 2, cl));
    loadW(min(c + 2, cl), wa);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    mma(wb, 1);
    storeX(0);
    loadX(min(c + 3, cl));
    loadW(min(c + 3, cl), wb);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  }
  if (nchunks & 1) mma(wa, 0);
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) epi.store4(m0 + 16 * mb + r16, n0 + 16 * nb + 4 * g4, acc[nb][mb]);
  if (tm == 0) epi.copy_base(tn * BN, tn * BN + BN);
  if constexpr (HasParts<Epi>::value) {
    // row partials over this workgroup's BN columns: lanes (4 columns each),
    // then the 4 lane groups of a row (shuffles), then the waves (LDS)
    __syncthreads();                        // every wave is past its last read of xs
    RowPart* red = reinterpret_cast<RowPart*>(&xs[0][0]);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float v[4 * NBW];
      int col[4 * NBW];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[4 * nb + i] = acc[nb][mb][i];
          col[4 * nb + i] = n0 + 16 * nb + 4 * g4 + i;
        }
      RowPart pt = lane_part(v, col, N, epi.typical, epi.inv_temp);
      part_xor(pt, 16, epi.typical);
      part_xor(pt, 32, epi.typical);
      if (g4 == 0) red[wave * BM + 16 * mb + r16] = pt;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < BM; r += NT) {
      if (m0 + r >= M) continue;
      RowPart pt = red[r];
      for (int w = 1; w < NWAVES; ++w) part_merge(pt, red[w * BM + r], epi.typical);
      epi.write_part(m0 + r, tn, pt);
    }
    epi.write_header();
  }
}

// ---------------------------------------------------------------- weight stream by LDS DMA
// The logits GEMMs of at most 80 rows over a wide vocabulary (the heads' LM
// pass, the batch-1 verify rows) and the heads' GEMM over wide weights (the
// 70B layer's 40960 x 8192): the same tile as gemm_tiled_bf16 (BM =
// 16*MB activation rows shared by NW waves of 16 weight rows each, the
// rotated K walk, the same MFMA order, so the same logits bit for bit), but
// both operands reach LDS by direct global->LDS loads through an NBUF-deep
// ring of 128-wide K chunks instead of through registers.  Measured on a
// plain read of 262 MB: 45.8 us into registers, 40.7 us by LDS DMA with the
// non-temporal hint, 45.4 us without it (1 GiB: 6.0, 7.0 and 6.0 TB/s).
//   * A ring slot holds the chunk's X rows and then each wave's 16 weight
//     rows, both row-major with their 16-byte pieces XOR-swizzled by row (as
//     the tiled kernel's X), so the fragment reads are free of bank
//     conflicts; each DMA issue covers four whole 256-byte chunk rows (a
//     gather of 16-byte pieces 64 bytes apart, one fragment's worth, ran at
//     half the rate).
//   * X units (four rows each) are dealt round-robin to the waves; a wave
//     past the last unit repeats one (the same bytes to the same place), so
//     every wave issues XI + 4 loads per chunk and waits on one count.  One
//     barrier per chunk.
//   * w_nt: the weights with the non-temporal hint.  The heads' LM pass
//     reads them without it, so the verify pass over the same weights finds
//     much of them in the last-level cache; the verify pass, the last reader
//     in the step, streams them non-temporally (7B batch 1: the LM pass 51 ->
//     47 us, the verify pass 48 -> 41.5 us).  X is re-read by every
//     workgroup from L2 and never takes the hint.
template <int MB, class Epi, int NW, int NBUF>
__global__ __launch_bounds__(64 * NW) void gemm_dma_bf16(const uint16_t* __restrict__ X,
                                                         int64_t ldx, int M,
                                                         const uint16_t* __restrict__ W, int N,
                                                         int Kd, int ntm, Epi epi, bool rev,
                                                         bool w_nt) {
  constexpr int NT = 64 * NW;
  constexpr int BM = 16 * MB;
  constexpr int BN = 16 * NW;
  constexpr int LDSROW = 128;                      // bf16 per chunk row
  constexpr int XU = BM / 4;                       // 1 KB X units per chunk
  constexpr int XI = (XU + NW - 1) / NW;           // X issues per wave and chunk
  constexpr int NI = XI + 4;                       // loads per wave and chunk
  constexpr int SLOT = (BM + BN) * LDSROW;         // elements per ring slot
  static_assert(NBUF >= 2 && NBUF <= 4, "ring of 2..4 chunks");
  auto xsw = [](int r) { return (r & 3) | ((r & 4) << 1); };
  __shared__ __attribute__((aligned(16))) uint16_t ring[NBUF * SLOT];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int t = xcd_tile(blockIdx.x, gridDim.x);
  const int tm = t % ntm, tn = t / ntm;
  const int m0 = tm * BM, n0 = tn * BN + wave * 16;
  const int nchunks = Kd >> 7;

  // lane l of a unit: row 4u + l/16 of the unit's four, slot l%16 of that
  // row, which holds piece (l%16) ^ xsw(row)
  const int urow = lane >> 4;
  const uint16_t* xsrc[XI];
  uint32_t xoff[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int u = (i * NW + wave) % XU;
    const int row = 4 * u + urow;
    xsrc[i] = X + (int64_t)min(m0 + row, M - 1) * ldx + 8 * ((lane & 15) ^ xsw(row));
    xoff[i] = (uint32_t)(u * 1024);
  }
  const uint16_t* wsrc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 4 * u + urow;
    wsrc[u] = W + (int64_t)min(n0 + row, N - 1) * Kd + 8 * ((lane & 15) ^ xsw(row));
  }
  const uint32_t wreg = (uint32_t)((BM + 16 * wave) * LDSROW * 2);
  const uint32_t rl = lds_u32(&ring[0]);
  // rotated K walk, as in gemm_tiled_bf16 (rev: backwards from the same chunk)
  const int rot = (int)(blockIdx.x % (unsigned)nchunks);
  auto rc = [&](int c) {
    if (rev) { const int q = rot - 1 - c; return q < 0 ? q + nchunks : q; }
    const int q = c + rot;
    return q >= nchunks ? q - nchunks : q;
  };
  auto issue = [&](int c, int buf) {
    const int k0 = rc(c) << 7;
    const uint32_t base = rl + (uint32_t)(buf * SLOT * 2);
#pragma unroll
    for (int i = 0; i < XI; ++i) dma16(xsrc[i] + k0, __builtin_amdgcn_readfirstlane(base + xoff[i]));
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t l = __builtin_amdgcn_readfirstlane(base + wreg + (uint32_t)(u * 1024));
      if (w_nt) dma16_nt(wsrc[u] + k0, l);
      else dma16(wsrc[u] + k0, l);
    }
  };

  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int sw = xsw(r16);
  auto compute = [&](int buf) {
    const uint16_t* xb = &ring[buf * SLOT + r16 * LDSROW];
    const uint16_t* wb = &ring[buf * SLOT + (BM + 16 * wave + r16) * LDSROW];
    uint4 w[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) w[s] = *reinterpret_cast<const uint4*>(wb + 8 * ((4 * g4 + s) ^ sw));
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint4 b = *reinterpret_cast<const uint4*>(xb + mb * 16 * LDSROW + 8 * ((4 * g4 + s) ^ sw));
        acc[mb] = mfma16x16x32(w[s], b, acc[mb]);
      }
  };

#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i)
    if (i < nchunks) issue(i, i);
  for (int c = 0; c < nchunks; ++c) {
    const int ahead = min(nchunks - 1 - c, NBUF - 2);   // chunks issued after chunk c
    if (ahead >= 2) vm_wait<2 * NI>();
    else if (ahead == 1) vm_wait<NI>();
    else vm_wait<0>();
    __syncthreads();   // chunk c landed from every wave; chunk c-1's slot is free
    if (c + NBUF - 1 < nchunks) issue(c + NBUF - 1, (c + NBUF - 1) % NBUF);
    compute(c % NBUF);
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) epi.store4(m0 + 16 * mb + r16, n0 + 4 * g4, acc[mb]);
  if (tm == 0) epi.copy_base(tn * BN, tn * BN + BN);
  if constexpr (HasParts<Epi>::value) {
    // row partials over this workgroup's BN columns, as in gemm_tiled_bf16
    __syncthreads();                        // every wave is past its last read of the ring
    RowPart* red = reinterpret_cast<RowPart*>(&ring[0]);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float v[4];
      int col[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = acc[mb][i];
        col[i] = n0 + 4 * g4 + i;
      }
      RowPart pt = lane_part(v, col, N, epi.typical, epi.inv_temp);
      part_xor(pt, 16, epi.typical);
      part_xor(pt, 32, epi.typical);
      if (g4 == 0) red[wave * BM + 16 * mb + r16] = pt;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < BM; r += NT) {
      if (m0 + r >= M) continue;
      RowPart pt = red[r];
      for (int w = 1; w < NW; ++w) part_merge(pt, red[w * BM + r], epi.typical);
      epi.write_part(m0 + r, tn, pt);
    }
    epi.write_header();
  }
}

// ---------------------------------------------------------------- MFMA-bound, LDS ring
// Tile BM = 32*WMB activation rows x BN = 16*WNB*NWN weight rows; waves 2
// (along M) x NWN (along N), each 16*WMB x 16*WNB outputs.  The operands
// stream in 32-wide K slices through a 4-deep LDS ring filled by direct
// global->LDS loads: while one slice is multiplied the next two are in
// flight and the third is issued, with no staging registers.  A slice row is 64 bytes; its four 16-byte chunks are
// XOR-swizzled by (row >> 1) & 3.  A fragment read has lanes 16 apart read two
// chunks of the same row; with this swizzle the rows and chunks that the LDS
// serves together land on distinct banks (bank-conflict counters read zero;
// swizzling by (row >> 2) & 3 left the LDS stalled on conflicts about half
// of its busy time).  One barrier per slice.
// Each DMA issue fills a 1 KB region (16 rows x 64 bytes).  A ring slot holds
// the activation rows followed by the weight rows, so the BM/16 + BN/16
// regions of a slice are numbered once and dealt round-robin to the first
// wave of each SIMD (waves 0..NW/2-1; the first (regions mod NW/2) of them
// issue one more and wait on their own count).  Those waves issue after the
// slice's MFMAs: the 30-odd loads of a slice take a few hundred cycles to
// issue (the CU's vector-memory path accepts about one 1 KB load per 15
// cycles), and issued right after the barrier they kept every SIMD's MFMA
// pipe idle meanwhile; the SIMD's first wave gets the pipe first, so its loads
// now go out while the second wave's MFMAs run, and the slot they fill was
// read before this slice's barrier.
template <int WMB, int WNB, int NWN, class Epi>
__global__ __launch_bounds__(128 * NWN) void gemm_ring_bf16(const uint16_t* __restrict__ X,
                                                           int64_t ldx, int M,
                                                           const uint16_t* __restrict__ W, int N,
                                                           int Kd, int ntm, Epi epi) {
  constexpr int NW = 2 * NWN;                        // waves: 2 along M x NWN along N
  constexpr int BM = 32 * WMB, BN = 16 * WNB * NWN, BK = 32, NS = 4;
  constexpr int XR = BM / 16, R = XR + BN / 16;      // 1 KB regions per slice
  constexpr int NI = NW / 2;                         // issuing waves: the first on each SIMD
  constexpr int DLO = R / NI, DHI = (R + NI - 1) / NI;  // DMA issues per issuing wave and slice
  constexpr int SL = (BM + BN) * BK;                 // one ring slot, elements
  __shared__ __attribute__((aligned(16))) uint16_t ring[NS][SL];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;
  const int t = xcd_tile(blockIdx.x, gridDim.x);
  const int tm = t % ntm, tn = t / ntm;
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk = Kd / BK;

  // region q < XR: activation rows 16q..16q+15, else weight rows 16(q-XR)..
  const bool issuer = wave < NI;
  const bool extra = issuer && wave < R % NI;        // this wave issues DHI regions
  const uint16_t* src[DHI];
  uint32_t off[DHI];
#pragma unroll
  for (int j = 0; j < DHI; ++j) {
    const int q = min(wave % NI + NI * j, R - 1);
    const int row = 16 * (q < XR ? q : q - XR) + (lane >> 2);
    const int ch = (lane & 3) ^ ((row >> 1) & 3);
    src[j] = q < XR ? X + (int64_t)min(m0 + row, M - 1) * ldx + 8 * ch
                    : W + (int64_t)min(n0 + row, N - 1) * Kd + 8 * ch;
    off[j] = (uint32_t)(q * 1024);
  }
  const uint32_t rl = lds_u32(&ring[0][0]);
  auto issue = [&](int kt, int buf) {
    if (!issuer) return;
    const int k0 = kt * BK;
    const uint32_t base = rl + (uint32_t)(buf * SL * 2);
#pragma unroll
    for (int j = 0; j < DLO; ++j) dma16(src[j] + k0, __builtin_amdgcn_readfirstlane(base + off[j]));
    if (DHI > DLO && extra)
      dma16(src[DHI - 1] + k0, __builtin_amdgcn_readfirstlane(base + off[DHI - 1]));
  };

  f32x4 acc[WNB][WMB];
#pragma unroll
  for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
    const uint16_t* xs = &ring[buf][0];
    const uint16_t* wsm = &ring[buf][BM * BK];
    uint4 a[WNB], bx[WMB];
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) {
      const int row = wn * 16 * WNB + 16 * nb + r16;
      a[nb] = *reinterpret_cast<const uint4*>(&wsm[row * BK + 8 * (g4 ^ ((row >> 1) & 3))]);
    }
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) {
      const int row = wm * 16 * WMB + 16 * mb + r16;
      bx[mb] = *reinterpret_cast<const uint4*>(&xs[row * BK + 8 * (g4 ^ ((row >> 1) & 3))]);
    }
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
      for (int mb = 0; mb < WMB; ++mb) acc[nb][mb] = mfma16x16x32(a[nb], bx[mb], acc[nb][mb]);
  };

#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (i < nk) issue(i, i);
  for (int kt = 0; kt < nk; ++kt) {
    // slices issued after slice kt so far: min(nk - 1 - kt, NS - 2), DHI or
    // DLO issues each (none outstanding on the waves that do not issue)
    const int ahead = min(nk - 1 - kt, NS - 2);
    if (DHI > DLO && extra) {
      if (ahead >= 2) vm_wait<2 * DHI>();
      else if (ahead == 1) vm_wait<DHI>();
      else vm_wait<0>();
    } else {
      if (ahead >= 2) vm_wait<2 * DLO>();
      else if (ahead == 1) vm_wait<DLO>();
      else vm_wait<0>();
    }
    __syncthreads();   // slice kt complete from every wave; slice kt-1's buffer is free
    compute(kt % NS);
    if (kt + NS - 1 < nk) issue(kt + NS - 1, (kt + NS - 1) % NS);
  }
#pragma unroll
  for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb)
      epi.store4(m0 + wm * 16 * WMB + 16 * mb + r16, n0 + wn * 16 * WNB + 16 * nb + 4 * g4,
                 acc[nb][mb]);
  if constexpr (HasParts<Epi>::value) {
    // row partials over this workgroup's BN columns (lanes, lane groups, the
    // NWN waves along N)
    __syncthreads();                        // every wave is past its last read of the ring
    RowPart* red = reinterpret_cast<RowPart*>(&ring[0][0]);
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) {
      float v[4 * WNB];
      int col[4 * WNB];
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[4 * nb + i] = acc[nb][mb][i];
          col[4 * nb + i] = n0 + wn * 16 * WNB + 16 * nb + 4 * g4 + i;
        }
      RowPart pt = lane_part(v, col, N, epi.typical, epi.inv_temp);
      part_xor(pt, 16, epi.typical);
      part_xor(pt, 32, epi.typical);
      if (g4 == 0) red[wn * BM + wm * 16 * WMB + 16 * mb + r16] = pt;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < BM; r += 128 * NWN) {
      if (m0 + r >= M) continue;
      RowPart pt = red[r];
      for (int w = 1; w < NWN; ++w) part_merge(pt, red[w * BM + r], epi.typical);
      epi.write_part(m0 + r, tn, pt);
    }
    epi.write_header();
  }
}

// ---------------------------------------------------------------- f32
// One wave per weight row n; lanes split K; M <= 64 rows, looped in groups of 8.
template <class Epi>
__global__ __launch_bounds__(256) void gemm_rowwave_f32(const float* __restrict__ X, int64_t ldx,
                                                        int M, const float* __restrict__ W, int N,
                                                        int Kd, Epi epi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = blockIdx.x * 4 + wave;
  if (n >= N) return;
  const float* w = W + (int64_t)n * Kd;
  for (int m0 = 0; m0 < M; m0 += 8) {
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
    for (int k = lane; k < Kd; k += 64) {
      float wv = w[k];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (m0 + j < M) acc[j] = fmaf(wv, X[(int64_t)(m0 + j) * ldx + k], acc[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float s = wave_sum(acc[j]);
      if (lane == 0 && m0 + j < M) epi.store1(m0 + j, n, s);
    }
  }
}

// copy x rows into slot 0 of u (the base head's hidden state is h itself)
template <typename T>
__global__ void copy_base_rows(T* U, const T* X, int64_t ldx, int M, int H, int R) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = (int64_t)M * H;
  if (i >= total) return;
  int m = (int)(i / H), o = (int)(i - (int64_t)m * H);
  U[(int64_t)m * R * H + o] = X[(int64_t)m * ldx + o];
}

// ---------------------------------------------------------------- launchers
// Kernel choice for a bf16 GEMM (M activation rows, N weight rows, K = Kd).
struct Bf16Plan {
  int kind;      // 0 skinny, 1 tiled, 2 ring
  int mb;        // tiled: 16-row activation blocks per workgroup
  int nw;        // tiled: waves per workgroup
  int wmb, wnb;  // ring: tile parameters
  int ntiles;    // workgroup tiles along N
  int snb;       // skinny: 16-row weight blocks per workgroup (1 or 2)
};

static Bf16Plan plan_bf16(int M, int N, int Kd, bool logits, bool skinny_ok) {
  Bf16Plan p{};
  const int mb = (M + 15) / 16;
  // 8-wave tiled workgroups own 128 weight rows: with enough rows to give
  // every CU one, they stream best; otherwise skinny (up to 16 rows) or
  // 4-wave tiled workgroups keep more of them in flight.
  const bool wide = N >= 240 * 128;
  if (skinny_ok && !wide && M <= 16 && N >= 256 * 32) {
    p.kind = 0;
    p.snb = 2;
    p.mb = 1;
    p.ntiles = (N + 31) / 32;
    return p;
  }
  // a single head (N = H): 16-row weight blocks so that the launch still has
  // about one workgroup per CU, up to 32 activation rows per workgroup
  if (skinny_ok && M <= 32 && N < 256 * 32) {
    p.kind = 0;
    p.snb = 1;
    p.mb = mb;
    p.ntiles = (N + 15) / 16;
    return p;
  }
  if (logits && mb > 5 && (Kd % 64) == 0) {
    // MFMA-bound: 8-wave ring kernel.  One workgroup fits a CU, so the tile
    // (BM = 128..256 rows x BN = 256 or 320 weight rows) minimises
    // (rounds of 256 workgroups) x (time of one round).  A round's time grows
    // with the operand rows each workgroup streams (BM + BN slices of K) more
    // than with its MFMA work (BM x BN): timed over six tiles at 2080 x 128256
    // x 4096 it fits 220 (BM + BN) + BM BN (160 x 256: 2409 us; 224 x 320 and
    // 256 x 320: 2190-2197 us).
    p.kind = 2;
    long best = -1;
    for (int wmb = 4; wmb <= 8; ++wmb)
      for (int wnb = 4; wnb <= 5; ++wnb) {
        const long tm = (M + 32 * wmb - 1) / (32 * wmb), tn = (N + 64 * wnb - 1) / (64 * wnb);
        const long bm = 32L * wmb, bn = 64L * wnb;
        const long cost = ((tm * tn + 255) / 256) * (220 * (bm + bn) + bm * bn);
        if (best < 0 || cost < best || (cost == best && wmb * wnb > p.wmb * p.wnb)) {
          best = cost;
          p.wmb = wmb;
          p.wnb = wnb;
        }
      }
    p.ntiles = (N + 64 * p.wnb - 1) / (64 * p.wnb);
    // Up to 160 rows the streaming kernel (8 or 10 row blocks per workgroup)
    // beats a ring of few workgroups: 32000 columns at 97-160 rows (125-250
    // ring workgroups) took 59-74 us against 83-85 us.  From 1.5 rounds of
    // the 256 CUs the ring is ahead: 160 rows x 128256 (501 workgroups of
    // 160 x 256) 275 us against 316-320 us streaming.
    const long ring_wgs = (long)((M + 32 * p.wmb - 1) / (32 * p.wmb)) * p.ntiles;
    if (mb > 10 || ring_wgs >= 384) return p;
    p = Bf16Plan{};
  }
  p.kind = 1;
  p.mb = mb <= 6 ? mb : mb <= 8 ? 8 : mb <= 10 ? 10 : 8;
  // Wide weights: 8-wave workgroups of 128 rows; when that leaves a partial
  // last round of workgroups on the 256 CUs (N between 2048 and 4096 16-row
  // blocks), 10/12/16-wave workgroups make exactly one round instead.
  const int units = (N + 15) / 16;
  if (!wide) p.nw = 4;
  else if (p.mb > 5 || units <= 8 * 256 || units > 16 * 256) p.nw = 8;
  else p.nw = units <= 10 * 256 ? 10 : units <= 12 * 256 ? 12 : 16;
  p.ntiles = (N + 16 * p.nw - 1) / (16 * p.nw);
  return p;
}

template <class Epi>
static hipError_t launch_bf16(const uint16_t* X, int64_t ldx, int M, const uint16_t* W, int N,
                              int Kd, const Epi& epi, hipStream_t st, bool rev = false,
                              int batch = 1, int64_t bsx = 0, int64_t bsw = 0, bool w_nt = false) {
  // logits always take the tiled / ring kernels, so the verify-rows logits of
  // medusa_heads and medusa_verify_logits come from the same kernel
  const Bf16Plan p = plan_bf16(M, N, Kd, IsLogits<Epi>::value, !IsLogits<Epi>::value);
  if (p.kind == 0) {
    // skinny: 4 waves split K, X (a few rows) read from L2; with 32-row
    // workgroups and K <= 4096 in whole chunk pairs, the weights by LDS DMA
    if (p.snb == 2 && p.mb == 1 && (Kd % 256) == 0 && Kd <= 4096) {
      hipLaunchKernelGGL((gemm_skinny_dma_bf16<Epi>), dim3(p.ntiles, batch), dim3(256), 0, st, X,
                         ldx, M, W, N, Kd, epi, bsx, bsw);
      return hipGetLastError();
    }
    // 16-row workgroups (single-head GEMMs): both operands by LDS DMA
    // (every bf16 entry point requires K % 128 == 0)
    if (p.snb == 1) {
      if (p.mb == 1)
        hipLaunchKernelGGL((gemm_skinny1_dma_bf16<1, Epi>), dim3(p.ntiles, batch), dim3(256), 0,
                           st, X, ldx, M, W, N, Kd, epi, bsx, bsw);
      else
        hipLaunchKernelGGL((gemm_skinny1_dma_bf16<2, Epi>), dim3(p.ntiles, batch), dim3(256), 0,
                           st, X, ldx, M, W, N, Kd, epi, bsx, bsw);
      return hipGetLastError();
    }
    // 32-row workgroups with K > 4096: the weights into registers
    hipLaunchKernelGGL((gemm_skinny_bf16<2, 1, Epi>), dim3(p.ntiles, batch), dim3(256), 0, st, X,
                       ldx, M, W, N, Kd, epi, bsx, bsw);
    return hipGetLastError();
  }
  if constexpr (IsLogits<Epi>::value) if (p.kind == 2) {
#define RING(WMB_, WNB_)                                                                        \
  do {                                                                                          \
    const int tm = (M + 32 * WMB_ - 1) / (32 * WMB_);                                           \
    hipLaunchKernelGGL((gemm_ring_bf16<WMB_, WNB_, 4, Epi>), dim3(tm * p.ntiles), dim3(512), 0,  \
                       st, X, ldx, M, W, N, Kd, tm, epi);                                       \
  } while (0)
    switch (p.wmb * 10 + p.wnb) {
      case 44: RING(4, 4); break;
      case 45: RING(4, 5); break;
      case 54: RING(5, 4); break;
      case 55: RING(5, 5); break;
      case 64: RING(6, 4); break;
      case 65: RING(6, 5); break;
      case 74: RING(7, 4); break;
      case 75: RING(7, 5); break;
      case 84: RING(8, 4); break;
      default: RING(8, 5); break;
    }
#undef RING
    return hipGetLastError();
  }
  // heads over wide weights from at most 16 rows (8- or 10-wave workgroups;
  // the weights are read once per step, non-temporally): the weight stream by
  // LDS DMA
  if constexpr (!IsLogits<Epi>::value)
    if ((p.nw == 8 || p.nw == 10) && p.mb == 1 && batch == 1 && (N % (16 * p.nw)) == 0) {
      if (p.nw == 8)
        hipLaunchKernelGGL((gemm_dma_bf16<1, Epi, 8, 3>), dim3(p.ntiles), dim3(512), 0, st, X,
                           ldx, M, W, N, Kd, 1, epi, rev, true);
      else
        hipLaunchKernelGGL((gemm_dma_bf16<1, Epi, 10, 3>), dim3(p.ntiles), dim3(640), 0, st, X,
                           ldx, M, W, N, Kd, 1, epi, rev, true);
      return hipGetLastError();
    }
  // logits over a wide vocabulary from at most 80 rows in 8-wave workgroups:
  // the weight stream by LDS DMA (one problem per launch)
  if constexpr (IsLogits<Epi>::value)
    if (p.nw == 8 && p.mb <= 5 && batch == 1 && (N % 128) == 0) {
      const int ntm = (M + 16 * p.mb - 1) / (16 * p.mb);
#define DMAK(MB_)                                                                                 \
  hipLaunchKernelGGL((gemm_dma_bf16<MB_, Epi, 8, 3>), dim3(ntm * p.ntiles), dim3(512), 0, st, X,  \
                     ldx, M, W, N, Kd, ntm, epi, rev, w_nt)
      switch (p.mb) {
        case 1: DMAK(1); break;
        case 2: DMAK(2); break;
        case 3: DMAK(3); break;
        case 4: DMAK(4); break;
        default: DMAK(5); break;
      }
#undef DMAK
      return hipGetLastError();
    }
#define TILED_NW(MB_, NW_)                                                                     \
  do {                                                                                         \
    const int ntm = (M + 16 * MB_ - 1) / (16 * MB_);                                           \
    hipLaunchKernelGGL((gemm_tiled_bf16<MB_, 1, Epi, NW_>), dim3(ntm * p.ntiles, batch),      \
                       dim3(64 * NW_), 0, st, X, ldx, M, W, N, Kd, ntm, epi, rev, bsx, bsw);   \
  } while (0)
#define TILED(MB_)                                                                             \
  do {                                                                                         \
    if (p.nw == 4) TILED_NW(MB_, 4);                                                           \
    else if (MB_ > 5 || p.nw == 8) TILED_NW(MB_, 8);                                           \
    else if (p.nw == 10) TILED_NW(MB_, (MB_ > 5 ? 8 : 10));                                    \
    else if (p.nw == 12) TILED_NW(MB_, (MB_ > 5 ? 8 : 12));                                    \
    else TILED_NW(MB_, (MB_ > 5 ? 8 : 16));                                                    \
  } while (0)
  switch (p.mb) {
    case 1: TILED(1); break;
    case 2: TILED(2); break;
    case 3: TILED(3); break;
    case 4: TILED(4); break;
    case 5: TILED(5); break;
    case 6: TILED(6); break;
    case 10: TILED(10); break;
    default: TILED(8); break;
  }
#undef TILED
#undef TILED_NW
  return hipGetLastError();
}

template <class Epi>
static hipError_t launch_f32(const float* X, int64_t ldx, int M, const float* W, int N, int Kd,
                             const Epi& epi, hipStream_t st) {
  hipLaunchKernelGGL((gemm_rowwave_f32<Epi>), dim3((N + 3) / 4), dim3(256), 0, st, X, ldx, M, W,
                     N, Kd, epi);
  return hipGetLastError();
}

hipError_t run_heads_hidden(const void* x, int M, int H, const void* W, int n_heads, int dtype,
                            void* u, int R, int base, hipStream_t st) {
  const int N = n_heads * H;
  if (dtype == kBF16) {
    const uint16_t* X = static_cast<const uint16_t*>(x);
    uint16_t* U = static_cast<uint16_t*>(u);
    if (base && n_heads == 0) {
      int64_t tot = (int64_t)M * H;
      hipLaunchKernelGGL(copy_base_rows<uint16_t>, dim3((unsigned)((tot + 255) / 256)), dim3(256),
                         0, st, U, X, (int64_t)H, M, H, R);
    }
    if (n_heads == 0) return hipGetLastError();
    EpiHeads<uint16_t> epi{U, X, (int64_t)H, H, R, base, M, N};
    return launch_bf16(X, H, M, static_cast<const uint16_t*>(W), N, H, epi, st);
  } else {
    const float* X = static_cast<const float*>(x);
    float* U = static_cast<float*>(u);
    if (base) {
      int64_t tot = (int64_t)M * H;
      hipLaunchKernelGGL(copy_base_rows<float>, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0,
                         st, U, X, (int64_t)H, M, H, R);
    }
    if (n_heads == 0) return hipGetLastError();
    EpiHeads<float> epi{U, X, (int64_t)H, H, R, base, M, N};
    return launch_f32(X, H, M, static_cast<const float*>(W), N, H, epi, st);
  }
}

hipError_t run_lm_logits(const void* x, int M, int H, const void* LM, int V, int dtype,
                         float* logits, hipStream_t st, bool rev, int64_t ldc, bool stream_w) {
  EpiLogits epi{logits, ldc > 0 ? ldc : (int64_t)V, M, V};
  if (dtype == kBF16)
    return launch_bf16(static_cast<const uint16_t*>(x), H, M, static_cast<const uint16_t*>(LM), V,
                       H, epi, st, rev, 1, 0, 0, stream_w);
  return launch_f32(static_cast<const float*>(x), H, M, static_cast<const float*>(LM), V, H, epi,
                    st);
}

// ---------------------------------------------------------------- MTP layer GEMMs
hipError_t run_mtp_qkv(const uint16_t* a, int M, int H, const uint16_t* Wqkv, int heads, int nq,
                       int nkv, int d, uint16_t* Q, uint16_t* Kc, uint16_t* Vc,
                       const int* seq_len, int Pmax, hipStream_t st) {
  const int N = (nq + 2 * nkv) * d;
  EpiQKV epi{Q, Kc, Vc, seq_len, nq * d, nkv * d, d, Pmax, M, N};
  return launch_bf16(a, H, M, Wqkv, N, H, epi, st, false, heads, (int64_t)M * H, (int64_t)N * H);
}

hipError_t run_mtp_resid(const uint16_t* x, int64_t ldx, int64_t sx, int M, int Kd,
                         const uint16_t* W, int N, int heads, uint16_t* O, int64_t so,
                         int64_t ldo, const uint16_t* R, int64_t sr, int64_t ldr, hipStream_t st) {
  EpiResid epi{O, R, so, ldo, sr, ldr, M, N};
  return launch_bf16(x, ldx, M, W, N, Kd, epi, st, false, heads, sx, (int64_t)N * Kd);
}

hipError_t run_mtp_swiglu(const uint16_t* a, int M, int H, const uint16_t* Wgu, int F, int heads,
                          uint16_t* z, hipStream_t st) {
  EpiSwiGLU epi{z, (int64_t)M * F, (int64_t)F, M, 2 * F};
  return launch_bf16(a, H, M, Wgu, 2 * F, H, epi, st, false, heads, (int64_t)M * H,
                     (int64_t)2 * F * H);
}

// ---------------------------------------------------------------- verify logits + partials
// f32 rows (tiny workload): one 256-thread workgroup per row folds the whole
// row into one partial (ntiles = 1).
__global__ __launch_bounds__(256) void row_parts_f32(const float* __restrict__ logits, int M, int V,
                                                     bool typical, float inv_temp,
                                                     int* __restrict__ header,
                                                     uint64_t* __restrict__ pkey,
                                                     RowStat* __restrict__ pstat) {
  const int row = blockIdx.x;
  const float* x = logits + (int64_t)row * V;
  RowPart pt;
  part_init(pt);
  for (int e = threadIdx.x; e < V; e += 256) part_add(pt, x[e], e, typical, inv_temp);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) part_xor(pt, o, typical);
  __shared__ RowPart red[4];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = pt;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) part_merge(pt, red[w], typical);
    if (typical) pstat[row] = RowStat{pt.m, pt.s, pt.t, 0.f};
    else pkey[row] = pt.key;
    if (row == 0) {
      header[kHdrTiles] = 1;
      header[kHdrKind] = typical ? 1 : 0;
      header[kHdrRows] = M;
      header[kHdrCols] = V;
      header[kHdrInvTemp] = __float_as_int(inv_temp);
      header[kHdrMagic] = kPartsMagic;
    }
  }
}

int verify_tiles(int M, int N, int Kd, int dtype) {
  if (dtype != kBF16) return 1;
  return plan_bf16(M, N, Kd, true, false).ntiles;
}

// Partials pay off when the logits are large (re-reading them for the
// statistics costs more than merging the partials): from 2^24 logits.
bool verify_uses_parts(int64_t M, int64_t N) { return M * N >= (int64_t)1 << 24; }

size_t verify_workspace(int M, int N, int Kd, int dtype, int mode) {
  if (!verify_uses_parts(M, N)) return kPartsHeader;
  const size_t per = mode == kTypical ? sizeof(RowStat) : sizeof(uint64_t);
  return kPartsHeader + (size_t)M * verify_tiles(M, N, Kd, dtype) * per;
}

hipError_t run_verify_logits(const void* x, int M, int H, const void* LM, int V, int dtype,
                             float* logits, int mode, float temperature, void* ws, hipStream_t st) {
  // the verify pass is the step's last reader of the LM weights: they stream
  // non-temporally where the weight-stream kernel runs
  if (!verify_uses_parts(M, V)) return run_lm_logits(x, M, H, LM, V, dtype, logits, st, false, 0, true);
  const bool typical = mode == kTypical;
  const float inv_temp = 1.0f / temperature;
  int* header = static_cast<int*>(ws);
  uint64_t* pkey = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + kPartsHeader);
  RowStat* pstat = reinterpret_cast<RowStat*>(static_cast<char*>(ws) + kPartsHeader);
  if (dtype == kBF16) {
    EpiLogitsStats epi{};
    epi.C = logits;
    epi.ldc = V;
    epi.M = M;
    epi.N = V;
    epi.typical = typical;
    epi.inv_temp = inv_temp;
    epi.ntiles = verify_tiles(M, V, H, dtype);
    epi.header = header;
    epi.pkey = pkey;
    epi.pstat = pstat;
    return launch_bf16(static_cast<const uint16_t*>(x), H, M, static_cast<const uint16_t*>(LM), V,
                       H, epi, st, false, 1, 0, 0, true);
  }
  hipError_t e = run_lm_logits(x, M, H, LM, V, dtype, logits, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_parts_f32, dim3(M), dim3(256), 0, st, logits, M, V, typical, inv_temp,
                     header, pkey, pstat);
  return hipGetLastError();
}

}  // namespace medusa
