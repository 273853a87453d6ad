// Tree-masked attention of the verification pass.
//
// inferensys.com "Medusa Heads" (tree attention): all candidate branches share
// the KV cache of the common prefix and every node is scored in one pass;
// aicassindra.com "Medusa deep dive" ("From top-k heads to a sparse candidate
// tree"): a node attends only to its own ancestors.  Node i of sequence b
// sees prefix slots [0, P), and the tree slots P + j for j in Anc(i) u {i};
// P = seq_len[b].  Scale 1/sqrt(d); q head h reads kv head floor(h*nkv/nq).
//
// bf16 kernel (gfx950 MFMA 16x16x32):
//   * One workgroup = one (sequence, kv head, key partition, row group).  The
//     query rows of a kv head are all (node, q head of the group) pairs, so a
//     KV tile brought into LDS serves every tree node and every grouped head.
//   * Per 64-key tile: K is stored row-major in LDS, V transposed (V^T).
//     Each wave computes S^T = K Q^T for its 16-row blocks (the query rows are
//     the MFMA columns), so a lane holds 4 keys x 1 query row: the online
//     softmax state of a row lives in the lane that owns it, the probabilities
//     feed the next MFMA (O^T = V^T P^T) straight from registers, and O^T
//     comes out with the same row-per-lane layout, so the rescale by the
//     running max is a per-lane multiply.
//   * The ancestor bitmask (<= 4 words for <= 256 nodes) sits in registers;
//     only keys >= P consult it.
//   * Key partitions ("split-KV") write unnormalised partial outputs with
//     their (max, sum) in log2 units; attn_merge combines them.  With a single
//     partition the kernel normalises and writes O directly.
//   * Workgroups are remapped so the row groups of one (sequence, kv head,
//     partition) are adjacent on one XCD and share its L2 for the KV tile.
// f32 kernel (tiny fp32 workload): one workgroup per (sequence, node, q head),
// scores staged in LDS, exact two-pass softmax.

#include "common.h"
#include "kernels.h"

namespace medusa {

constexpr int kMaxF32Keys = 16384;  // f32 kernel keeps scores in LDS

__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int x = b & 7, j = b >> 3;
  const int q = total >> 3, r = total & 7;
  return x * q + min(x, r) + j;
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): within each 16-lane group,
// lane j receives element (j % 4) of the 64-bit words addressed by lanes
// 4*i + j/4, i = 0..3.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(
          (__attribute__((address_space(3))) char*)(uintptr_t)(const void*)p));
  return __builtin_bit_cast(uint2, r);
}

constexpr int kRB = 1;              // 16-row blocks per wave
constexpr int kWaves = 8;           // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsWG = 16 * kRB * kWaves;   // query rows per workgroup
constexpr int kKT2 = 64;            // keys per tile

// Tree attention, bf16.  Workgroup = (sequence b, kv head g, key partition,
// group of 128 query rows); each of the 8 waves owns one 16-row block.  Small
// per-wave state (one row block) lets two workgroups share a CU, so one
// hides the other's load latency.
//   * Each 64-key tile of K and V is loaded cooperatively (16-byte pieces,
//     coalesced) into a double-buffered LDS tile, rows stored contiguously
//     with 16-byte chunks XOR-swizzled by row, so that both the K fragment
//     reads and the transposing V reads are free of bank conflicts.
//   * S^T = K Q^T per 16-row block (keys are MFMA rows, query rows MFMA
//     columns: a lane holds 4 keys x 1 query row).  The probabilities feed
//     O^T = V^T P^T straight from the S^T accumulators; V^T fragments come
//     from ds_read_b64_tr_b16 on the row-major V tile.  A row's softmax state
//     and its output column therefore live in the same lane.
//   * The running max is raised (O^T, l rescaled) only when a tile's max
//     exceeds it by more than 2^8, so most tiles skip the rescale.
//   * One barrier per tile: tile i+1 is written to the other LDS buffer while
//     tile i is multiplied, and tile i+2's loads are in flight.
//   * Key partitions write unnormalised partial outputs with (max, sum) in
//     log2 units for attn_merge; with one partition O is written directly.
template <int D>
__global__ __launch_bounds__(kThreads) void tree_attn_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
    const uint16_t* __restrict__ Vc, const int* __restrict__ seq_len,
    const uint64_t* __restrict__ anc, int anc_words, int T, int nq, int nkv, int Pmax,
    float scale_log2, int nsplit, int rowgroups, int tiles_per_split, uint16_t* __restrict__ O,
    float* __restrict__ ws_o, float2* __restrict__ ws_ml) {
  constexpr int DS = D / 32;            // MFMA steps over the head dim (S^T)
  constexpr int DB = D / 16;            // 16-wide head-dim blocks (O^T)
  constexpr int CPR = D * 2 / 16;       // 16-byte chunks per K/V row
  constexpr int SWZ = CPR - 1;
  constexpr int PIECES = kKT2 * CPR / kThreads;  // chunks per thread per tensor per tile
  __shared__ __attribute__((aligned(16))) uint16_t kbuf[2][kKT2 * D];
  __shared__ __attribute__((aligned(16))) uint16_t vbuf[2][kKT2 * D];
  __shared__ uint64_t anc_s[kMaxT * kMaxAncWords];

  const int tile_id = xcd_remap(blockIdx.x, gridDim.x);
  const int rg = tile_id % rowgroups;
  const int rest = tile_id / rowgroups;
  const int split = rest % nsplit;
  const int bg = rest / nsplit;
  const int b = bg / nkv, g = bg - b * nkv;
  const int G = nq / nkv;
  const int rows = T * G;
  const int rows_pad = rowgroups * kRowsWG;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int wrow0 = rg * kRowsWG + wave * 16 * kRB;
  // row blocks of this wave holding at least one real row
  const int nvb = max(0, min(kRB, (rows - wrow0 + 15) / 16));

  const int P = seq_len[b];
  const bool valid = P >= 0 && P + T <= Pmax;
  const int nkeys = valid ? P + T : 0;
  const int ntiles = (nkeys + kKT2 - 1) / kKT2;
  const int t_begin = split * tiles_per_split;
  const int t_end = min(ntiles, t_begin + tiles_per_split);
  const int64_t kvbase = ((int64_t)b * nkv + g) * (int64_t)Pmax * D;

  for (int i = threadIdx.x; i < T * anc_words; i += kThreads)
    anc_s[(i / anc_words) * kMaxAncWords + i % anc_words] = anc[i];

  uint4 qf[kRB][DS];
  int node[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int rr = min(wrow0 + 16 * rb + r16, rows - 1);
    const int t = rr / G, hg = rr - t * G;
    node[rb] = t;
    const uint16_t* qp = Q + (((int64_t)b * T + t) * nq + g * G + hg) * D + 8 * g4;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[rb][ds] = ldg16(qp + 32 * ds);
  }
  f32x4 acc[kRB][DB];
  float m_run[kRB], l_run[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
  }

  uint4 kr[PIECES], vr[PIECES];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int c = threadIdx.x + kThreads * i;
      const int row = c / CPR, ch = c % CPR;
      const int64_t off = kvbase + (int64_t)min(tile * kKT2 + row, Pmax - 1) * D + 8 * ch;
      kr[i] = ldg16(Kc + off);
      vr[i] = ldg16(Vc + off);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int c = threadIdx.x + kThreads * i;
      const int row = c / CPR, ch = c % CPR;
      const int dst = row * D + 8 * (ch ^ (row & SWZ));
      *reinterpret_cast<uint4*>(&kbuf[buf][dst]) = kr[i];
      *reinterpret_cast<uint4*>(&vbuf[buf][dst]) = vr[i];
    }
  };
  auto compute = [&](int tile, int buf) {
    const int key0 = tile * kKT2;
    const bool tree_tile = key0 + kKT2 > P;
    const uint16_t* kb_ = kbuf[buf];
    const uint16_t* vb_ = vbuf[buf];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      if (rb >= nvb) break;
      f32x4 s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int krow = 16 * kb + r16;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const uint4 kf = *reinterpret_cast<const uint4*>(kb_ + krow * D + 8 * ((4 * ds + g4) ^ (krow & SWZ)));
          s[kb] = mfma16x16x32(kf, qf[rb][ds], s[kb]);
        }
      }
      float x[4][4];
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = key0 + 16 * kb + 4 * g4 + i;
          bool vis = key < P;
          if (tree_tile && !vis && key < nkeys) {
            const int j = key - P;
            vis = (anc_s[node[rb] * kMaxAncWords + (j >> 6)] >> (j & 63)) & 1ull;
          }
          x[kb][i] = vis ? s[kb][i] * scale_log2 : -INFINITY;
          mt = fmaxf(mt, x[kb][i]);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      // lazy max: raised only when the tile max exceeds it by more than 2^8
      const bool raise = mt > m_run[rb] + 8.0f;
      if (__any(raise)) {
        const float m_new = raise ? mt : m_run[rb];
        const float alpha = m_run[rb] == -INFINITY ? 0.f : exp2f(m_run[rb] - m_new);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          acc[rb][db][0] *= alpha; acc[rb][db][1] *= alpha;
          acc[rb][db][2] *= alpha; acc[rb][db][3] *= alpha;
        }
        l_run[rb] *= alpha;
        m_run[rb] = m_new;
      }
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[kb][i] = x[kb][i] == -INFINITY ? 0.f : exp2f(x[kb][i] - m_run[rb]);
          psum += x[kb][i];
        }
      l_run[rb] += psum;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4 pb;   // P^T slots 8*g4 + j <-> keys 32*ks + 16*(j/4) + 4*g4 + j%4
        pb.x = pack_bf16x2(x[2 * ks][0], x[2 * ks][1]);
        pb.y = pack_bf16x2(x[2 * ks][2], x[2 * ks][3]);
        pb.z = pack_bf16x2(x[2 * ks + 1][0], x[2 * ks + 1][1]);
        pb.w = pack_bf16x2(x[2 * ks + 1][2], x[2 * ks + 1][3]);
        // lane j of group g4 addresses V[32*ks + 4*g4 + j/4 (+16)][16*db + 4*(j%4) .. +4];
        // the transposing read returns V[32*ks + 4*g4 + i (+16)][16*db + j], i = 0..3
        const int vrow = 32 * ks + 4 * g4 + (r16 >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int cb = 32 * db + 8 * (r16 & 3);
          const int ch = cb >> 4, he = (cb & 15) >> 1;
          const uint2 lo = lds_read_tr16(vb_ + vrow * D + 8 * (ch ^ (vrow & SWZ)) + he);
          const uint2 hi = lds_read_tr16(vb_ + (vrow + 16) * D + 8 * (ch ^ ((vrow + 16) & SWZ)) + he);
          uint4 va;
          va.x = lo.x; va.y = lo.y; va.z = hi.x; va.w = hi.y;
          acc[rb][db] = mfma16x16x32(va, pb, acc[rb][db]);
        }
      }
    }
  };

  __syncthreads();   // anc_s
  if (t_begin < t_end) {
    const int tl = t_end - 1;
    load_tile(t_begin);
    store_tile(0);
    load_tile(min(t_begin + 1, tl));
    __syncthreads();
    for (int tile = t_begin; tile < t_end; ++tile) {
      const int buf = (tile - t_begin) & 1;
      __builtin_amdgcn_sched_barrier(0);
      compute(tile, buf);
      __builtin_amdgcn_sched_barrier(0);
      store_tile(buf ^ 1);                 // tile + 1 (a repeat of the last tile at the end)
      load_tile(min(tile + 2, tl));
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    }
  }

  // epilogue
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    float l = l_run[rb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int row = wrow0 + 16 * rb + r16;
    if (row >= rows) continue;
    if (nsplit == 1) {
      const int t = row / G, hg = row - t * G;
      uint16_t* op = O + (((int64_t)b * T + t) * nq + g * G + hg) * D + 4 * g4;
      const float inv = 1.0f / l;       // l == 0 only for an invalid seq_len: NaN output
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        uint2 o;
        o.x = pack_bf16x2(acc[rb][db][0] * inv, acc[rb][db][1] * inv);
        o.y = pack_bf16x2(acc[rb][db][2] * inv, acc[rb][db][3] * inv);
        *reinterpret_cast<uint2*>(op + 16 * db) = o;
      }
    } else {
      const int64_t prow = ((int64_t)bg * nsplit + split) * rows_pad + row;
      float* wp = ws_o + prow * D + 4 * g4;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(wp + 16 * db) = acc[rb][db];
      if (g4 == 0) ws_ml[prow] = make_float2(m_run[rb], l);
    }
  }
}

// Combine key partitions: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// One thread per (row, 4 dims); the loads of every partition are issued before
// any is used (at most kMaxSplit partitions), then a single pass combines them.
constexpr int kMaxSplit = 16;

template <int D>
__global__ __launch_bounds__(256) void attn_merge(const float* __restrict__ ws_o,
                                                  const float2* __restrict__ ws_ml, int nsplit,
                                                  int rows, int rows_pad, int T, int nq, int nkv,
                                                  uint16_t* __restrict__ O) {
  constexpr int TPR = D / 4;           // threads per row
  constexpr int RPB = 256 / TPR;       // rows per block
  const int bg = blockIdx.y;
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = (threadIdx.x % TPR) * 4;
  if (row >= rows) return;
  const int b = bg / nkv, g = bg - b * nkv;
  const int G = nq / nkv;
  const int64_t pbase = (int64_t)bg * nsplit * rows_pad + row;
  float2 ml[kMaxSplit];
  f32x4 o[kMaxSplit];
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s) {
    if (s < nsplit) {
      const int64_t prow = pbase + (int64_t)s * rows_pad;
      ml[s] = ws_ml[prow];
      o[s] = *reinterpret_cast<const f32x4*>(ws_o + prow * D + c);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s)
    if (s < nsplit) M = fmaxf(M, ml[s].x);
  float den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s) {
    if (s < nsplit && ml[s].x != -INFINITY) {
      const float w = exp2f(ml[s].x - M);
      den += w * ml[s].y;
      num[0] += w * o[s][0]; num[1] += w * o[s][1]; num[2] += w * o[s][2]; num[3] += w * o[s][3];
    }
  }
  const float inv = 1.0f / den;
  const int t = row / G, hg = row - t * G;
  uint16_t* op = O + (((int64_t)b * T + t) * nq + g * G + hg) * D + c;
  uint2 r;
  r.x = pack_bf16x2(num[0] * inv, num[1] * inv);
  r.y = pack_bf16x2(num[2] * inv, num[3] * inv);
  *reinterpret_cast<uint2*>(op) = r;
}

// ---------------------------------------------------------------- f32
__global__ __launch_bounds__(256) void tree_attn_f32(const float* __restrict__ Q,
                                                     const float* __restrict__ Kc,
                                                     const float* __restrict__ Vc,
                                                     const int* __restrict__ seq_len,
                                                     const uint64_t* __restrict__ anc,
                                                     int anc_words, int T, int nq, int nkv, int D,
                                                     int Pmax, float scale, float* __restrict__ O) {
  __shared__ float qs[256];
  __shared__ float sc[kMaxF32Keys];
  __shared__ float red[4];
  const int id = blockIdx.x;
  const int h = id % nq, t = (id / nq) % T, b = id / (nq * T);
  const int g = (h * nkv) / nq;
  const int P = seq_len[b];
  const bool valid = P >= 0 && P + T <= Pmax && P + T <= kMaxF32Keys;
  const int nkeys = valid ? P + T : 0;
  const float* q = Q + (((int64_t)b * T + t) * nq + h) * D;
  const int64_t kvbase = ((int64_t)b * nkv + g) * (int64_t)Pmax * D;
  for (int c = threadIdx.x; c < D; c += 256) qs[c] = q[c];
  __syncthreads();
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < nkeys; j += 256) {
    bool vis = j < P;
    if (!vis) {
      const int n = j - P;
      vis = (anc[(int64_t)t * anc_words + (n >> 6)] >> (n & 63)) & 1ull;
    }
    float s = -INFINITY;
    if (vis) {
      const float* k = Kc + kvbase + (int64_t)j * D;
      float a = 0.f;
      for (int c = 0; c < D; ++c) a = fmaf(qs[c], k[c], a);
      s = a * scale;
    }
    sc[j] = s;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.f;
  for (int j = threadIdx.x; j < nkeys; j += 256) {
    const float p = sc[j] == -INFINITY ? 0.f : expf(sc[j] - mx);
    sc[j] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sum;
  __syncthreads();
  sum = (red[0] + red[1]) + (red[2] + red[3]);
  float* o = O + (((int64_t)b * T + t) * nq + h) * D;
  for (int c = threadIdx.x; c < D; c += 256) {
    float a = 0.f;
    for (int j = 0; j < nkeys; ++j) a = fmaf(sc[j], Vc[kvbase + (int64_t)j * D + c], a);
    o[c] = a / sum;
  }
}

// ---------------------------------------------------------------- host side
AttnPlan attn_plan(int b, int T, int nq, int nkv, int d, int Pmax, int dtype) {
  AttnPlan p{1, 1, 1, 0};
  if (dtype != kBF16) return p;
  const int G = nq / nkv;
  const int rows = T * G;
  p.rb = kRB;
  p.rowgroups = (rows + kRowsWG - 1) / kRowsWG;
  const int tiles = (Pmax + kKT2 - 1) / kKT2;
  const int base = b * nkv * p.rowgroups;
  // aim at >= 512 workgroups, >= 4 tiles (256 keys) per partition
  int want = (512 + base - 1) / base;
  int maxsplit = tiles / 2 > 0 ? tiles / 2 : 1;
  p.nsplit = want < maxsplit ? want : maxsplit;
  if (p.nsplit > kMaxSplit) p.nsplit = kMaxSplit;
  if (p.nsplit < 1) p.nsplit = 1;
  if (p.nsplit > 1) {
    const size_t rows_pad = (size_t)p.rowgroups * kRowsWG;
    p.ws_bytes = (size_t)b * nkv * p.nsplit * rows_pad * ((size_t)d * sizeof(float) + sizeof(float2));
  }
  return p;
}

hipError_t run_tree_attn(const void* Q, const void* Kc, const void* Vc, const int* seq_len,
                         const uint64_t* anc, int anc_words, int b, int T, int nq, int nkv, int d,
                         int Pmax, float scale, int dtype, void* O, void* ws, const AttnPlan& p,
                         hipStream_t st) {
  if (dtype == kF32) {
    hipLaunchKernelGGL(tree_attn_f32, dim3(b * T * nq), dim3(256), 0, st,
                       static_cast<const float*>(Q), static_cast<const float*>(Kc),
                       static_cast<const float*>(Vc), seq_len, anc, anc_words, T, nq, nkv, d, Pmax,
                       scale, static_cast<float*>(O));
    return hipGetLastError();
  }
  const float scale_log2 = scale * 1.4426950408889634f;
  const int tiles = (Pmax + kKT2 - 1) / kKT2;
  const int tps = (tiles + p.nsplit - 1) / p.nsplit;
  const int rows = T * (nq / nkv);
  const int rows_pad = p.rowgroups * kRowsWG;
  float* ws_o = static_cast<float*>(ws);
  float2* ws_ml = reinterpret_cast<float2*>(
      static_cast<char*>(ws) + (size_t)b * nkv * p.nsplit * rows_pad * d * sizeof(float));
  const int nblk = b * nkv * p.nsplit * p.rowgroups;
  const uint16_t* q = static_cast<const uint16_t*>(Q);
  const uint16_t* k = static_cast<const uint16_t*>(Kc);
  const uint16_t* v = static_cast<const uint16_t*>(Vc);
  uint16_t* o = static_cast<uint16_t*>(O);
  if (d == 128)
    hipLaunchKernelGGL(tree_attn_bf16<128>, dim3(nblk), dim3(kThreads), 0, st, q, k, v, seq_len, anc,
                       anc_words, T, nq, nkv, Pmax, scale_log2, p.nsplit, p.rowgroups, tps, o, ws_o,
                       ws_ml);
  else
    hipLaunchKernelGGL(tree_attn_bf16<64>, dim3(nblk), dim3(kThreads), 0, st, q, k, v, seq_len, anc,
                       anc_words, T, nq, nkv, Pmax, scale_log2, p.nsplit, p.rowgroups, tps, o, ws_o,
                       ws_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  if (d == 128)
    hipLaunchKernelGGL(attn_merge<128>, dim3((rows + 7) / 8, b * nkv), dim3(256), 0, st, ws_o,
                       ws_ml, p.nsplit, rows, rows_pad, T, nq, nkv, o);
  else
    hipLaunchKernelGGL(attn_merge<64>, dim3((rows + 15) / 16, b * nkv), dim3(256), 0, st, ws_o,
                       ws_ml, p.nsplit, rows, rows_pad, T, nq, nkv, o);
  return hipGetLastError();
}

}  // namespace medusa
