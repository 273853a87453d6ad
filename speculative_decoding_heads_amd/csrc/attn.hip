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
//     KV tile brought into LDS serves every tree node and every grouped head;
//     a row group holds up to 24 16-row blocks (384 rows), and the plan sizes
//     the groups so that their busiest SIMD carries as few blocks as the
//     number of CUs allows.
//   * K/V tiles stream through a 4-deep LDS ring filled by direct
//     global->LDS loads (three tiles in flight per workgroup), non-temporal:
//     the cache is read once per step (measured: the batch-16 verify GEMM
//     after it 290 -> 281-285 us, the weights staying in the last-level cache).
//   * Each wave computes S^T = K Q^T for its 16-row blocks (the query rows are
//     the MFMA columns), so a lane holds 4 keys x 1 query row: the online
//     softmax state of a row lives in the lane that owns it, the probabilities
//     feed the next MFMA (O^T = V^T P^T) straight from registers, and O^T
//     comes out with the same row-per-lane layout, so the rescale by the
//     running max is a per-lane multiply.
//   * The ancestor bitmask (<= 4 words per node) sits in LDS; only keys >= P
//     consult it.
//   * Key partitions ("split-KV") write unnormalised partial outputs with
//     their (max, sum) in log2 units; attn_merge combines them.  With a single
//     partition the kernel normalises and writes O directly.
//   * Workgroups are remapped so the row groups of one (sequence, kv head,
//     partition) are adjacent on one XCD and share its L2 for the KV tile.
// f32 kernel (tiny fp32 workload): one workgroup per (sequence, node, q head),
// scores staged in LDS, exact two-pass softmax.

#include <mutex>
#include <type_traits>

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

constexpr int kWaves = 8;           // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kKT2 = 64;            // keys per tile
// LDS ring depth in tiles: 4 (three in flight, 136 KB: one workgroup per CU),
// or 2 (one in flight, 72 KB) so that two workgroups of one 16-row block per
// wave share a CU

// Tree attention, bf16.  Workgroup = (sequence b, kv head g, key partition,
// group of bpg <= 8 RB 16-row blocks of query rows); 8 waves, each owning up
// to RB blocks (block rb of wave w is block 8*rb + w of the group, so short
// groups spread over all waves).
//   * K and V tiles of 64 keys stream through a 4-deep LDS ring by direct
//     global->LDS loads: three tiles are in flight while one is multiplied,
//     with no staging registers.  Rows are stored contiguously with 16-byte
//     chunks XOR-swizzled by row, so both the K fragment reads and the
//     transposing V reads are free of bank conflicts.  One barrier per tile.
//   * S^T = K Q^T per 16-row block (keys are MFMA rows, query rows MFMA
//     columns: a lane holds 4 keys x 1 query row); each K fragment read from
//     LDS serves all RB row blocks.  The probabilities feed O^T = V^T P^T
//     straight from the S^T accumulators; V^T fragments come from
//     ds_read_b64_tr_b16 on the row-major V tile and also serve all RB blocks.
//     A row's softmax state and its output column live in the same lane.
//   * The running max is raised (O^T, l rescaled) only when a tile's max
//     exceeds it by more than 2^8, so most tiles skip the rescale.
//   * Key partitions write unnormalised partial outputs with (max, sum) in
//     log2 units for attn_merge; with one partition O is written directly.
template <int D, int RB, int NBUF>
__global__ __launch_bounds__(kThreads) void tree_attn_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
    const uint16_t* __restrict__ Vc, const int* __restrict__ seq_len,
    const uint64_t* __restrict__ anc, int anc_words, int T, int nq, int nkv, int Pmax,
    float scale_log2, int nsplit, int rowgroups, int bpg, int tiles_per_split,
    uint16_t* __restrict__ O,
    float* __restrict__ ws_o, float2* __restrict__ ws_ml) {
  constexpr int DS = D / 32;            // MFMA steps over the head dim (S^T)
  constexpr int DB = D / 16;            // 16-wide head-dim blocks (O^T)
  constexpr int CPR = D * 2 / 16;       // 16-byte chunks per K/V row
  constexpr int SWZ = CPR - 1;
  constexpr int ROWS_KB = 1024 / (2 * D);          // K/V rows per 1 KB DMA region
  constexpr int NI = kKT2 / ROWS_KB / kWaves;      // DMA issues per thread per tensor per tile
  static_assert(NI >= 1 && kKT2 % (ROWS_KB * kWaves) == 0, "tile must split into DMA regions");
  static_assert(NBUF >= 2 && NBUF <= 4, "ring of 2..4 tiles");
  __shared__ __attribute__((aligned(16))) uint16_t kbuf[NBUF][kKT2 * D];
  __shared__ __attribute__((aligned(16))) uint16_t vbuf[NBUF][kKT2 * D];
  __shared__ uint64_t anc_s[kMaxT * kMaxAncWords];

  const int tile_id = xcd_remap(blockIdx.x, gridDim.x);
  const int rg = tile_id % rowgroups;
  const int rest = tile_id / rowgroups;
  const int split = rest % nsplit;
  const int bg = rest / nsplit;
  const int b = bg / nkv, g = bg - b * nkv;
  const int G = nq / nkv;
  const int rows = T * G;
  const int rows_pad = rowgroups * bpg * 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  // the group's bpg <= 8 RB row blocks: block j of the group goes to slot
  // j / 8 of wave j % 8
  int blk[RB];
  int nvb = 0;   // row blocks of this wave holding at least one real row
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int j = kWaves * rb + wave;
    blk[rb] = rg * bpg + min(j, bpg - 1);
    if (j < bpg && blk[rb] * 16 < rows) nvb = rb + 1;
  }

  const int P = seq_len[b];
  const bool valid = P >= 0 && P + T <= Pmax;
  const int nkeys = valid ? P + T : 0;
  const int ntiles = (nkeys + kKT2 - 1) / kKT2;
  const int t_begin = split * tiles_per_split;
  const int nt = max(0, min(ntiles, t_begin + tiles_per_split) - t_begin);
  const int64_t kvbase = ((int64_t)b * nkv + g) * (int64_t)Pmax * D;

  // DMA issue j of this thread fills 1 KB region j*8 + wave of a tile: rows
  // ROWS_KB*region + lane/CPR, LDS chunk lane%CPR <- global chunk
  // (lane%CPR) ^ swz(row).  With 16 chunks per row swz(row) = (row & 7) << 1
  // (chunk bit 0 free): the K fragment reads pair neighbouring chunks of one
  // row (lanes 16 apart) and the transposing V reads neighbouring chunks of
  // four rows, and both then land on distinct banks (row & 15 made them
  // collide).
  auto swz = [](int row) { return CPR == 16 ? ((row & 7) << 1) : (row & SWZ); };
  int drow[NI], dcol[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    drow[j] = (j * kWaves + wave) * ROWS_KB + lane / CPR;
    dcol[j] = 8 * ((lane % CPR) ^ swz(drow[j]));
  }
  const uint32_t klds = lds_u32(&kbuf[0][0]), vlds = lds_u32(&vbuf[0][0]);
  auto issue = [&](int tile, int buf) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int64_t off = kvbase + (int64_t)min(tile * kKT2 + drow[j], Pmax - 1) * D + dcol[j];
      const uint32_t reg = (uint32_t)(buf * kKT2 * D * 2 + (j * kWaves + wave) * 1024);
      dma16_nt(Kc + off, __builtin_amdgcn_readfirstlane(klds + reg));
      dma16_nt(Vc + off, __builtin_amdgcn_readfirstlane(vlds + reg));
    }
  };

  // the first tiles go out before anything else
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i)
    if (i < nt) issue(t_begin + i, i);

  uint4 qf[RB][DS];
  int node[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rr = min(blk[rb] * 16 + r16, rows - 1);
    const int t = rr / G, hg = rr - t * G;
    node[rb] = t;
    const uint16_t* qp = Q + (((int64_t)b * T + t) * nq + g * G + hg) * D + 8 * g4;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[rb][ds] = ldg16(qp + 32 * ds);
  }
  for (int i = threadIdx.x; i < T * anc_words; i += kThreads)
    anc_s[(i / anc_words) * kMaxAncWords + i % anc_words] = anc[i];
  // every ordinary load (Q, ancestors) has landed: vmcnt(0), as the compiler
  // sees it, so no wait for Q is placed inside the tile loop
  __builtin_amdgcn_s_waitcnt(0x0F70);

  f32x4 acc[RB][DB];
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
  }

  // One tile in two halves of 32 keys (ks): S^T for the half, its softmax
  // update, then its share of O^T.  Halves keep the S^T accumulators of all RB
  // blocks small enough to live beside O^T.  Tiles wholly inside the prefix
  // (every key visible) take the unmasked path; the few tiles that reach the
  // tree slots or the end of the keys apply the ancestor mask.
  //   Softmax: each lane checks its own scores against the running max m (in
  //   log2 units); only when some lane exceeds m + 8 are the row maxima formed
  //   across the 4 lanes of a row and m raised (O^T and l rescaled), so the
  //   common path has no cross-lane traffic.  p = 2^(s*scale - m) <= 2^8.
  auto compute = [&](int tile, int buf, auto nv_tag) {
    constexpr int NV = decltype(nv_tag)::value;   // row blocks of this wave with real rows
    const int key0 = tile * kKT2;
    const bool masked = key0 + kKT2 > P;   // uniform: tile reaches the tree slots
    const uint16_t* kb_ = kbuf[buf];
    const uint16_t* vb_ = vbuf[buf];
#pragma unroll 1
    for (int ks = 0; ks < 2; ++ks) {
      f32x4 s[RB][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int rb = 0; rb < NV; ++rb) s[rb][h] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int krow = 32 * ks + 16 * h + r16;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const uint4 kf = *reinterpret_cast<const uint4*>(kb_ + krow * D + 8 * ((4 * ds + g4) ^ swz(krow)));
#pragma unroll
          for (int rb = 0; rb < NV; ++rb) s[rb][h] = mfma16x16x32(kf, qf[rb][ds], s[rb][h]);
        }
      }
      uint4 pb[NV];   // P^T slots 8*g4 + j <-> keys 32*ks + 16*(j/4) + 4*g4 + j%4
#pragma unroll
      for (int rb = 0; rb < NV; ++rb) {
        if (masked) {   // hidden scores become -inf, whose 2^x is 0
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = key0 + 32 * ks + 16 * h + 4 * g4 + i;
              const int j = key - P;
              const bool in_tree = (unsigned)j < (unsigned)T;
              const uint64_t w = anc_s[node[rb] * kMaxAncWords + (in_tree ? (j >> 6) : 0)];
              const bool vis = key < P || (in_tree && ((w >> (j & 63)) & 1ull));
              s[rb][h][i] = vis ? s[rb][h][i] : -INFINITY;
            }
        }
        float mo = -INFINITY;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) mo = fmaxf(mo, s[rb][h][i]);
        mo *= scale_log2;
        if (__any(mo > m_run[rb] + 8.0f)) {
          float rm = fmaxf(mo, __shfl_xor(mo, 16, 64));
          rm = fmaxf(rm, __shfl_xor(rm, 32, 64));
          const float m_new = rm > m_run[rb] + 8.0f ? rm : m_run[rb];
          const float alpha = m_run[rb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            acc[rb][db][0] *= alpha; acc[rb][db][1] *= alpha;
            acc[rb][db][2] *= alpha; acc[rb][db][3] *= alpha;
          }
          l_run[rb] *= alpha;
          m_run[rb] = m_new;
        }
        // m is -inf only while every score of the row so far is hidden
        const float nm = m_run[rb] == -INFINITY ? 0.f : -m_run[rb];
        float x[2][4];
        float psum = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[h][i] = __builtin_amdgcn_exp2f(fmaf(s[rb][h][i], scale_log2, nm));
            psum += x[h][i];
          }
        l_run[rb] += psum;
        pb[rb].x = pack_bf16x2(x[0][0], x[0][1]);
        pb[rb].y = pack_bf16x2(x[0][2], x[0][3]);
        pb[rb].z = pack_bf16x2(x[1][0], x[1][1]);
        pb[rb].w = pack_bf16x2(x[1][2], x[1][3]);
      }
      // lane j of group g4 addresses V[32*ks + 4*g4 + j/4 (+16)][16*db + 4*(j%4) .. +4];
      // the transposing read returns V[32*ks + 4*g4 + i (+16)][16*db + j], i = 0..3
      const int vrow = 32 * ks + 4 * g4 + (r16 >> 2);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int cb = 32 * db + 8 * (r16 & 3);
        const int ch = cb >> 4, he = (cb & 15) >> 1;
        const uint2 lo = lds_read_tr16(vb_ + vrow * D + 8 * (ch ^ swz(vrow)) + he);
        const uint2 hi = lds_read_tr16(vb_ + (vrow + 16) * D + 8 * (ch ^ swz(vrow + 16)) + he);
        uint4 va;
        va.x = lo.x; va.y = lo.y; va.z = hi.x; va.w = hi.y;
#pragma unroll
        for (int rb = 0; rb < NV; ++rb) acc[rb][db] = mfma16x16x32(va, pb[rb], acc[rb][db]);
      }
    }
  };

  // Waves whose last row blocks are empty skip them (MFMA work follows the
  // real rows); the tile loop is instantiated once per block count.
  auto run_tiles = [&](auto nv_tag) {
    for (int i = 0; i < nt; ++i) {
      // tiles issued after tile i so far: min(nt - 1 - i, NBUF - 2), 2*NI issues each
      const int ahead = min(nt - 1 - i, NBUF - 2);
      if (ahead >= 2) vm_wait<4 * NI>();
      else if (ahead == 1) vm_wait<2 * NI>();
      else vm_wait<0>();
      __syncthreads();   // tile i complete from every wave; tile i-1's buffer is free
      if (i + NBUF - 1 < nt) issue(t_begin + i + NBUF - 1, (i + NBUF - 1) % NBUF);
      if constexpr (decltype(nv_tag)::value > 0) compute(t_begin + i, i % NBUF, nv_tag);
    }
  };
  __syncthreads();   // anc_s
  if (nvb == RB) run_tiles(std::integral_constant<int, RB>{});
  else if (RB > 1 && nvb == RB - 1) run_tiles(std::integral_constant<int, RB - 1>{});
  else if (RB > 2 && nvb == 1) run_tiles(std::integral_constant<int, 1>{});
  else run_tiles(std::integral_constant<int, 0>{});

  // epilogue
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (rb >= nvb) continue;            // uniform: the slot holds no block of this group
    float l = l_run[rb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int row = blk[rb] * 16 + r16;
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
// Row groups, key partitions and ring depth.  With the 4-deep ring one
// workgroup fits a CU (two with the 64-wide head), and a workgroup's time per
// KV tile follows its busiest SIMD: block j of a group sits on SIMD j % 4, so
// a group of bpg row blocks costs about c0 + c1 ceil(bpg / 4) per tile
// (measured: 1.26 us with two blocks on a SIMD at the 7B batch-1 shape, 2.7 us
// with six at the 70B-layer shape).  Groups of one block per wave (128-wide
// head) may take the 2-deep ring instead: alone on a CU its tiles cost about
// 0.93x (the first tile lands sooner when each workgroup asks for one, not
// three: 7B batch 1, 18.8 against 20.2 us), and two workgroups can share a
// CU, each tile then taking about 1.7x as long with twice as many workgroups
// resident (7B batch 16, 512 workgroups: 170-186 us against 199-226 us).
// Two or three blocks per wave gain nothing from it (70B layer, 128k).
// Split keys add the merge: a launch, and the partials written and read back
// at about 5 TB/s.  The plan cuts a kv head's row blocks into equal groups of
// at most 24 and its keys into at most 16 partitions, taking the least
// (rounds of resident workgroups) x (tiles per partition) x (tile cost) +
// merge; ties go to the 4-deep ring, fewer groups, then fewer partitions.
AttnPlan attn_plan(int b, int T, int nq, int nkv, int d, int Pmax, int dtype) {
  AttnPlan p{1, 1, 1, 0, 1, 1, 4};
  if (dtype != kBF16) return p;
  const int G = nq / nkv;
  const int rows = T * G;
  const int nb = (rows + 15) / 16;                 // 16-row blocks per kv head
  const int tiles = (Pmax + kKT2 - 1) / kKT2;
  const long pairs = (long)b * nkv;
  constexpr double c0 = 0.54, c1 = 0.36;           // us per tile
  constexpr double merge_us = 2.5, bytes_per_us = 5e6;
  double best = -1.0;
  for (int nbuf = 4; nbuf >= 2; nbuf -= 2) {
    const long per_round = nbuf == 2 ? 512 : d == 64 ? 512 : 256;   // resident workgroups
    for (int groups = 1; groups <= nb; ++groups) {
      const int bpg = (nb + groups - 1) / groups;
      if (bpg > 3 * kWaves || (nb + bpg - 1) / bpg != groups) continue;
      if (nbuf == 2 && (d != 128 || bpg > kWaves)) continue;
      const double tile_us = c0 + c1 * ((bpg + 3) / 4);
      for (int want = 1; want <= kMaxSplit && want <= tiles; ++want) {
        const int tps = (tiles + want - 1) / want;
        const int ns = (tiles + tps - 1) / tps;
        const long wgs = pairs * groups * ns;
        const long rounds = (wgs + per_round - 1) / per_round;
        const double share = nbuf == 4 ? 1.0 : wgs <= 256 ? 0.93 : 1.7;
        double cost = (double)(rounds * tps) * tile_us * share;
        if (ns > 1) {
          const double partials = (double)wgs * bpg * 16 * (d * 4.0 + 8.0);
          cost += merge_us + 2.0 * partials / bytes_per_us;
        }
        if (best < 0 || cost < best - 1e-9) {
          best = cost;
          p.bpg = bpg;
          p.rowgroups = groups;
          p.nsplit = ns;
          p.tiles_per_split = tps;
          p.nbuf = nbuf;
        }
      }
    }
  }
  p.rb = (p.bpg + kWaves - 1) / kWaves;
  if (p.nsplit > 1) {
    const size_t rows_pad = (size_t)p.rowgroups * p.bpg * 16;
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
  const int rows = T * (nq / nkv);
  const int rows_pad = p.rowgroups * 16 * p.bpg;
  float* ws_o = static_cast<float*>(ws);
  float2* ws_ml = reinterpret_cast<float2*>(
      static_cast<char*>(ws) + (size_t)b * nkv * p.nsplit * rows_pad * d * sizeof(float));
  const int nblk = b * nkv * p.nsplit * p.rowgroups;
  const uint16_t* q = static_cast<const uint16_t*>(Q);
  const uint16_t* k = static_cast<const uint16_t*>(Kc);
  const uint16_t* v = static_cast<const uint16_t*>(Vc);
  uint16_t* o = static_cast<uint16_t*>(O);
#define ATTN(D_, RB_, NB_)                                                                     \
  hipLaunchKernelGGL((tree_attn_bf16<D_, RB_, NB_>), dim3(nblk), dim3(kThreads), 0, st, q, k, v, \
                     seq_len, anc, anc_words, T, nq, nkv, Pmax, scale_log2, p.nsplit,            \
                     p.rowgroups, p.bpg, p.tiles_per_split, o, ws_o, ws_ml)
  if (d == 128) {
    if (p.rb == 1 && p.nbuf == 2) ATTN(128, 1, 2);
    else if (p.rb == 1) ATTN(128, 1, 4);
    else if (p.rb == 2) ATTN(128, 2, 4);
    else ATTN(128, 3, 4);
  } else {
    if (p.rb == 1) ATTN(64, 1, 4);
    else if (p.rb == 2) ATTN(64, 2, 4);
    else ATTN(64, 3, 4);
  }
#undef ATTN
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

// ---------------------------------------------------------------- no-allocation variant
// medusa_tree_attn_noalloc keeps the split-KV partials in this file-scope
// device array instead of a caller workspace.  Each GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, so its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// passed to kernels.  Nothing in it needs to start at zero: every partial
// (output rows and (max, sum) pairs) is written by the attention kernel before
// attn_merge reads it.  Calls that overlap on one GPU share the array and race.
static __device__ __align__(256) unsigned char scratch[kAttnScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex scratch_mu;
static void* scratch_ptr[kMaxDevices];

size_t attn_scratch_bytes() { return kAttnScratchBytes; }

hipError_t attn_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace medusa
