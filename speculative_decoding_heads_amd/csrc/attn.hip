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

constexpr int kKT = 64;             // keys per tile
constexpr int kMaxF32Keys = 16384;  // f32 kernel keeps scores in LDS

__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int x = b & 7, j = b >> 3;
  const int q = total >> 3, r = total & 7;
  return x * q + min(x, r) + j;
}

template <int D, int RB>
__global__ __launch_bounds__(256) void tree_attn_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
    const uint16_t* __restrict__ Vc, const int* __restrict__ seq_len,
    const uint64_t* __restrict__ anc, int anc_words, int T, int nq, int nkv, int Pmax,
    float scale_log2, int nsplit, int rowgroups, int tiles_per_split, uint16_t* __restrict__ O,
    float* __restrict__ ws_o, float2* __restrict__ ws_ml) {
  constexpr int KS = D + 8;    // LDS row stride of K (elements): +16 B against bank conflicts
  constexpr int VS = kKT + 8;  // LDS row stride of V^T
  constexpr int DS = D / 32;   // MFMA steps over the head dim
  constexpr int DB = D / 16;   // 16-wide blocks of the head dim
  constexpr int KLOADS = D / 32;  // 16-byte K loads per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t ks[kKT * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * VS];

  const int total = gridDim.x;
  const int tile_id = xcd_remap(blockIdx.x, total);
  const int rg = tile_id % rowgroups;
  const int rest = tile_id / rowgroups;
  const int split = rest % nsplit;
  const int bg = rest / nsplit;
  const int b = bg / nkv, g = bg - b * nkv;
  const int G = nq / nkv;
  const int rows = T * G;
  const int rows_pad = rowgroups * 64 * RB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;

  const int P = seq_len[b];
  const bool valid = P >= 0 && P + T <= Pmax;
  const int nkeys = valid ? P + T : 0;
  const int ntiles = (nkeys + kKT - 1) / kKT;
  const int t_begin = split * tiles_per_split;
  const int t_end = min(ntiles, t_begin + tiles_per_split);
  const int64_t kvbase = ((int64_t)b * nkv + g) * (int64_t)Pmax * D;

  uint4 qf[RB][DS];
  uint64_t aw[RB][kMaxAncWords];
  f32x4 acc[RB][DB];
  float m_run[RB], l_run[RB];
  int row_id[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = rg * 64 * RB + wave * 16 * RB + rb * 16 + r16;
    row_id[rb] = row;
    const int rr = min(row, rows - 1);
    const int t = rr / G, hg = rr - t * G;
    const uint16_t* qp = Q + (((int64_t)b * T + t) * nq + g * G + hg) * D + 8 * g4;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[rb][ds] = ldg16(qp + 32 * ds);
#pragma unroll
    for (int w = 0; w < kMaxAncWords; ++w) aw[rb][w] = w < anc_words ? anc[(int64_t)t * anc_words + w] : 0ull;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
  }

  // tile loaders: K rows (4 threads per key), V as (4 keys) x (8 dims) per thread
  const int kkey = threadIdx.x >> 2, kpart = threadIdx.x & 3;
  const int vkq = threadIdx.x & 15, vdc = threadIdx.x >> 4;
  const bool vact = vdc < D / 8;
  uint4 kr[KLOADS], vr[4];
  auto load_tile = [&](int tile) {
    const int key0 = tile * kKT;
    const int kk = min(key0 + kkey, Pmax - 1);
    const uint16_t* src = Kc + kvbase + (int64_t)kk * D + kpart * (D / 4);
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) kr[i] = ldg16(src + 8 * i);
    if (vact) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int vk = min(key0 + 4 * vkq + i, Pmax - 1);
        vr[i] = ldg16(Vc + kvbase + (int64_t)vk * D + 8 * vdc);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KLOADS; ++i)
      *reinterpret_cast<uint4*>(&ks[kkey * KS + kpart * (D / 4) + 8 * i]) = kr[i];
    if (vact) {
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vr[0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vr[1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vr[2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vr[3]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sh = (j & 1) * 16;
        const uint32_t e0 = (w0[j >> 1] >> sh) & 0xffffu, e1 = (w1[j >> 1] >> sh) & 0xffffu;
        const uint32_t e2 = (w2[j >> 1] >> sh) & 0xffffu, e3 = (w3[j >> 1] >> sh) & 0xffffu;
        uint2 pk;
        pk.x = e0 | (e1 << 16);
        pk.y = e2 | (e3 << 16);
        *reinterpret_cast<uint2*>(&vt[(8 * vdc + j) * VS + 4 * vkq]) = pk;
      }
    }
  };

  if (t_begin < t_end) load_tile(t_begin);
  for (int tile = t_begin; tile < t_end; ++tile) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (tile + 1 < t_end) load_tile(tile + 1);
    const int key0 = tile * kKT;
    const bool tree_tile = key0 + kKT > P;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint16_t* kp = &ks[(16 * kb + r16) * KS + 8 * g4];
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
          s[kb] = mfma16x16x32(*reinterpret_cast<const uint4*>(kp + 32 * ds), qf[rb][ds], s[kb]);
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
            const uint64_t w = j < 64 ? aw[rb][0] : j < 128 ? aw[rb][1] : j < 192 ? aw[rb][2] : aw[rb][3];
            vis = (w >> (j & 63)) & 1ull;
          }
          x[kb][i] = vis ? s[kb][i] * scale_log2 : -INFINITY;
          mt = fmaxf(mt, x[kb][i]);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_run[rb], mt);
      float alpha = 1.f;
      float psum = 0.f;
      if (m_new != -INFINITY) {
        alpha = exp2f(m_run[rb] - m_new);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[kb][i] = exp2f(x[kb][i] - m_new);
            psum += x[kb][i];
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[kb][i] = 0.f;
      }
      m_run[rb] = m_new;
      l_run[rb] = l_run[rb] * alpha + psum;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        acc[rb][db][0] *= alpha; acc[rb][db][1] *= alpha;
        acc[rb][db][2] *= alpha; acc[rb][db][3] *= alpha;
      }
#pragma unroll
      for (int kstep = 0; kstep < 2; ++kstep) {
        uint4 pb;
        pb.x = pack_bf16x2(x[2 * kstep][0], x[2 * kstep][1]);
        pb.y = pack_bf16x2(x[2 * kstep][2], x[2 * kstep][3]);
        pb.z = pack_bf16x2(x[2 * kstep + 1][0], x[2 * kstep + 1][1]);
        pb.w = pack_bf16x2(x[2 * kstep + 1][2], x[2 * kstep + 1][3]);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint16_t* vp = &vt[(16 * db + r16) * VS + 32 * kstep + 4 * g4];
          const uint2 lo = *reinterpret_cast<const uint2*>(vp);
          const uint2 hi = *reinterpret_cast<const uint2*>(vp + 16);
          uint4 va;
          va.x = lo.x; va.y = lo.y; va.z = hi.x; va.w = hi.y;
          acc[rb][db] = mfma16x16x32(va, pb, acc[rb][db]);
        }
      }
    }
  }

  // epilogue
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float l = l_run[rb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int row = row_id[rb];
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
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ws_ml[((int64_t)bg * nsplit + s) * rows_pad + row].x);
  float den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const int64_t prow = ((int64_t)bg * nsplit + s) * rows_pad + row;
    const float2 ml = ws_ml[prow];
    if (ml.x == -INFINITY) continue;
    const float w = exp2f(ml.x - M);
    den += w * ml.y;
    const f32x4 o = *reinterpret_cast<const f32x4*>(ws_o + prow * D + c);
    num[0] += w * o[0]; num[1] += w * o[1]; num[2] += w * o[2]; num[3] += w * o[3];
  }
  const float inv = 1.0f / den;
  const int t = row / G, hg = row - t * G;
  uint16_t* op = O + (((int64_t)b * T + t) * nq + g * G + hg) * D + c;
  uint2 o;
  o.x = pack_bf16x2(num[0] * inv, num[1] * inv);
  o.y = pack_bf16x2(num[2] * inv, num[3] * inv);
  *reinterpret_cast<uint2*>(op) = o;
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
  p.rb = rows > 64 ? 2 : 1;
  p.rowgroups = (rows + 64 * p.rb - 1) / (64 * p.rb);
  const int tiles = (Pmax + kKT - 1) / kKT;
  const int base = b * nkv * p.rowgroups;
  int want = (768 + base - 1) / base;
  int maxsplit = tiles / 2 > 0 ? tiles / 2 : 1;
  p.nsplit = want < maxsplit ? want : maxsplit;
  if (p.nsplit < 1) p.nsplit = 1;
  if (p.nsplit > 1) {
    const size_t rows_pad = (size_t)p.rowgroups * 64 * p.rb;
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
  const int tiles = (Pmax + kKT - 1) / kKT;
  const int tps = (tiles + p.nsplit - 1) / p.nsplit;
  const int rows = T * (nq / nkv);
  const int rows_pad = p.rowgroups * 64 * p.rb;
  float* ws_o = static_cast<float*>(ws);
  float2* ws_ml = reinterpret_cast<float2*>(
      static_cast<char*>(ws) + (size_t)b * nkv * p.nsplit * rows_pad * d * sizeof(float));
  const int nblk = b * nkv * p.nsplit * p.rowgroups;
  const uint16_t* q = static_cast<const uint16_t*>(Q);
  const uint16_t* k = static_cast<const uint16_t*>(Kc);
  const uint16_t* v = static_cast<const uint16_t*>(Vc);
  uint16_t* o = static_cast<uint16_t*>(O);
#define ATTN(D_, RB_)                                                                          \
  hipLaunchKernelGGL((tree_attn_bf16<D_, RB_>), dim3(nblk), dim3(256), 0, st, q, k, v, seq_len, \
                     anc, anc_words, T, nq, nkv, Pmax, scale_log2, p.nsplit, p.rowgroups, tps, o, \
                     ws_o, ws_ml)
  if (d == 128) {
    if (p.rb == 2) ATTN(128, 2); else ATTN(128, 1);
  } else {
    if (p.rb == 2) ATTN(64, 2); else ATTN(64, 1);
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

}  // namespace medusa
