// Device helpers shared by the Medusa HIP kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace medusa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kWave = 64;

// ---- bf16 <-> f32 -----------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// Two floats to packed bf16 with gfx950's v_cvt_pk_bf16_f32 (round to nearest
// even, as f32_to_bf16 for finite inputs).
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ---- MFMA ---------------------------------------------------------------------
// v_mfma_f32_16x16x32_bf16.  Lane l supplies A[l%16][slot 8*(l/16)+j] and
// B[slot 8*(l/16)+j][l%16], j = 0..7, and receives D[4*(l/16)+i][l%16],
// i = 0..3.  Kernels pair A and B slots themselves, so any fixed assignment
// of contraction indices to slots is valid as long as both operands use it.
__device__ __forceinline__ f32x4 mfma16x16x32(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---- loads ----------------------------------------------------------------------
__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// LDS DMA (gfx950 global_load_lds_dwordx4): each lane's 16 bytes from its own
// global address land at LDS byte m0 + 16 * lane.  The compiler does not see
// this write: the caller waits with vm_wait<N>() and a barrier before any
// wave reads the destination.  M0 is set in the same statement, one wait state
// ahead of its use.  The 64-bit address register is consumed at issue.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_addr)
               : "memory", "m0");
}
// The same with the non-temporal hint, for data read once per call (the K/V
// cache): it then displaces less of what later calls reuse (the weights) from
// the last-level cache.
__device__ __forceinline__ void dma16_nt(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(g), "s"(lds_addr)
               : "memory", "m0");
}
// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ uint32_t lds_u32(const void* p) { return (uint32_t)(uintptr_t)p; }

// ---- wave reductions ------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
// 64-bit wave max with DPP row operations instead of LDS-routed shuffles:
// quad xor 1, quad xor 2, half-row mirror and row mirror leave every lane of a
// 16-lane row with the row max; row broadcasts 15 and 31 fold rows into lane 63,
// which is then read as a scalar.  The result is the same in every lane.
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v, int ctrl_id) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  uint32_t tlo, thi;
  switch (ctrl_id) {
    case 0:  // quad_perm [1,0,3,2]
      tlo = __builtin_amdgcn_update_dpp(lo, lo, 0xB1, 0xF, 0xF, false);
      thi = __builtin_amdgcn_update_dpp(hi, hi, 0xB1, 0xF, 0xF, false);
      break;
    case 1:  // quad_perm [2,3,0,1]
      tlo = __builtin_amdgcn_update_dpp(lo, lo, 0x4E, 0xF, 0xF, false);
      thi = __builtin_amdgcn_update_dpp(hi, hi, 0x4E, 0xF, 0xF, false);
      break;
    case 2:  // row_half_mirror
      tlo = __builtin_amdgcn_update_dpp(lo, lo, 0x141, 0xF, 0xF, false);
      thi = __builtin_amdgcn_update_dpp(hi, hi, 0x141, 0xF, 0xF, false);
      break;
    case 3:  // row_mirror
      tlo = __builtin_amdgcn_update_dpp(lo, lo, 0x140, 0xF, 0xF, false);
      thi = __builtin_amdgcn_update_dpp(hi, hi, 0x140, 0xF, 0xF, false);
      break;
    case 4:  // row_bcast15 into rows 1 and 3
      tlo = __builtin_amdgcn_update_dpp(lo, lo, 0x142, 0xA, 0xF, false);
      thi = __builtin_amdgcn_update_dpp(hi, hi, 0x142, 0xA, 0xF, false);
      break;
    default:  // row_bcast31 into rows 2 and 3
      tlo = __builtin_amdgcn_update_dpp(lo, lo, 0x143, 0xC, 0xF, false);
      thi = __builtin_amdgcn_update_dpp(hi, hi, 0x143, 0xC, 0xF, false);
      break;
  }
  const uint64_t t = ((uint64_t)thi << 32) | tlo;
  return t > v ? t : v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step(v, 0);
  v = dpp_max_step(v, 1);
  v = dpp_max_step(v, 2);
  v = dpp_max_step(v, 3);
  v = dpp_max_step(v, 4);
  v = dpp_max_step(v, 5);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Online softmax statistics of a row x' (x' = logits / temperature):
// m = max x', s = sum e^(x'-m), t = sum e^(x'-m) (x'-m).  Then the entropy is
// H = ln s - t/s and log softmax(x')_i = x'_i - m - ln s.
struct RowStat {
  float m, s, t, pad;
};

__device__ __forceinline__ void stat_add(float& m, float& s, float& t, float x) {
  if (x <= m) {
    const float d = x - m;
    const float e = expf(d);
    s += e;
    t = fmaf(e, d, t);
  } else {
    if (s > 0.f) {
      const float d = m - x;          // < 0
      const float r = expf(d);
      t = r * fmaf(d, s, t);
      s = fmaf(r, s, 1.f);
    } else {
      s = 1.f;
      t = 0.f;
    }
    m = x;
  }
}

__device__ __forceinline__ void stat_merge(float& m, float& s, float& t, float m2, float s2,
                                           float t2) {
  if (s2 == 0.f) return;
  if (s == 0.f) {
    m = m2; s = s2; t = t2;
    return;
  }
  const float M = fmaxf(m, m2);
  const float d1 = m - M, d2 = m2 - M;
  const float r1 = expf(d1), r2 = expf(d2);
  t = r1 * fmaf(d1, s, t) + r2 * fmaf(d2, s2, t2);
  s = r1 * s + r2 * s2;
  m = M;
}

// ---- order-preserving key for (value desc, index asc) selection ---------------
// key = ord(x) << 32 | (0xffffffff - idx); a larger key is a larger value, and
// among equal values the lower index.  -0.0 is folded onto +0.0.  Key 0 is
// below every real key and marks an empty slot.
__device__ __forceinline__ uint32_t float_ord(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float ord_float(uint32_t o) {
  uint32_t b = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(b);
}
__device__ __forceinline__ uint64_t make_key(float x, uint32_t idx) {
  return ((uint64_t)float_ord(x) << 32) | (uint64_t)(0xffffffffu - idx);
}
__device__ __forceinline__ uint32_t key_index(uint64_t k) { return 0xffffffffu - (uint32_t)k; }
__device__ __forceinline__ float key_value(uint64_t k) { return ord_float((uint32_t)(k >> 32)); }

// Acceptance partial of one row over a range of its columns: the argmax key
// (greedy) or the online statistics of x' = x / temperature (typical).
struct RowPart {
  uint64_t key;
  float m, s, t;
};
__device__ __forceinline__ void part_init(RowPart& p) {
  p.key = 0;
  p.m = -INFINITY;
  p.s = 0.f;
  p.t = 0.f;
}
__device__ __forceinline__ void part_add(RowPart& p, float v, int n, bool typical, float inv_temp) {
  if (typical) {
    stat_add(p.m, p.s, p.t, v * inv_temp);
  } else {
    const uint64_t k = make_key(v, (uint32_t)n);
    p.key = k > p.key ? k : p.key;
  }
}
__device__ __forceinline__ void part_merge(RowPart& p, const RowPart& q, bool typical) {
  if (typical) stat_merge(p.m, p.s, p.t, q.m, q.s, q.t);
  else p.key = q.key > p.key ? q.key : p.key;
}
// merge with the partial of lane ^ o (only the fields of the mode move)
__device__ __forceinline__ void part_xor(RowPart& p, int o, bool typical) {
  RowPart q;
  if (typical) {
    q.m = __shfl_xor(p.m, o, 64);
    q.s = __shfl_xor(p.s, o, 64);
    q.t = __shfl_xor(p.t, o, 64);
  } else {
    q.key = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(p.key >> 32), o, 64) << 32) |
            (uint32_t)__shfl_xor((int)(uint32_t)p.key, o, 64);
  }
  part_merge(p, q, typical);
}

// Partial of NV values of one row held by a lane, at increasing columns col[k]
// (columns >= N are ignored): greedy takes the largest value and then its
// lowest column; typical forms (m, s, t) of x' = v / temperature in two passes
// (max, then the sums) with the hardware exponential.
template <int NV>
__device__ __forceinline__ RowPart lane_part(const float (&v)[NV], const int (&col)[NV], int N,
                                             bool typical, float inv_temp) {
  RowPart p;
  part_init(p);
  float mx = -INFINITY;
  bool any = false;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const bool ok = col[k] < N;
    const float x = typical ? v[k] * inv_temp : v[k];
    mx = ok ? fmaxf(mx, x) : mx;
    any = any || ok;
  }
  if (!any) return p;
  if (typical) {
    float s = 0.f, t = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const float d = v[k] * inv_temp - mx;
      const float e = col[k] < N ? __expf(d) : 0.f;
      s += e;
      t = fmaf(e, d, t);
    }
    p.m = mx;
    p.s = s;
    p.t = t;
  } else {
    int ci = 0;
#pragma unroll
    for (int k = NV - 1; k >= 0; --k) ci = (col[k] < N && v[k] == mx) ? col[k] : ci;
    p.key = make_key(mx, (uint32_t)ci);
  }
  return p;
}

// ---- counter-based uniform draws (SplitMix64, Steele/Lea/Flood 2014) ---------
__device__ __forceinline__ uint64_t splitmix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
// u in [0,1) with 24 random bits from (seed, step, seq, draw).
__device__ __forceinline__ double counter_uniform(uint64_t seed, uint64_t step, uint64_t seq,
                                                  uint64_t draw) {
  uint64_t x = splitmix64(seed ^ (step << 32) ^ (seq << 8) ^ draw);
  return (double)(x >> 40) * (1.0 / 16777216.0);
}

}  // namespace medusa
