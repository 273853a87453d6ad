// Plain streaming read of a device buffer: the yardstick for the weight
// streams (the heads' and LM passes read 134 MB and 262 MB once each at the
// 7B shape, and the pages put the step's cost in that memory traffic:
// aicassindra.com "Medusa deep dive", "What it costs on a CPU-bound SLM").
// It computes nothing of the method; bench.py times it on buffers of the
// weight streams' sizes to give the rate this part reaches for a read of
// that many bytes, next to the 8 TB/s of the specification.
//
// The fastest plain read found on MI355X (134 MB, 262 MB and 1 GiB, three
// rotated buffers so the last-level cache cannot serve them): direct
// global->LDS loads with the non-temporal hint, 256 workgroups of 8 waves,
// each wave two 1 KB loads per group (at most four in flight), grid-stride
// over 1 KB units: 22.1 us, 40.7 us and 154 us.  Loads into registers (four
// 16-byte loads in flight per thread, 512 workgroups of 256 threads) took
// 24.3, 45.8 and 178 us; LDS DMA without the hint 23.5, 45.4 and 179 us;
// four or eight loads per group, or 512 workgroups, 2-15% longer.
// Each lane folds the 16 bytes it brought in by XOR (read back from LDS) and
// writes its fold to sink only when it equals the caller's `never`, so every
// word is seen by some lane and nothing can be dropped; the last partial
// 1 KB unit is read into registers by the first workgroup.

#include "common.h"
#include "kernels.h"

namespace medusa {

constexpr int kReadWaves = 8;
constexpr int kReadBlocks = 256;
constexpr int kReadGroup = 2;          // 1 KB loads per wave and group

__global__ __launch_bounds__(64 * kReadWaves) void stream_read(const uint8_t* __restrict__ p,
                                                               size_t bytes, uint32_t never,
                                                               uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint4 lds[kReadWaves][2][kReadGroup][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const size_t units = bytes >> 10;
  const size_t tw = (size_t)gridDim.x * kReadWaves;
  size_t u = (size_t)blockIdx.x * kReadWaves + wave;
  uint32_t acc = 0;
  auto fold = [&](const uint4& v) { acc ^= v.x ^ v.y ^ v.z ^ v.w; };
  int slot = 0;
  for (; u + (size_t)(kReadGroup - 1) * tw < units; u += (size_t)kReadGroup * tw) {
#pragma unroll
    for (int j = 0; j < kReadGroup; ++j)
      dma16_nt(p + (u + (size_t)j * tw) * 1024 + 16 * lane,
               __builtin_amdgcn_readfirstlane(lds_u32(&lds[wave][slot][j][0])));
    // the previous group (the other slot) has landed; fold it
    vm_wait<kReadGroup>();
    if (u >= (size_t)kReadGroup * tw) {
#pragma unroll
      for (int j = 0; j < kReadGroup; ++j) fold(lds[wave][slot ^ 1][j][lane]);
    }
    // the other slot is refilled next group only after these reads
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    slot ^= 1;
  }
  vm_wait<0>();
  if (u >= (size_t)kReadGroup * tw) {
#pragma unroll
    for (int j = 0; j < kReadGroup; ++j) fold(lds[wave][slot ^ 1][j][lane]);
  }
  for (; u < units; u += tw) fold(*reinterpret_cast<const uint4*>(p + u * 1024 + 16 * lane));
  if (blockIdx.x == 0) {
    const size_t tail = bytes & 1023;
    for (size_t o = 16 * (size_t)threadIdx.x; o < tail; o += 16 * 64 * kReadWaves)
      fold(*reinterpret_cast<const uint4*>(p + (units << 10) + o));
  }
  if (acc == never) sink[0] = acc;
}

hipError_t run_stream_read(const void* buf, size_t bytes, uint32_t never, uint32_t* sink,
                           hipStream_t st) {
  hipLaunchKernelGGL(stream_read, dim3(kReadBlocks), dim3(64 * kReadWaves), 0, st,
                     static_cast<const uint8_t*>(buf), bytes, never, sink);
  return hipGetLastError();
}

}  // namespace medusa
