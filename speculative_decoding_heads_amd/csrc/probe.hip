// Plain streaming read of a device buffer: the yardstick for the weight
// streams (the heads' and LM passes read 134 MB and 262 MB once each at the
// 7B shape, and the pages put the step's cost in that memory traffic:
// aicassindra.com "Medusa deep dive", "What it costs on a CPU-bound SLM").
// It computes nothing of the method; bench.py times it on buffers of the
// weight streams' sizes to give the rate this part reaches for a read of
// that many bytes, next to the 8 TB/s of the specification.
//
// Layout chosen by a sweep on MI355X (134 MB, 262 MB and 1 GiB, three
// rotated buffers so the last-level cache cannot serve them): 512 workgroups
// of 256 threads (two per CU), each thread four 16-byte loads in flight,
// grid-stride.  Eight loads in flight, or four and eight workgroups per CU,
// were 5-20% slower; a contiguous region per workgroup (as a GEMM workgroup
// reads its weight rows) 2-5% slower at 134 MB.

#include "common.h"
#include "kernels.h"

namespace medusa {

constexpr int kReadThreads = 256;
constexpr int kReadBlocks = 512;
constexpr int kReadUnroll = 4;

// Each thread folds the words it loaded by XOR and writes its fold to sink
// only when it equals the caller's `never`, so the loads cannot be dropped
// (for a value no fold takes, nothing is written).
__global__ __launch_bounds__(kReadThreads) void stream_read(const uint4* __restrict__ p, size_t n16,
                                                            uint32_t never,
                                                            uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  size_t i = blockIdx.x * (size_t)kReadThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == never) sink[0] = acc;
}

hipError_t run_stream_read(const void* buf, size_t bytes, uint32_t never, uint32_t* sink,
                           hipStream_t st) {
  hipLaunchKernelGGL(stream_read, dim3(kReadBlocks), dim3(kReadThreads), 0, st,
                     static_cast<const uint4*>(buf), bytes / 16, never, sink);
  return hipGetLastError();
}

}  // namespace medusa
