// HBM read-stream ceiling for the benchmark (not part of the attention library).
//
// Every 16-byte word of a buffer is read exactly once per launch by
// non-temporal vector loads (streaming data, as the split-KV decode reads
// its K and V; plain loads measured ~12% slower), UNROLL words in flight per
// lane, and folded into a value that is stored only if it equals a constant
// the benchmark's zero-filled buffer never produces.  The best rate over a
// few launch shapes is the practical read bandwidth that an HBM-bound kernel
// (the split-KV decode) can be held against, beside the published peak.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int UNROLL = 8;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ void stream_read_kernel(const uint4* __restrict__ p, size_t n_words,
                                   unsigned* __restrict__ sink) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  unsigned acc = 0;
  for (; i + (UNROLL - 1) * stride < n_words; i += UNROLL * stride) {
    uint4 w[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(&p[i + u * stride]));
      w[u].x = x[0];
      w[u].y = x[1];
      w[u].z = x[2];
      w[u].w = x[3];
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  for (; i < n_words; i += stride) acc ^= p[i].x ^ p[i].y ^ p[i].z ^ p[i].w;
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` bytes at device pointer `buf` (16-byte aligned, bytes a multiple
// of 16) with `blocks` workgroups of `threads` threads (a multiple of 64, at
// most 1024) on `stream`.  `sink`: a device word that receives a value only for
// a buffer whose folded contents match the constant above.  Returns 0 on
// success, 1 for bad arguments, 2 for a HIP launch error.
int stream_read(const void* buf, size_t bytes, unsigned* sink, int blocks, int threads,
                void* stream) {
  if (!buf || !sink || bytes % 16 != 0 || ((uintptr_t)buf & 15) != 0 || blocks <= 0 ||
      threads <= 0 || threads > 1024 || threads % 64 != 0)
    return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3((unsigned)threads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
