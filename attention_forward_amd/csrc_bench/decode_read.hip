// Read ceiling shaped like the split-KV decode, for the benchmark (not part of
// the attention library).
//
// The decode kernel's memory side without its math: one single-wave
// workgroup per (kv head, split) with 64 KiB of dynamic LDS (two per compute
// unit), K and V tiles of 16 KiB (64 keys of 128 bf16) moved by non-temporal
// direct-to-LDS loads, each of the two buffers re-issued as soon as its tile
// has landed, one tile ahead.  Two forms: the tiles of K and V from two arrays
// (the decode's two streams per workgroup), or from one array with a tile's K
// and V bytes adjacent (a single stream).  What the decode loses against the
// first is its compute and waits; against the second, also its layout.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int TILE = 16384;  // bytes of one K or V tile
constexpr int CHUNKS = TILE / 1024;
constexpr unsigned LDS_BYTES = 65536;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const unsigned char* base) {
  // raw buffer over one tile; gfx9 word 3 for 32-bit data
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(base), (short)0, TILE,
                                           0x00020000);
}

// s_waitcnt on vmcnt only (gfx9 encoding, the other counters at their maxima)
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <bool ONE_STREAM>
__global__ __launch_bounds__(64, 2) void decode_read_kernel(const unsigned char* __restrict__ k,
                                                            const unsigned char* __restrict__ v,
                                                            int tiles, unsigned* __restrict__ sink) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  typedef __attribute__((address_space(3))) unsigned char lds_byte;
  lds_byte* kt = (lds_byte*)smem;
  lds_byte* vt = kt + TILE;
  const int lane = threadIdx.x;
  const size_t wg = blockIdx.x;
  const size_t step = ONE_STREAM ? 2 * TILE : TILE;
  const unsigned char* kb = k + wg * tiles * step;
  const unsigned char* vb = ONE_STREAM ? kb + TILE : v + wg * tiles * step;
  auto issue = [&](const unsigned char* base, int t, lds_byte* dst) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(base + t * step);
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + c * 1024),
                                               16, lane * 16 + c * 1024, 0, 0, 2);
  };
  issue(kb, 0, kt);
  issue(vb, 0, vt);
  for (int t = 0; t < tiles; ++t) {
    const bool more = t + 1 < tiles;
    vm_wait<CHUNKS>();  // K(t); V(t) may be in flight
    if (more) issue(kb, t + 1, kt);
    if (more)
      vm_wait<CHUNKS>();  // V(t); K(t+1) may be in flight
    else
      vm_wait<0>();
    if (more) issue(vb, t + 1, vt);
  }
  vm_wait<0>();
  // keep the loads: a store only for contents the benchmark's zeroed buffers never hold
  if (lane == 0 && kt[0] == 0x5a && vt[0] == 0x5a) sink[0] = 1;
}

}  // namespace

extern "C" {

// Reads `workgroups` x `tiles` tiles of K and of V (16 KiB each) on `stream`:
// from k and v (one_stream = 0; each holds workgroups * tiles * 16 KiB) or
// from k alone (one_stream = 1; 2 * workgroups * tiles * 16 KiB, v unused).
// Pointers 16-byte aligned.  Returns 0 on success, 1 for bad arguments, 2 for
// a HIP launch error.
int decode_read(const void* k, const void* v, int workgroups, int tiles, int one_stream,
                unsigned* sink, void* stream) {
  if (!k || !sink || (!one_stream && !v) || workgroups <= 0 || tiles <= 0 ||
      ((uintptr_t)k & 15) != 0 || (!one_stream && ((uintptr_t)v & 15) != 0))
    return 1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (one_stream)
    hipLaunchKernelGGL((decode_read_kernel<true>), dim3((unsigned)workgroups), dim3(64),
                       LDS_BYTES, s, static_cast<const unsigned char*>(k),
                       static_cast<const unsigned char*>(k), tiles, sink);
  else
    hipLaunchKernelGGL((decode_read_kernel<false>), dim3((unsigned)workgroups), dim3(64),
                       LDS_BYTES, s, static_cast<const unsigned char*>(k),
                       static_cast<const unsigned char*>(v), tiles, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
