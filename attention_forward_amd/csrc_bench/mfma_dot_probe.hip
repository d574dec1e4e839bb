// Dot-product precision of the matrix instructions the attention kernels use
// (a measurement for the tests, not part of the attention library).
//
// One single-wave workgroup per dot product w.  Every row of the A operand is
// a[w] and every column of the B operand is b[w], so each of the 32 x 32
// accumulator entries holds the same dot product, whatever the operands' lane
// layouts: steps chained instructions over K = 64 * steps E4M3 terms
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales, format 0) or
// K = 16 * steps bfloat16 terms (v_mfma_f32_32x32x16_bf16, format 1).  The
// wave stores the minimum and the maximum of its 1024 entries, so a caller
// can check that they agree and compare the value with an exact sum.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// lane l supplies k values 32 * (l / 32) .. +31 of each 64-term E4M3 step (the
// same bytes to A and B, so the pairing of a and b terms is exact)
__global__ __launch_bounds__(64) void dot_fp8_kernel(const unsigned char* __restrict__ a,
                                                     const unsigned char* __restrict__ b,
                                                     float* __restrict__ out, int steps) {
  const int w = blockIdx.x, g = threadIdx.x >> 5;
  f32x16 c = {};
  for (int s = 0; s < steps; ++s) {
    const size_t off = ((size_t)w * steps + s) * 64 + 32 * g;
    const unsigned* pa = reinterpret_cast<const unsigned*>(a + off);
    const unsigned* pb = reinterpret_cast<const unsigned*>(b + off);
    i32x8 av, bv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      av[e] = (int)pa[e];
      bv[e] = (int)pb[e];
    }
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
  }
  float lo = c[0], hi = c[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) {
    lo = fminf(lo, c[r]);
    hi = fmaxf(hi, c[r]);
  }
  for (int sh = 32; sh >= 1; sh >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, sh));
    hi = fmaxf(hi, __shfl_xor(hi, sh));
  }
  if (threadIdx.x == 0) {
    out[2 * (size_t)w] = lo;
    out[2 * (size_t)w + 1] = hi;
  }
}

// lane l supplies k values 8 * (l / 32) .. +7 of each 16-term bfloat16 step
__global__ __launch_bounds__(64) void dot_bf16_kernel(const uint16_t* __restrict__ a,
                                                      const uint16_t* __restrict__ b,
                                                      float* __restrict__ out, int steps) {
  const int w = blockIdx.x, g = threadIdx.x >> 5;
  f32x16 c = {};
  for (int s = 0; s < steps; ++s) {
    const size_t off = ((size_t)w * steps + s) * 16 + 8 * g;
    bf16x8 av, bv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      av[e] = __builtin_bit_cast(__bf16, a[off + e]);
      bv[e] = __builtin_bit_cast(__bf16, b[off + e]);
    }
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
  }
  float lo = c[0], hi = c[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) {
    lo = fminf(lo, c[r]);
    hi = fmaxf(hi, c[r]);
  }
  for (int sh = 32; sh >= 1; sh >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, sh));
    hi = fmaxf(hi, __shfl_xor(hi, sh));
  }
  if (threadIdx.x == 0) {
    out[2 * (size_t)w] = lo;
    out[2 * (size_t)w + 1] = hi;
  }
}

}  // namespace

extern "C" {

// n dot products of length 64 * steps (format 0: E4M3 bytes) or 16 * steps
// (format 1: bfloat16 bit patterns): a and b hold n * length elements each,
// dot product w taking elements [w * length, (w + 1) * length) of both; out
// receives 2 * n floats, (min, max) of the 1024 accumulator entries of each.
// Device pointers, 4-byte aligned; enqueued on `stream`.  Returns 0 on
// success, 1 for bad arguments (nothing launched), 2 for a HIP launch error.
int mfma_dot_probe(const void* a, const void* b, float* out, int n, int steps, int format,
                   void* stream) {
  if (!a || !b || !out || n <= 0 || steps <= 0 || steps > 64 || (format != 0 && format != 1) ||
      ((uintptr_t)a & 3) != 0 || ((uintptr_t)b & 3) != 0 || ((uintptr_t)out & 3) != 0)
    return 1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (format == 0)
    hipLaunchKernelGGL(dot_fp8_kernel, dim3((unsigned)n), dim3(64), 0, s,
                       static_cast<const unsigned char*>(a), static_cast<const unsigned char*>(b),
                       out, steps);
  else
    hipLaunchKernelGGL(dot_bf16_kernel, dim3((unsigned)n), dim3(64), 0, s,
                       static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), out,
                       steps);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
