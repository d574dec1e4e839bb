// Internal launchers shared between the kernel sources and the C ABI layer.
// Arguments are already validated by the caller; each launcher only enqueues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// the head dimensions the kernels implement
constexpr bool head_dim_supported(int d) { return d == 64 || d == 128; }

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Sq, Sk, d;
  int causal;
  float scale_log2;  // scale * log2(e) (* Q and K descales in FP8), rounded once to fp32 on the host
  int dtype;         // of O (and of Q, K, V unless fp8)
  float o_scale = 1.0f;  // multiplies O (V's descale in FP8)
  int fp8 = 0;           // Q, K, V are OCP E4M3 (head dimension 128)
};

// split-KV prefill: partial outputs of num_splits key ranges of split_keys
// keys each (a multiple of the 64-key tile)
struct FwdSplitArgs {
  float* o_part;    // [B, Hq, Sq, num_splits, d] fp32
  float* lse_part;  // [B, Hq, Sq, num_splits] fp32, natural log
  int num_splits;
  int split_keys;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o_part;    // [B, Hq, num_splits, d] fp32
  float* lse_part;  // [B, Hq, num_splits] fp32, natural log
  int B, Hq, Hkv, Sk, d;
  int num_splits;
  float scale_log2;
  int dtype;
};

struct CombineArgs {
  const float* o_part;
  const float* lse_part;
  void* o;
  float* lse;
  int rows;  // B * Hq
  int num_splits;
  int d;
  int dtype;
};

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_split(const FwdArgs& a, const FwdSplitArgs& sa, hipStream_t stream);
hipError_t launch_decode_split(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

// Which wave groups of the prefill kernel issue the K/V tile loads
// (0: group A, 1: group B, 2: both, half each; 3: both, half each, in their
// softmax phases, with three stages per ring).  -1: the scheme each input
// format measured best with (its LOAD_MODE).
#ifndef ATTN_LOADERS
#define ATTN_LOADERS -1
#endif

// Number of 32-query blocks per wave and waves per workgroup of the prefill kernel.
#ifndef ATTN_FWD_QB
#define ATTN_FWD_QB 1
#endif
#ifndef ATTN_FWD_NW
#define ATTN_FWD_NW 8
#endif
#ifndef ATTN_FWD_WPE
#define ATTN_FWD_WPE 2
#endif
constexpr int FWD_QB = ATTN_FWD_QB;
constexpr int FWD_NW = ATTN_FWD_NW;
constexpr int FWD_WAVES_PER_SIMD = ATTN_FWD_WPE;  // occupancy the register budget is sized for
constexpr int FWD_BR = FWD_QB * FWD_NW * 32;  // query rows per workgroup
constexpr int FWD_KT = 64;                     // keys per K/V tile
// prefill work items below which the split-KV form is recommended: one
// workgroup per compute unit
constexpr int FWD_FILL_ITEMS = 256;

}  // namespace attn
