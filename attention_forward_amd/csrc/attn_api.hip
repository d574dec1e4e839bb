// C ABI of libattn.so (declared in include/attn.h): argument validation, the
// thread-local error message, and dispatch to the kernel launchers.  Every
// check runs before the first HIP call, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "attn.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int check_device() {
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n <= 0)
    return fail(ATTN_ERR_NO_DEVICE, "no HIP device visible (%s)", hipGetErrorString(e));
  return ATTN_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ATTN_OK;
  return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

float fold_log2e(float scale) { return (float)((double)scale * 1.4426950408889634074); }

constexpr size_t kAlign = 256;
// rows of one head are addressed through a buffer descriptor whose byte range
// is 32-bit: S * 256 bytes must stay below 2^32
constexpr int kMaxSeq = (1 << 24) - 1;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// ---- the library-owned decode scratch (attn_fwd_decode_noalloc) ----
// One fixed buffer per GPU for the split partials of callers that cannot
// allocate.  In host code `scratch` names a host-side stand-in, not device
// memory: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels.  Every call on a GPU shares the buffer; the split kernel
// writes every partial it covers, so nothing needs clearing between calls.
constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices] = {};

// device address of this library's scratch on the device `stream` runs on
int scratch_address(hipStream_t stream, const char* fn, void** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: device of the stream: %s", fn,
                                   hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: device %d (at most %d devices)", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_addr[dev] == nullptr) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t restore = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess || p == nullptr)
      return fail(ATTN_ERR_HIP, "%s: address of the decode scratch on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    if (restore != hipSuccess)
      return fail(ATTN_ERR_HIP, "%s: restoring device %d: %s", fn, cur,
                  hipGetErrorString(restore));
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return ATTN_OK;
}

size_t decode_workspace_bytes(int B, int Hq, int d, int num_splits) {
  if (B <= 0 || Hq <= 0 || d <= 0 || num_splits <= 0) return 0;
  const size_t rows = (size_t)B * Hq * num_splits;
  return round_up(rows * d * sizeof(float)) + round_up(rows * sizeof(float));
}

// attn_fwd_decode with the caller's workspace, or (noalloc) the library's scratch
int decode(const char* fn, const void* q, const void* k, const void* v, void* o, float* lse, int B,
           int Hq, int Hkv, int Sk, int d, float scale, int dtype, int num_splits,
           void* workspace, size_t workspace_bytes, void* stream, bool noalloc) {
  g_err[0] = '\0';
  if (!q || !k || !v || !o) return fail(ATTN_ERR_NULL, "%s: q, k, v and o must be non-NULL", fn);
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sk <= 0 || d <= 0)
    return fail(ATTN_ERR_SHAPE, "%s: sizes must be positive", fn);
  if (Hq % Hkv != 0)
    return fail(ATTN_ERR_SHAPE, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (dtype != ATTN_F16 && dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
  if (!attn::head_dim_supported(d))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: head dim %d (64 and 128 are implemented)", fn, d);
  if (Hq / Hkv > 32)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: query heads per kv head %d > 32", fn, Hq / Hkv);
  if (num_splits < 1 || num_splits > Sk)
    return fail(ATTN_ERR_VALUE, "%s: num_splits=%d not in [1, Sk=%d]", fn, num_splits, Sk);
  if (!std::isfinite(scale) || scale < 0.0f)
    return fail(ATTN_ERR_VALUE, "%s: scale must be finite and >= 0", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse && !aligned4(lse)))
    return fail(ATTN_ERR_ALIGN, "%s: q, k, v, o must be 16-byte aligned, lse 4-byte", fn);
  const size_t need = decode_workspace_bytes(B, Hq, d, num_splits);
  if (noalloc) {
    if (need > kScratchBytes)
      return fail(ATTN_ERR_WORKSPACE,
                  "%s: the split partials need %zu bytes, above the library's %zu-byte scratch "
                  "(fewer splits or a smaller batch fit; attn_fwd_decode takes a workspace)",
                  fn, need, kScratchBytes);
  } else {
    if (!workspace || workspace_bytes < need)
      return fail(ATTN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(ATTN_ERR_ALIGN, "%s: misaligned workspace", fn);
  }
  if ((long long)B * Hkv * num_splits > INT_MAX || (long long)B * Hq > INT_MAX ||
      (long long)B * Hkv * Sk * d > (1LL << 46))
    return fail(ATTN_ERR_SHAPE, "%s: problem too large for one launch", fn);
  if (Sk > kMaxSeq) return fail(ATTN_ERR_SHAPE, "%s: Sk above %d", fn, kMaxSeq);
  int st = check_device();
  if (st != ATTN_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (noalloc) {
    st = scratch_address(s, fn, &workspace);
    if (st != ATTN_OK) return st;
  }
  const size_t rows = (size_t)B * Hq * num_splits;
  float* o_part = static_cast<float*>(workspace);
  float* lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             round_up(rows * d * sizeof(float)));
  attn::DecodeArgs da{q, k, v, o_part, lse_part, B, Hq, Hkv, Sk, d, num_splits,
                      fold_log2e(scale), dtype};
  st = hip_status(attn::launch_decode_split(da, s), "decode split launch");
  if (st != ATTN_OK) return st;
  attn::CombineArgs ca{o_part, lse_part, o, lse, B * Hq, num_splits, d, dtype};
  return hip_status(attn::launch_combine(ca, s), "decode combine launch");
}

}  // namespace

extern "C" {

const char* attn_last_error(void) { return g_err; }

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
             int Hkv, int Sq, int Sk, int d, int causal, float scale, int dtype, void* stream) {
  g_err[0] = '\0';
  if (!q || !k || !v || !o) return fail(ATTN_ERR_NULL, "attn_fwd: q, k, v and o must be non-NULL");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Sk <= 0 || d <= 0)
    return fail(ATTN_ERR_SHAPE, "attn_fwd: sizes must be positive (B=%d Hq=%d Hkv=%d Sq=%d Sk=%d d=%d)",
                B, Hq, Hkv, Sq, Sk, d);
  if (Hq % Hkv != 0)
    return fail(ATTN_ERR_SHAPE, "attn_fwd: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (dtype != ATTN_F16 && dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd: dtype %d is not 0 (fp16) or 1 (bf16)", dtype);
  if (!attn::head_dim_supported(d))
    return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd: head dim %d (64 and 128 are implemented)", d);
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_VALUE, "attn_fwd: causal must be 0 or 1");
  if (!std::isfinite(scale) || scale < 0.0f)
    return fail(ATTN_ERR_VALUE, "attn_fwd: scale must be finite and >= 0");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse && !aligned4(lse)))
    return fail(ATTN_ERR_ALIGN, "attn_fwd: q, k, v, o must be 16-byte aligned, lse 4-byte");
  const long long items = (long long)B * Hq * ((Sq + attn::FWD_BR - 1) / attn::FWD_BR);
  const long long q_elems = (long long)B * Hq * Sq * d;
  const long long kv_elems = (long long)B * Hkv * Sk * d;
  if (items > INT_MAX || q_elems > (1LL << 46) || kv_elems > (1LL << 46))
    return fail(ATTN_ERR_SHAPE, "attn_fwd: problem too large for one launch");
  if (Sq > kMaxSeq || Sk > kMaxSeq)
    return fail(ATTN_ERR_SHAPE, "attn_fwd: sequence length above %d", kMaxSeq);
  int st = check_device();
  if (st != ATTN_OK) return st;
  attn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, causal, fold_log2e(scale), dtype};
  return hip_status(attn::launch_fwd(a, static_cast<hipStream_t>(stream)), "attn_fwd launch");
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                 int Hkv, int Sq, int Sk, int d, int causal, float scale, float q_descale,
                 float k_descale, float v_descale, int out_dtype, void* stream) {
  g_err[0] = '\0';
  if (!q || !k || !v || !o) return fail(ATTN_ERR_NULL, "attn_fwd_fp8: q, k, v and o must be non-NULL");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Sk <= 0 || d <= 0)
    return fail(ATTN_ERR_SHAPE,
                "attn_fwd_fp8: sizes must be positive (B=%d Hq=%d Hkv=%d Sq=%d Sk=%d d=%d)", B, Hq,
                Hkv, Sq, Sk, d);
  if (Hq % Hkv != 0)
    return fail(ATTN_ERR_SHAPE, "attn_fwd_fp8: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (out_dtype != ATTN_F16 && out_dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_fp8: output dtype %d is not 0 (fp16) or 1 (bf16)",
                out_dtype);
  if (d != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_fp8: head dim %d (128 is implemented)", d);
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_VALUE, "attn_fwd_fp8: causal must be 0 or 1");
  const double folded = (double)scale * q_descale * k_descale;
  if (!std::isfinite(scale) || scale < 0.0f || !std::isfinite(q_descale) || q_descale <= 0.0f ||
      !std::isfinite(k_descale) || k_descale <= 0.0f || !std::isfinite(v_descale) ||
      v_descale <= 0.0f || !std::isfinite(folded * 1.4426950408889634074) ||
      !std::isfinite((float)(folded * 1.4426950408889634074)))
    return fail(ATTN_ERR_VALUE,
                "attn_fwd_fp8: scale must be finite and >= 0, descales finite and > 0");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse && !aligned4(lse)))
    return fail(ATTN_ERR_ALIGN, "attn_fwd_fp8: q, k, v, o must be 16-byte aligned, lse 4-byte");
  const long long items = (long long)B * Hq * ((Sq + attn::FWD_BR - 1) / attn::FWD_BR);
  const long long q_elems = (long long)B * Hq * Sq * d;
  const long long kv_elems = (long long)B * Hkv * Sk * d;
  if (items > INT_MAX || q_elems > (1LL << 46) || kv_elems > (1LL << 46))
    return fail(ATTN_ERR_SHAPE, "attn_fwd_fp8: problem too large for one launch");
  if (Sq > kMaxSeq || Sk > kMaxSeq)
    return fail(ATTN_ERR_SHAPE, "attn_fwd_fp8: sequence length above %d", kMaxSeq);
  int st = check_device();
  if (st != ATTN_OK) return st;
  attn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, causal,
                  (float)(folded * 1.4426950408889634074), out_dtype, v_descale, 1};
  return hip_status(attn::launch_fwd(a, static_cast<hipStream_t>(stream)), "attn_fwd_fp8 launch");
}

int attn_fwd_num_splits(int B, int Hq, int Sq, int Sk, int d) {
  if (B <= 0 || Hq <= 0 || Sq <= 0 || Sk <= 0 || !attn::head_dim_supported(d)) return 1;
  const long long items = (long long)B * Hq * ((Sq + attn::FWD_BR - 1) / attn::FWD_BR);
  const int tiles = (Sk + attn::FWD_KT - 1) / attn::FWD_KT;
  if (items >= attn::FWD_FILL_ITEMS) return 1;
  // enough splits for one workgroup per compute unit, keeping at least two
  // tiles per split (one-tile splits measured no faster: each split pays for
  // its Q load and fp32 partial round trip)
  const long long want = (attn::FWD_FILL_ITEMS + items - 1) / items;
  const long long cap = tiles / 2 > 1 ? tiles / 2 : 1;
  return (int)(want < cap ? want : cap);
}

size_t attn_fwd_split_workspace_bytes(int B, int Hq, int Sq, int d, int num_splits) {
  if (B <= 0 || Hq <= 0 || Sq <= 0 || d <= 0 || num_splits <= 0) return 0;
  const size_t rows = (size_t)B * Hq * Sq * num_splits;
  return round_up(rows * d * sizeof(float)) + round_up(rows * sizeof(float));
}

int attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int Hq, int Hkv, int Sq, int Sk, int d, int causal, float scale, int dtype,
                   int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = '\0';
  if (!q || !k || !v || !o)
    return fail(ATTN_ERR_NULL, "attn_fwd_split: q, k, v and o must be non-NULL");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Sk <= 0 || d <= 0)
    return fail(ATTN_ERR_SHAPE,
                "attn_fwd_split: sizes must be positive (B=%d Hq=%d Hkv=%d Sq=%d Sk=%d d=%d)", B,
                Hq, Hkv, Sq, Sk, d);
  if (Hq % Hkv != 0)
    return fail(ATTN_ERR_SHAPE, "attn_fwd_split: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (dtype != ATTN_F16 && dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_split: dtype %d is not 0 (fp16) or 1 (bf16)",
                dtype);
  if (!attn::head_dim_supported(d))
    return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_split: head dim %d (64 and 128 are implemented)",
                d);
  if (causal != 0 && causal != 1)
    return fail(ATTN_ERR_VALUE, "attn_fwd_split: causal must be 0 or 1");
  if (!std::isfinite(scale) || scale < 0.0f)
    return fail(ATTN_ERR_VALUE, "attn_fwd_split: scale must be finite and >= 0");
  if (Sq > kMaxSeq || Sk > kMaxSeq)
    return fail(ATTN_ERR_SHAPE, "attn_fwd_split: sequence length above %d", kMaxSeq);
  const int tiles = (Sk + attn::FWD_KT - 1) / attn::FWD_KT;
  if (num_splits < 1 || num_splits > tiles)
    return fail(ATTN_ERR_VALUE, "attn_fwd_split: num_splits=%d not in [1, %d] (64-key tiles)",
                num_splits, tiles);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse && !aligned4(lse)))
    return fail(ATTN_ERR_ALIGN, "attn_fwd_split: q, k, v, o must be 16-byte aligned, lse 4-byte");
  const size_t need = attn_fwd_split_workspace_bytes(B, Hq, Sq, d, num_splits);
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "attn_fwd_split: workspace of %zu bytes needed, %zu given",
                need, workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(ATTN_ERR_ALIGN, "attn_fwd_split: misaligned workspace");
  const long long items =
      (long long)B * Hq * ((Sq + attn::FWD_BR - 1) / attn::FWD_BR) * num_splits;
  const long long rows = (long long)B * Hq * Sq;
  if (items > INT_MAX || rows > INT_MAX || rows * d > (1LL << 46) ||
      (long long)B * Hkv * Sk * d > (1LL << 46))
    return fail(ATTN_ERR_SHAPE, "attn_fwd_split: problem too large for one launch");
  int st = check_device();
  if (st != ATTN_OK) return st;
  const size_t prow = (size_t)rows * num_splits;
  float* o_part = static_cast<float*>(workspace);
  float* lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             round_up(prow * d * sizeof(float)));
  // split s covers keys [s * split_keys, (s + 1) * split_keys): whole tiles,
  // as evenly as whole tiles allow (trailing splits may be short or empty)
  const int split_keys = (tiles + num_splits - 1) / num_splits * attn::FWD_KT;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  attn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, causal, fold_log2e(scale), dtype};
  attn::FwdSplitArgs sa{o_part, lse_part, num_splits, split_keys};
  st = hip_status(attn::launch_fwd_split(a, sa, hs), "attn_fwd_split partial launch");
  if (st != ATTN_OK) return st;
  attn::CombineArgs ca{o_part, lse_part, o, lse, (int)rows, num_splits, d, dtype};
  return hip_status(attn::launch_combine(ca, hs), "attn_fwd_split combine launch");
}

size_t attn_decode_workspace_bytes(int B, int Hq, int d, int num_splits) {
  return decode_workspace_bytes(B, Hq, d, num_splits);
}

int attn_splitkv_combine(const float* o_part, const float* lse_part, void* o, float* lse, int B,
                         int Hq, int d, int num_splits, int dtype, void* stream) {
  g_err[0] = '\0';
  if (!o_part || !lse_part || !o)
    return fail(ATTN_ERR_NULL, "attn_splitkv_combine: o_part, lse_part and o must be non-NULL");
  if (B <= 0 || Hq <= 0 || d <= 0)
    return fail(ATTN_ERR_SHAPE, "attn_splitkv_combine: sizes must be positive");
  if (num_splits <= 0) return fail(ATTN_ERR_VALUE, "attn_splitkv_combine: num_splits must be >= 1");
  if (dtype != ATTN_F16 && dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_splitkv_combine: dtype %d", dtype);
  if (!attn::head_dim_supported(d))
    return fail(ATTN_ERR_UNSUPPORTED,
                "attn_splitkv_combine: head dim %d (64 and 128 are implemented)", d);
  if (!aligned16(o_part) || !aligned4(lse_part) || !aligned16(o) || (lse && !aligned4(lse)))
    return fail(ATTN_ERR_ALIGN, "attn_splitkv_combine: misaligned pointer");
  if ((long long)B * Hq > INT_MAX)
    return fail(ATTN_ERR_SHAPE, "attn_splitkv_combine: too many rows");
  int st = check_device();
  if (st != ATTN_OK) return st;
  attn::CombineArgs a{o_part, lse_part, o, lse, B * Hq, num_splits, d, dtype};
  return hip_status(attn::launch_combine(a, static_cast<hipStream_t>(stream)),
                    "attn_splitkv_combine launch");
}

int attn_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int Hq, int Hkv, int Sk, int d, float scale, int dtype, int num_splits,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return decode("attn_fwd_decode", q, k, v, o, lse, B, Hq, Hkv, Sk, d, scale, dtype, num_splits,
                workspace, workspace_bytes, stream, false);
}

int attn_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int Sk, int d, float scale, int dtype,
                            int num_splits, void* stream) {
  return decode("attn_fwd_decode_noalloc", q, k, v, o, lse, B, Hq, Hkv, Sk, d, scale, dtype,
                num_splits, nullptr, 0, stream, true);
}

size_t attn_decode_scratch_bytes(void) { return kScratchBytes; }

}  // extern "C"
