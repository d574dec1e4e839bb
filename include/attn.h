/*
 * attn.h -- C ABI of the gfx950 FlashAttention forward library (libattn.so).
 *
 * What is computed.  Per (batch b, query head hq), with kv head
 * hkv = hq / (Hq / Hkv) (contiguous groups of query heads share one K/V head):
 *
 *     O[i,:] = sum_j softmax_j( scale * q_i . k_j  [+ causal mask] ) v_j
 *     LSE[i] = ln sum_{visible j} exp(scale * q_i . k_j)
 *
 * computed with an online softmax whose running max and sum are carried across
 * key tiles, so the score matrix never leaves the chip ("The FA5090
 * Optimization Journey", sec. 2.2 and 2.6; "10 rounds of hand-written fused
 * attention ...", "The trajectory", round R8).  Inputs are IEEE binary16 or
 * bfloat16; products accumulate in fp32; O has the input dtype; LSE is fp32.
 *
 * Causal masking: key j is visible to query i iff j <= i + (Sk - Sq)
 * (bottom-right aligned; j <= i when Sq == Sk).  A query row that sees no key
 * gets O = 0 and LSE = -inf.
 *
 * Layout.  Every tensor is contiguous row-major with d innermost:
 *     q, o: [B, Hq, Sq, d]      k, v: [B, Hkv, Sk, d]      lse: [B, Hq, Sq]
 * All data pointers are device pointers, 16-byte aligned, owned by the caller.
 * The library allocates nothing and keeps no state between calls; the one
 * exception is attn_fwd_decode_noalloc's fixed per-GPU scratch (below).
 *
 * Streams.  Work is enqueued on `stream` (a hipStream_t; NULL = the default
 * stream) and the call returns before it completes.  Concurrent calls on
 * different streams are independent.
 *
 * Errors.  Arguments are validated before any HIP call; a failing check
 * returns its status and enqueues nothing.  A HIP launch error returns
 * ATTN_ERR_HIP.  attn_last_error() then describes the failure (thread-local).
 * The library never aborts, exits or throws across this interface.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_F16 = 0, ATTN_BF16 = 1 } attn_dtype;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* non-positive size, Hq % Hkv != 0, Sq or Sk >= 2^24, size overflow */
  ATTN_ERR_UNSUPPORTED = 3, /* valid but not implemented: d not 64 or 128, dtype, GQA group > 32 */
  ATTN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  ATTN_ERR_WORKSPACE = 5,   /* split workspace missing or too small */
  ATTN_ERR_NO_DEVICE = 6,   /* no HIP device visible */
  ATTN_ERR_HIP = 7,         /* a HIP call failed; see attn_last_error() */
  ATTN_ERR_VALUE = 8        /* bad scalar: causal not 0/1, scale negative or not finite,
                               descale not positive, num_splits out of range */
} attn_status;

/*
 * Prefill / full forward pass.
 *   q, k, v  : inputs (dtype given by `dtype`), layouts above.
 *   o        : output [B,Hq,Sq,d], same dtype as the inputs.
 *   lse      : fp32 [B,Hq,Sq] natural-log LSE of the scaled scores over the
 *              visible keys; may be NULL when not wanted.
 *   scale    : multiplies q.k before the softmax (usually 1/sqrt(d)); >= 0.
 *   causal   : 0 or 1.
 *   d        : head dimension; 64 and 128 are implemented.
 * The exponentials run in base 2 with scale*log2(e) folded into one multiply
 * ("The FA5090 Optimization Journey", sec. 2.6; "G5: Pipeline ...", V33).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, float scale,
             int dtype, void* stream);

/*
 * FP8 prefill: attn_fwd on OCP E4M3 ("E4M3FN": 1 sign, 4 exponent bits with
 * bias 7, 3 fraction bits, no infinities, max 448) inputs with per-tensor
 * scales.  The real inputs are q8 * q_descale, k8 * k_descale and
 * v8 * v_descale; q, k, v hold the E4M3 bytes in the layouts above (1 byte per
 * element).  Both products run on the FP8 matrix unit with fp32
 * accumulation: the scores directly from the bytes (scale * q_descale *
 * k_descale * log2(e) folded into one fp32 multiply), and P.V with the
 * unnormalised softmax weights rounded to E4M3 (taken against the exact
 * running max, so they are at most 1, inside the format's range); V's descale
 * multiplies O before it is rounded to out_dtype.  LSE is fp32 as in attn_fwd.  The pages measured an
 * FP8 arm and rejected it on their hardware, for lack of an 8-bit operand load
 * and for accuracy ("The FA5090 Optimization Journey", scope and sec. 3, the
 * comparison with FA3 and FA4); the MI355X matrix unit runs FP8 at twice the
 * 16-bit rate, and this entry point is judged by its own accuracy gate.
 *   d = 128 only; out_dtype 0 (fp16) or 1 (bf16); descales finite and > 0.
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, float scale,
                 float q_descale, float k_descale, float v_descale, int out_dtype,
                 void* stream);

/*
 * Split-KV prefill for grids too small to fill the chip (few batch*head
 * pairs, short queries).  The same result as attn_fwd, up to rounding, computed
 * by cutting the keys into num_splits ranges of whole 64-key tiles, as evenly as
 * whole tiles allow (split s covers keys [s*c, (s+1)*c) with
 * c = 64*ceil(ceil(Sk/64)/num_splits); trailing splits may be short or empty),
 * attending to each range independently with fp32 partial outputs, and merging
 * them by their LSEs (attn_splitkv_combine).  The pages measured split-KV as a
 * scheduling lever for under-filled prefill grids ("The FA5090 Optimization
 * Journey", sec. 2.7, the fourth lever; a loss there because the fp32 round
 * trip missed L2); here it is a separate entry point that a caller picks,
 * e.g. with attn_fwd_num_splits.
 *   Arguments as attn_fwd, plus:
 *   num_splits: in [1, ceil(Sk/64)].
 *   workspace : device buffer of at least attn_fwd_split_workspace_bytes(...)
 *               bytes, owned by the caller; its contents on entry are ignored.
 * Enqueues the partial kernel, then the combine kernel, on `stream`.
 */
int attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, float scale,
                   int dtype, int num_splits, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * Bytes of device workspace attn_fwd_split needs: fp32 partial outputs
 * [B,Hq,Sq,num_splits,d] followed (256-byte aligned) by fp32 partial LSEs
 * [B,Hq,Sq,num_splits].  Returns 0 for invalid arguments.
 */
size_t attn_fwd_split_workspace_bytes(int B, int Hq, int Sq, int d, int num_splits);

/*
 * Recommended num_splits for attn_fwd_split: 1 when attn_fwd's grid (B*Hq
 * blocks of 256 query rows) already has one workgroup per compute unit (256),
 * else enough splits to reach that, with at least two 64-key tiles per split.
 * Returns 1 for invalid arguments.
 */
int attn_fwd_num_splits(int B, int Hq, int Sq, int Sk, int d);

/*
 * Bytes of device workspace attn_fwd_decode needs: fp32 partial outputs
 * [B,Hq,num_splits,d] followed (256-byte aligned) by fp32 partial LSEs
 * [B,Hq,num_splits].  Returns 0 for invalid arguments.
 */
size_t attn_decode_workspace_bytes(int B, int Hq, int d, int num_splits);

/*
 * Single-token decode with split-KV: the same result as attn_fwd with Sq = 1
 * and causal = 0, computed by cutting the Sk keys into num_splits consecutive
 * chunks of ceil(Sk/num_splits) keys, attending to each chunk independently
 * (one read of each K/V row serves all Hq/Hkv query heads of its group), and
 * merging the partial results by their LSEs (attn_splitkv_combine).  Split-KV
 * as a way to spread one row's keys over more of the chip: "The FA5090
 * Optimization Journey", sec. 2.7.
 *   q, o     : [B,Hq,1,d]; k, v: [B,Hkv,Sk,d]; lse: fp32 [B,Hq] or NULL.
 *   num_splits in [1, Sk]; Hq/Hkv <= 32; d is 64 or 128.
 *   workspace: device buffer of at least attn_decode_workspace_bytes(...)
 *              bytes, owned by the caller; its contents on entry are ignored.
 * Enqueues the split kernel, then the combine kernel, on `stream`.
 */
int attn_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int Sk, int d, float scale, int dtype,
                    int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_fwd_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid allocation.  The split partials go to a buffer the
 * library owns, one fixed array of attn_decode_scratch_bytes() bytes (32 MiB)
 * per GPU, held from the library's load until the process ends; nothing is
 * allocated, on the device or the host, by this call.
 *   Arguments, result and errors as attn_fwd_decode; ATTN_ERR_WORKSPACE when
 *   attn_decode_workspace_bytes(B,Hq,d,num_splits) exceeds the scratch (the
 *   64 x 32 x 16-split decode needs 16.9 MB of it).
 * Every call on one GPU shares that GPU's scratch, and the buffer keeps the
 * last call's partials: calls that overlap on one GPU (on different streams,
 * or from several host threads without ordering) race and give wrong results.
 * Serialise them, e.g. on one stream.
 */
int attn_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int Sk, int d, float scale, int dtype,
                            int num_splits, void* stream);

/* Size in bytes of the per-GPU scratch attn_fwd_decode_noalloc uses. */
size_t attn_decode_scratch_bytes(void);

/*
 * Merge split partials: for each of the B*Hq rows,
 *     M = max_s lse_s,  w_s = exp(lse_s - M),  L = sum_s w_s,
 *     O = sum_s (w_s / L) o_s  (rounded to dtype),  LSE = M + ln L.
 * A row whose partial LSEs are all -inf gets O = 0 and LSE = -inf.  This is the
 * online-softmax merge of two running states applied across splits ("The FA5090
 * Optimization Journey", sec. 2.6, the running max and the final 1/l).
 *   o_part  : fp32 [B,Hq,num_splits,d], each partial already normalised; d is 64 or 128.
 *   lse_part: fp32 [B,Hq,num_splits], natural log.
 *   o       : [B,Hq,d] in dtype;  lse: fp32 [B,Hq] or NULL.
 */
int attn_splitkv_combine(const float* o_part, const float* lse_part, void* o, float* lse,
                         int B, int Hq, int d, int num_splits, int dtype, void* stream);

/* Description of the last non-OK status returned on this thread ("" if none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
