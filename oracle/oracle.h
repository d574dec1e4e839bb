/*
 * FP64 CPU oracle for the attention forward pass.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test-suite, the package smoke check and the benchmark's CPU-baseline
 * leg may load this library.  The product path never calls it, and it shares no
 * code, header, table or helper with the GPU library.
 *
 * What it computes (plain definition, score rows materialised, no tiling):
 *   for each query row i of head (b, hq), with kv head hkv = hq / (Hq / Hkv):
 *     s_j = scale * sum_c q[i,c] * k[j,c]                    (all j, FP64)
 *     visible set: all j, or j <= i + (Sk - Sq) when causal
 *     m = max_visible s_j ;  p_j = exp(s_j - m) ;  l = sum p_j
 *     O[i,:] = sum_j (p_j / l) v[j,:] ;  LSE[i] = m + ln(l)
 *     no visible key: O = 0, LSE = -inf
 * Sources: "The FA5090 Optimization Journey" sec. 2.1 (an oracle in higher
 * precision plus a same-dtype reference define the correctness gate) and
 * sec. 2.2 (the naive kernel materialises the score matrix); "10 rounds of
 * hand-written fused attention ..." , "The correctness trap" (an f64 CPU
 * reference from the first kernel).
 *
 * The "same-dtype reference" additionally rounds each normalised P_j to the
 * input dtype (IEEE round-to-nearest-even) before the P.V product, accumulates
 * in FP64 and rounds O to the input dtype.
 *
 * Inputs are raw 16-bit patterns (dtype 0 = IEEE binary16, 1 = bfloat16),
 * contiguous row-major: q [B,Hq,Sq,d], k and v [B,Hkv,Sk,d].
 * Every function returns 0 on success and a negative value on bad arguments.
 */
#ifndef ATTN_ORACLE_H
#define ATTN_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Decode n 16-bit patterns of the given dtype to doubles (exact). */
int oracle_decode(const uint16_t* in, int64_t n, int dtype, double* out);

/* Round n doubles to the dtype with round-to-nearest-even; writes bit patterns. */
int oracle_round(const double* in, int64_t n, int dtype, uint16_t* out);

/*
 * Attention for a list of flattened query rows r = (b*Hq + hq)*Sq + i.
 * o: [n_rows, d] exact result.  lse: [n_rows] natural-log LSE.
 * o_ref (may be NULL): [n_rows, d] same-dtype reference, already rounded to
 * the dtype and widened back to double.  nthreads <= 0: OpenMP default.
 */
int oracle_attention_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int dtype,
                          int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, double scale,
                          const int64_t* rows, int64_t n_rows,
                          double* o, double* lse, double* o_ref, int nthreads);

/*
 * Split-KV partials of a single-query (decode) attention: keys are cut into
 * num_splits consecutive chunks of ceil(Sk/num_splits) keys (the last may be
 * short or empty).  For chunk s: o_part[b,hq,s,:] is the attention output over
 * that chunk alone and lse_part[b,hq,s] its natural-log LSE; an empty chunk has
 * o_part = 0 and lse_part = -inf.  q: [B,Hq,1,d]; k,v: [B,Hkv,Sk,d].
 */
int oracle_split_partials(const uint16_t* q, const uint16_t* k, const uint16_t* v, int dtype,
                          int B, int Hq, int Hkv, int Sk, int d, double scale, int num_splits,
                          double* o_part, double* lse_part);

/*
 * Merge split partials: M = max_s lse_s ; w_s = exp(lse_s - M) ; L = sum w_s ;
 * O = sum_s (w_s / L) o_s ; LSE = M + ln L.  All lse_s = -inf gives O = 0,
 * LSE = -inf.  o_part [R, num_splits, d], lse_part [R, num_splits] with
 * R = number of (b, hq) rows; o [R, d], lse [R].
 */
int oracle_combine(const double* o_part, const double* lse_part, int64_t R, int d, int num_splits,
                   double* o, double* lse);

/*
 * OCP 8-bit floating point, E4M3 with no infinities ("E4M3FN"; the OCP 8-bit
 * Floating Point Specification, OFP8): 1 sign, 4 exponent bits (bias 7),
 * 3 fraction bits; subnormals m * 2^-9; S.1111.111 is NaN; largest finite
 * magnitude 448.  Decode is exact; rounding is to nearest, ties to even, with
 * magnitudes beyond 448 saturated to 448.
 */
int oracle_decode_e4m3(const uint8_t* in, int64_t n, double* out);
int oracle_round_e4m3(const double* in, int64_t n, uint8_t* out);

/*
 * FP8 attention.  q, k, v hold E4M3 patterns; the real inputs are
 * q8 * q_descale, k8 * k_descale and v8 * v_descale (per-tensor scales).  o
 * and lse are the plain definition above on those real values.
 * o_ref (may be NULL) is the FP8 reference: the unnormalised weights
 * exp(s_j - m) (m the exact row max, so each is in (0, 1]) are rounded to
 * E4M3 before the product with V, the sum of the unrounded weights
 * normalises, and O is rounded to out_dtype (0 = binary16, 1 = bfloat16).
 * An FP8 kernel can only round the weights it feeds to the matrix unit, which
 * are unnormalised; the normalisation follows in fp32.
 */
int oracle_attention_fp8_rows(const uint8_t* q, const uint8_t* k, const uint8_t* v, int B, int Hq,
                              int Hkv, int Sq, int Sk, int d, int causal, double scale,
                              double q_descale, double k_descale, double v_descale, int out_dtype,
                              const int64_t* rows, int64_t n_rows, double* o, double* lse,
                              double* o_ref, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
