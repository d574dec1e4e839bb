/*
 * FP64 CPU oracle for the attention forward pass.  TEST INFRASTRUCTURE ONLY:
 * loaded by the tests, the smoke check and the benchmark's CPU-baseline leg,
 * never by the product path.  It shares no code with the GPU library.
 *
 * The definitions implemented here are stated in oracle.h with their sources.
 * Plain C, one query row at a time, the whole score row materialised, FP64
 * throughout, OpenMP across rows.  No tiling, no online softmax, no exp2 trick.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- 16-bit float formats, written from the IEEE 754 / bfloat16 layouts ---- */

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
 * bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
typedef struct {
  int frac_bits;
  int exp_bits;
  int bias;
} fmt16;

static const fmt16 FMT[2] = {{10, 5, 15}, {7, 8, 127}};

static double decode1(uint16_t h, const fmt16* f) {
  int sign = (h >> 15) & 1;
  int e = (h >> f->frac_bits) & ((1 << f->exp_bits) - 1);
  int m = h & ((1 << f->frac_bits) - 1);
  int emax = (1 << f->exp_bits) - 1;
  double v;
  if (e == emax) {
    v = m ? NAN : INFINITY;
  } else if (e == 0) {
    /* subnormal: m * 2^(1 - bias - frac_bits) */
    v = ldexp((double)m, 1 - f->bias - f->frac_bits);
  } else {
    v = ldexp((double)((1 << f->frac_bits) + m), e - f->bias - f->frac_bits);
  }
  return sign ? -v : v;
}

/* Round |x| to the format with round-to-nearest, ties to even; returns bits. */
static uint16_t round1(double x, const fmt16* f) {
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  int emax = (1 << f->exp_bits) - 1;
  if (isnan(x)) return (uint16_t)(sign | (emax << f->frac_bits) | (1 << (f->frac_bits - 1)));
  double a = fabs(x);
  if (isinf(a)) return (uint16_t)(sign | (emax << f->frac_bits));
  if (a == 0.0) return sign;
  /* unbiased exponent of a: a = g * 2^ex with g in [0.5, 1) */
  int ex;
  frexp(a, &ex);
  int e = ex - 1;                      /* a in [2^e, 2^(e+1)) */
  int emin = 1 - f->bias;              /* smallest normal exponent */
  int qexp = (e < emin ? emin : e) - f->frac_bits; /* quantum = 2^qexp */
  double q = ldexp(a, -qexp);          /* exact: scaling by a power of two */
  double fl = floor(q);
  double rem = q - fl;                 /* exact */
  double r = fl;
  if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) r = fl + 1.0;
  /* r is the significand in units of the quantum; re-normalise */
  long long n = (long long)r;
  int be;                               /* biased exponent */
  if (e < emin) {
    /* subnormal range; rounding may carry into the smallest normal */
    if (n >= (1LL << f->frac_bits)) {
      be = 1;
      n -= (1LL << f->frac_bits);
    } else {
      be = 0;
    }
  } else {
    be = e + f->bias;
    if (n >= (2LL << f->frac_bits)) { /* carried to the next binade */
      n >>= 1;
      be += 1;
    }
    n -= (1LL << f->frac_bits);
  }
  if (be >= emax) return (uint16_t)(sign | (emax << f->frac_bits)); /* overflow to inf */
  return (uint16_t)(sign | (be << f->frac_bits) | (uint16_t)n);
}

int oracle_decode(const uint16_t* in, int64_t n, int dtype, double* out) {
  if (dtype < 0 || dtype > 1 || n < 0 || (n && (!in || !out))) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = decode1(in[i], &FMT[dtype]);
  return 0;
}

int oracle_round(const double* in, int64_t n, int dtype, uint16_t* out) {
  if (dtype < 0 || dtype > 1 || n < 0 || (n && (!in || !out))) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = round1(in[i], &FMT[dtype]);
  return 0;
}

/* ---- attention, one query row ---- */

/* Computes O, LSE (and the same-dtype reference) for query row i of head (b, hq).
 * s: scratch of Sk doubles; qd, kd, vd: the row / head slices already decoded. */
static void attend_row(const double* qrow, const double* kh, const double* vh, int Sk, int d,
                       int nvis, double scale, double* s, double* o, double* lse, double* o_ref,
                       const fmt16* f) {
  for (int c = 0; c < d; ++c) o[c] = 0.0;
  if (o_ref)
    for (int c = 0; c < d; ++c) o_ref[c] = 0.0;
  if (nvis <= 0) {
    *lse = -INFINITY;
    return;
  }
  (void)Sk;
  /* scores of the visible keys 0 .. nvis-1 */
  double m = -INFINITY;
  for (int j = 0; j < nvis; ++j) {
    double acc = 0.0;
    const double* kr = kh + (int64_t)j * d;
    for (int c = 0; c < d; ++c) acc += qrow[c] * kr[c];
    s[j] = scale * acc;
    if (s[j] > m) m = s[j];
  }
  /* max-subtracted softmax */
  double l = 0.0;
  for (int j = 0; j < nvis; ++j) {
    s[j] = exp(s[j] - m);
    l += s[j];
  }
  for (int j = 0; j < nvis; ++j) {
    double p = s[j] / l;
    const double* vr = vh + (int64_t)j * d;
    for (int c = 0; c < d; ++c) o[c] += p * vr[c];
    if (o_ref) {
      double pr = decode1(round1(p, f), f);
      for (int c = 0; c < d; ++c) o_ref[c] += pr * vr[c];
    }
  }
  *lse = m + log(l);
  if (o_ref)
    for (int c = 0; c < d; ++c) o_ref[c] = decode1(round1(o_ref[c], f), f);
}

/* ---- OCP 8-bit E4M3 (the "FN" variant: no infinities), from the format's
 * definition: 1 sign, 4 exponent bits (bias 7), 3 fraction bits; exponent
 * field 0 holds subnormals m * 2^-9; S.1111.111 is NaN, so the largest finite
 * magnitude is S.1111.110 = 1.75 * 2^8 = 448. ---- */
static double decode_e4m3(uint8_t b) {
  int sign = (b >> 7) & 1;
  int e = (b >> 3) & 15;
  int m = b & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 7 - 3);
  return sign ? -v : v;
}

/* Round to E4M3 with round-to-nearest, ties to even; magnitudes past 448
 * saturate to 448 (the format has no infinity); NaN stays NaN. */
static uint8_t round_e4m3(double x) {
  uint8_t sign = signbit(x) ? 0x80u : 0u;
  if (isnan(x)) return (uint8_t)(sign | 0x7Fu);
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);
  int ex;
  frexp(a, &ex);
  int e = ex - 1;                     /* a in [2^e, 2^(e+1)) */
  int qexp = (e < -6 ? -6 : e) - 3;   /* quantum: 2^-9 for subnormals, 2^(e-3) else */
  double q = ldexp(a, -qexp);
  double fl = floor(q);
  double rem = q - fl;
  double r = fl;
  if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) r = fl + 1.0;
  /* the value is r * 2^qexp; re-encode it (a carry may reach the next binade) */
  double y = ldexp(r, qexp);
  if (y >= 448.0) return (uint8_t)(sign | 0x7Eu);
  if (y < ldexp(1.0, -6)) return (uint8_t)(sign | (uint8_t)r); /* subnormal: m = r */
  frexp(y, &ex);
  e = ex - 1;
  int m = (int)(ldexp(y, 3 - e)) - 8;
  return (uint8_t)(sign | ((e + 7) << 3) | m);
}

int oracle_decode_e4m3(const uint8_t* in, int64_t n, double* out) {
  if (n < 0 || (n && (!in || !out))) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = decode_e4m3(in[i]);
  return 0;
}

int oracle_round_e4m3(const double* in, int64_t n, uint8_t* out) {
  if (n < 0 || (n && (!in || !out))) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = round_e4m3(in[i]);
  return 0;
}

static int check_shapes(int B, int Hq, int Hkv, int Sq, int Sk, int d);

int oracle_attention_fp8_rows(const uint8_t* q, const uint8_t* k, const uint8_t* v, int B, int Hq,
                              int Hkv, int Sq, int Sk, int d, int causal, double scale,
                              double q_descale, double k_descale, double v_descale, int out_dtype,
                              const int64_t* rows, int64_t n_rows, double* o, double* lse,
                              double* o_ref, int nthreads) {
  if (out_dtype < 0 || out_dtype > 1 || check_shapes(B, Hq, Hkv, Sq, Sk, d)) return -1;
  if (!q || !k || !v || !rows || !o || !lse || n_rows < 0) return -1;
  const int64_t total_rows = (int64_t)B * Hq * Sq;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= total_rows) return -2;
  const fmt16* f = &FMT[out_dtype];
  const int group = Hq / Hkv;
  /* the real inputs are q8 * q_descale etc.; the descales of q and k only
   * scale the scores, v's scales the output */
  const double s_scale = scale * q_descale * k_descale;
  int err = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Sk);
    double* qd = (double*)malloc(sizeof(double) * (size_t)d);
    double* kd = (double*)malloc(sizeof(double) * (size_t)Sk * d);
    double* vd = (double*)malloc(sizeof(double) * (size_t)Sk * d);
    int64_t cached_head = -1;
    if (!s || !qd || !kd || !vd) {
#pragma omp atomic write
      err = -3;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (err) continue;
      int64_t row = rows[r];
      int i = (int)(row % Sq);
      int64_t bh = row / Sq;
      int hq = (int)(bh % Hq);
      int b = (int)(bh / Hq);
      int64_t kv_head = (int64_t)b * Hkv + hq / group;
      if (kv_head != cached_head) {
        const uint8_t* kh = k + kv_head * Sk * d;
        const uint8_t* vh = v + kv_head * Sk * d;
        for (int64_t e = 0; e < (int64_t)Sk * d; ++e) {
          kd[e] = decode_e4m3(kh[e]);
          vd[e] = v_descale * decode_e4m3(vh[e]);
        }
        cached_head = kv_head;
      }
      const uint8_t* qr = q + row * d;
      for (int c = 0; c < d; ++c) qd[c] = decode_e4m3(qr[c]);
      int64_t last = causal ? (int64_t)i + (Sk - Sq) : (int64_t)Sk - 1;
      int nvis = last < 0 ? 0 : (last >= Sk ? Sk : (int)(last + 1));
      double* orow = o + r * d;
      attend_row(qd, kd, vd, Sk, d, nvis, s_scale, s, orow, lse + r, NULL, f);
      if (o_ref) {
        /* s[0 .. nvis) now holds the weights exp(s_j - m) against the row max */
        double* oref = o_ref + r * d;
        double l = 0.0;
        for (int c = 0; c < d; ++c) oref[c] = 0.0;
        for (int j = 0; j < nvis; ++j) {
          l += s[j];
          double pr = decode_e4m3(round_e4m3(s[j]));
          const double* vr = vd + (int64_t)j * d;
          for (int c = 0; c < d; ++c) oref[c] += pr * vr[c];
        }
        for (int c = 0; c < d; ++c)
          oref[c] = nvis > 0 ? decode1(round1(oref[c] / l, f), f) : 0.0;
      }
    }
    free(s);
    free(qd);
    free(kd);
    free(vd);
  }
  return err;
}

static int check_shapes(int B, int Hq, int Hkv, int Sq, int Sk, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Sk <= 0 || d <= 0) return -1;
  if (Hq % Hkv != 0) return -1;
  return 0;
}

int oracle_attention_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int dtype,
                          int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, double scale,
                          const int64_t* rows, int64_t n_rows, double* o, double* lse, double* o_ref,
                          int nthreads) {
  if (dtype < 0 || dtype > 1 || check_shapes(B, Hq, Hkv, Sq, Sk, d)) return -1;
  if (!q || !k || !v || !rows || !o || !lse || n_rows < 0) return -1;
  const int64_t total_rows = (int64_t)B * Hq * Sq;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= total_rows) return -2;
  const fmt16* f = &FMT[dtype];
  const int group = Hq / Hkv;
  int err = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Sk);
    double* qd = (double*)malloc(sizeof(double) * (size_t)d);
    double* kd = (double*)malloc(sizeof(double) * (size_t)Sk * d);
    double* vd = (double*)malloc(sizeof(double) * (size_t)Sk * d);
    int64_t cached_head = -1; /* (b, hkv) whose K, V are decoded in kd, vd */
    if (!s || !qd || !kd || !vd) {
#pragma omp atomic write
      err = -3;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (err) continue;
      int64_t row = rows[r];
      int i = (int)(row % Sq);
      int64_t bh = row / Sq;
      int hq = (int)(bh % Hq);
      int b = (int)(bh / Hq);
      int hkv = hq / group;
      int64_t kv_head = (int64_t)b * Hkv + hkv;
      if (kv_head != cached_head) {
        const uint16_t* kh = k + kv_head * Sk * d;
        const uint16_t* vh = v + kv_head * Sk * d;
        for (int64_t e = 0; e < (int64_t)Sk * d; ++e) {
          kd[e] = decode1(kh[e], f);
          vd[e] = decode1(vh[e], f);
        }
        cached_head = kv_head;
      }
      const uint16_t* qr = q + row * d;
      for (int c = 0; c < d; ++c) qd[c] = decode1(qr[c], f);
      /* visible keys: j <= i + (Sk - Sq) when causal, i.e. a prefix */
      int64_t last = causal ? (int64_t)i + (Sk - Sq) : (int64_t)Sk - 1;
      int nvis = last < 0 ? 0 : (last >= Sk ? Sk : (int)(last + 1));
      attend_row(qd, kd, vd, Sk, d, nvis, scale, s, o + r * d, lse + r, o_ref ? o_ref + r * d : NULL,
                 f);
    }
    free(s);
    free(qd);
    free(kd);
    free(vd);
  }
  return err;
}

int oracle_split_partials(const uint16_t* q, const uint16_t* k, const uint16_t* v, int dtype,
                          int B, int Hq, int Hkv, int Sk, int d, double scale, int num_splits,
                          double* o_part, double* lse_part) {
  if (dtype < 0 || dtype > 1 || check_shapes(B, Hq, Hkv, 1, Sk, d)) return -1;
  if (!q || !k || !v || !o_part || !lse_part || num_splits <= 0) return -1;
  const fmt16* f = &FMT[dtype];
  const int group = Hq / Hkv;
  const int chunk = (Sk + num_splits - 1) / num_splits;
  const int64_t R = (int64_t)B * Hq;
  int err = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)chunk);
    double* qd = (double*)malloc(sizeof(double) * (size_t)d);
    double* kd = (double*)malloc(sizeof(double) * (size_t)chunk * d);
    double* vd = (double*)malloc(sizeof(double) * (size_t)chunk * d);
    if (!s || !qd || !kd || !vd) {
#pragma omp atomic write
      err = -3;
    }
#pragma omp for schedule(dynamic, 1) collapse(2)
    for (int64_t bh = 0; bh < R; ++bh) {
      for (int sp = 0; sp < num_splits; ++sp) {
        if (err) continue;
        int hq = (int)(bh % Hq), b = (int)(bh / Hq);
        int64_t kv_head = (int64_t)b * Hkv + hq / group;
        int j0 = sp * chunk;
        int n = Sk - j0;
        if (n > chunk) n = chunk;
        if (n < 0) n = 0;
        for (int c = 0; c < d; ++c) qd[c] = decode1(q[bh * d + c], f);
        for (int64_t e = 0; e < (int64_t)n * d; ++e) {
          kd[e] = decode1(k[(kv_head * Sk + j0) * d + e], f);
          vd[e] = decode1(v[(kv_head * Sk + j0) * d + e], f);
        }
        attend_row(qd, kd, vd, n, d, n, scale, s, o_part + (bh * num_splits + sp) * d,
                   lse_part + bh * num_splits + sp, NULL, f);
      }
    }
    free(s);
    free(qd);
    free(kd);
    free(vd);
  }
  return err;
}

int oracle_combine(const double* o_part, const double* lse_part, int64_t R, int d, int num_splits,
                   double* o, double* lse) {
  if (!o_part || !lse_part || !o || !lse || R < 0 || d <= 0 || num_splits <= 0) return -1;
  for (int64_t r = 0; r < R; ++r) {
    const double* ls = lse_part + r * num_splits;
    double M = -INFINITY;
    for (int s = 0; s < num_splits; ++s)
      if (ls[s] > M) M = ls[s];
    double* orow = o + r * d;
    for (int c = 0; c < d; ++c) orow[c] = 0.0;
    if (M == -INFINITY) {
      lse[r] = -INFINITY;
      continue;
    }
    double L = 0.0;
    for (int s = 0; s < num_splits; ++s) L += exp(ls[s] - M);
    for (int s = 0; s < num_splits; ++s) {
      double w = exp(ls[s] - M) / L;
      const double* op = o_part + (r * num_splits + s) * d;
      for (int c = 0; c < d; ++c) orow[c] += w * op[c];
    }
    lse[r] = M + log(L);
  }
  return 0;
}
