/*
 * moe_ref.c: the oracle of one Stable-LatentMoE layer with MXFP4 experts.
 *
 * TEST INFRASTRUCTURE ONLY (see moe_ref.h): plain loops, one thread, every
 * sum in fp64, rounded once at the points the layer defines.  Built with
 * -ffp-contract=off so no multiply-add is fused behind the reader's back.
 */
#include "moe_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ sizes */

/* kimi-k3-in-c post, "experts that are already 4-bit MXFP4": 0.5 B per weight
 * plus 1/32 B of shared scale, times 3 matrices of d_latent * d_ffn weights. */
size_t moe_ref_expert_bytes(int32_t d_latent, int32_t d_ffn) {
  size_t w = (size_t)3 * (size_t)d_latent * (size_t)d_ffn;
  return w / 2 + w / 32;
}

/* ------------------------------------------------------------- MXFP4 value */

/* E2M1 (OCP MX v1.0): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
 * Exponent field 0 is subnormal: 0 or 0.5.  Read off the format definition:
 *   magnitude code 0..7 -> 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
float moe_ref_e2m1(int32_t code) {
  int mag = code & 7;
  int ex = mag >> 1;
  int man = mag & 1;
  float v;
  if (ex == 0)
    v = 0.5f * (float)man;                           /* subnormal: man * 2^-1 */
  else
    v = ldexpf(1.0f + 0.5f * (float)man, ex - 1);    /* (1 + man/2) * 2^(ex-1) */
  return (code & 8) ? -v : v;
}

/* kimi-k3-mlx digest, quantisation tiers (e8m0 scale) and kimi-k3-in-c post,
 * MXFP4 section (one 8-bit exponent per 32 weights): weight = E2M1 * 2^(s-127).
 * e8m0 255 encodes NaN (OCP MX v1.0).  ldexpf is exact here except overflow,
 * which gives +-inf as fp32 rounding would. */
float moe_ref_mxfp4_value(int32_t code, int32_t scale) {
  if (scale == 255) return nanf("");
  return ldexpf(moe_ref_e2m1(code), scale - 127);
}

/* Low-nibble-first (kimi-k3-mlx digest, quantisation tiers): element 2j of a
 * row is the low nibble of byte j, element 2j+1 the high nibble.  The scale of
 * element c of row r is scales[r][c/32].  One row is dequantised at a time, to
 * the weights' exact values: E2M1 * 2^(s-127) in fp64 (at most two significant
 * bits, exponents from -128 to 129, so never rounded; NaN for s = 255).  The
 * expert products use these values; dequantisation to fp32 rounds them once,
 * which changes nothing except the weights of magnitude 2^128 and above (scales
 * 253 and 254 with large codes), which become +-inf as in moe_ref_mxfp4_value. */
static void mx_row(const uint8_t* codes, const uint8_t* scales, int64_t cols, int64_t r, double* out) {
  double lut[16];
  for (int c = 0; c < 16; ++c) lut[c] = (double)moe_ref_e2m1(c);
  const uint8_t* cr = codes + r * (cols / 2);
  const uint8_t* sr = scales + r * (cols / 32);
  for (int64_t b = 0; b < cols / 32; ++b) {
    double sc = sr[b] == 255 ? (double)nanf("") : ldexp(1.0, (int)sr[b] - 127);
    for (int64_t i = 0; i < 32; ++i) {
      int64_t c = b * 32 + i;
      uint8_t byte = cr[c / 2];
      int code = (c & 1) ? (byte >> 4) : (byte & 15);
      out[c] = lut[code] * sc;
    }
  }
}

int moe_ref_dequant_matrix(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                           float* out) {
  if (!codes || !scales || !out || rows < 0 || cols <= 0 || cols % 32) return MOE_REF_ERR_ARG;
  double* row = (double*)malloc(sizeof(double) * (size_t)cols);
  if (!row) return MOE_REF_ERR_ARG;
  for (int64_t r = 0; r < rows; ++r) {
    mx_row(codes, scales, cols, r, row);
    for (int64_t c = 0; c < cols; ++c) out[r * cols + c] = (float)row[c]; /* exact, or +-inf past fp32 */
  }
  free(row);
  return MOE_REF_OK;
}

/* --------------------------------------------------------------- rounding */

/* bf16 keeps 8 significant bits, exponent range of fp32 (normals from 2^-126,
 * subnormal spacing 2^-133).  Round v to that grid, ties to even. */
uint16_t moe_ref_bf16_from_f64(double v) {
  if (isnan(v)) return 0x7FC0;
  if (isinf(v)) return v > 0 ? 0x7F80 : 0xFF80;
  if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
  int e;
  frexp(v, &e);                  /* |v| = m * 2^e, 0.5 <= m < 1 */
  int qexp = e - 8;              /* spacing of 8-bit significands at this binade */
  if (qexp < -133) qexp = -133;  /* bf16 subnormal spacing */
  double q = ldexp(1.0, qexp);
  double r = nearbyint(v / q) * q; /* v/q and the product are exact; nearbyint ties to even */
  if (fabs(r) >= ldexp(1.0, 128)) return r > 0 ? 0x7F80 : 0xFF80;
  float f = (float)r;             /* exact: r has <= 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static inline double bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ------------------------------------------------ exact router dot product */

/*
 * The router logit is defined as the correctly rounded fp32 value of the exact
 * sum of products of bf16 numbers.  A bf16 number is m * 2^q with m an integer
 * below 2^8 (q = be - 134 for a normal biased exponent be, q = -133 for a
 * subnormal).  A product is M * 2^Q with M < 2^16 and Q >= -266.  The sum is
 * accumulated exactly in a fixed-point integer whose least significant bit is
 * 2^-266: KW signed 64-bit "digits" of 32 bits each, carries resolved at the end.
 */
#define KW 20
#define KLSB 266

typedef struct {
  int64_t acc[KW];
  int nan, pinf, ninf;
} kulisch;

static void k_add_product(kulisch* K, uint16_t a, uint16_t b) {
  int sa = a >> 15, sb = b >> 15;
  int ea = (a >> 7) & 0xFF, eb = (b >> 7) & 0xFF;
  int fa = a & 0x7F, fb = b & 0x7F;
  int a_inf = (ea == 255 && fa == 0), b_inf = (eb == 255 && fb == 0);
  int a_nan = (ea == 255 && fa != 0), b_nan = (eb == 255 && fb != 0);
  int a_zero = (ea == 0 && fa == 0), b_zero = (eb == 0 && fb == 0);
  if (a_nan || b_nan || (a_inf && b_zero) || (b_inf && a_zero)) {
    K->nan = 1;
    return;
  }
  if (a_inf || b_inf) {
    if (sa ^ sb) K->ninf = 1; else K->pinf = 1;
    return;
  }
  if (a_zero || b_zero) return;
  int64_t ma = ea ? (128 + fa) : fa, mb = eb ? (128 + fb) : fb;
  int qa = ea ? ea - 134 : -133, qb = eb ? eb - 134 : -133;
  uint64_t M = (uint64_t)(ma * mb);
  int o = qa + qb + KLSB; /* >= 0 */
  int wi = o >> 5, sh = o & 31;
  uint64_t v = M << sh; /* < 2^47 */
  int64_t lo = (int64_t)(v & 0xFFFFFFFFull), hi = (int64_t)(v >> 32);
  if (sa ^ sb) {
    K->acc[wi] -= lo;
    K->acc[wi + 1] -= hi;
  } else {
    K->acc[wi] += lo;
    K->acc[wi + 1] += hi;
  }
}

static int get_bit(const uint32_t* dig, int i) { return (dig[i >> 5] >> (i & 31)) & 1; }

static float k_round(const kulisch* K) {
  if (K->nan || (K->pinf && K->ninf)) return nanf("");
  if (K->pinf) return INFINITY;
  if (K->ninf) return -INFINITY;
  uint32_t dig[KW];
  int64_t carry = 0;
  for (int w = 0; w < KW; ++w) {
    int64_t v = K->acc[w] + carry;
    dig[w] = (uint32_t)v;
    carry = (v - (int64_t)dig[w]) / 4294967296LL; /* exact: numerator is a multiple of 2^32 */
  }
  int neg = carry < 0;
  if (neg) { /* two's complement negate the KW-digit number */
    uint64_t c = 1;
    for (int w = 0; w < KW; ++w) {
      uint64_t v = (uint64_t)(uint32_t)~dig[w] + c;
      dig[w] = (uint32_t)v;
      c = v >> 32;
    }
  }
  int P = -1;
  for (int i = KW * 32 - 1; i >= 0; --i)
    if (get_bit(dig, i)) { P = i; break; }
  if (P < 0) return 0.0f;
  /* fp32: 24 significant bits; least significant bit no lower than 2^-149 */
  int lsb = P - 23;
  if (lsb < KLSB - 149) lsb = KLSB - 149;
  uint32_t mant = 0;
  for (int i = P; i >= lsb; --i) mant = (mant << 1) | (uint32_t)get_bit(dig, i);
  int rbit = get_bit(dig, lsb - 1);
  int sticky = 0;
  for (int i = lsb - 2; i >= 0 && !sticky; --i) sticky = get_bit(dig, i);
  if (rbit && (sticky || (mant & 1))) mant += 1;
  float r = ldexpf((float)mant, lsb - KLSB); /* exact, or overflow to inf */
  return neg ? -r : r;
}

float moe_ref_dot_bf16_exact(const uint16_t* a, const uint16_t* b, int64_t n) {
  kulisch K;
  memset(&K, 0, sizeof K);
  for (int64_t i = 0; i < n; ++i) k_add_product(&K, a[i], b[i]);
  return k_round(&K);
}

/*
 * The same correctly rounded value, found faster when an fp64 sum decides it.
 * Every product of two bf16 numbers is exact in fp64 (at most 16 significant
 * bits, exponents within [-266, 256]).  Summed left to right in fp64, the
 * computed s differs from the exact sum by at most (n-1)u * sum|p_i|, u = 2^-53
 * (the textbook bound for recursive summation); B below is more than twice that,
 * which also covers the rounding of S and of s -+ B.  Rounding to fp32 is
 * monotone, so when s - B and s + B round to the same fp32 bit pattern the exact
 * sum, which lies between them, rounds to it too.  Otherwise (an fp32 rounding
 * boundary within B of s, a sign of zero undecided, or a non-finite input) the
 * fixed-point accumulator above decides.
 */
static float router_dot(const uint16_t* a, const uint16_t* b, int64_t n) {
  double s = 0.0, S = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double p = bf16_to_f64(a[i]) * bf16_to_f64(b[i]);
    s += p;
    S += fabs(p);
  }
  if (isfinite(s) && isfinite(S)) {
    if (S == 0.0) return 0.0f;  /* every product is zero: the exact sum is +0 */
    double B = (double)(n + 4) * ldexp(S, -52);
    float lo = (float)(s - B), hi = (float)(s + B);
    uint32_t ulo, uhi;
    memcpy(&ulo, &lo, 4);
    memcpy(&uhi, &hi, 4);
    if (ulo == uhi) return lo;
  }
  return moe_ref_dot_bf16_exact(a, b, n);
}

/* ----------------------------------------------------------------- router */

/* kimi-k3-mlx digest, architecture table (896 routed experts, router picks 16
 * per token); the router reads the 7168-wide token.  Bias is optional.  Each
 * logit is the correctly rounded fp32 of the exact dot product (router_dot). */
int moe_ref_router_logits(const uint16_t* x, const uint16_t* router_w, const float* bias,
                          int64_t bias_stride, int64_t T, int32_t d, int32_t E, float* logits) {
  if (!x || !router_w || !logits || T < 0 || d <= 0 || E <= 0) return MOE_REF_ERR_ARG;
  for (int64_t t = 0; t < T; ++t)
    for (int32_t e = 0; e < E; ++e) {
      float l = router_dot(x + t * d, router_w + (int64_t)e * d, d);
      if (bias) {
        volatile float s = l + bias[t * bias_stride + e]; /* one fp32 rounding */
        l = s;
      }
      logits[t * E + e] = l;
    }
  return MOE_REF_OK;
}

/* Order for selection: larger logit first; equal logits (+0 and -0 are equal)
 * go to the lower expert index; NaN ranks below every number. */
static int ranks_before(float va, int ia, float vb, int ib) {
  int na = isnan(va), nb = isnan(vb);
  if (na != nb) return nb;          /* the non-NaN one is first */
  if (!na && va != vb) return va > vb;
  return ia < ib;
}

static int cmp_int(const void* a, const void* b) {
  int x = *(const int*)a, y = *(const int*)b;
  return (x > y) - (x < y);
}

/* kimi-k3-mlx digest, REAP section: router weights are probabilities that are
 * renormalised over the surviving experts; here over the k selected ones. */
int moe_ref_select(const float* logits, int64_t T, int32_t E, int32_t k, int32_t renormalize,
                   int32_t* idx, float* w) {
  if (!logits || !idx || T < 0 || E <= 0 || k < 1 || k > E) return MOE_REF_ERR_ARG;
  char* taken = (char*)malloc((size_t)E);
  if (!taken) return MOE_REF_ERR_ARG;
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    int32_t* it = idx + t * k;
    memset(taken, 0, (size_t)E);
    for (int32_t j = 0; j < k; ++j) { /* k passes of "take the first not yet taken" */
      int best = -1;
      for (int32_t e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || ranks_before(l[e], e, l[best], best))) best = e;
      taken[best] = 1;
      it[j] = best;
    }
    qsort(it, (size_t)k, sizeof(int32_t), cmp_int);
    if (w) {
      double m = -INFINITY;
      for (int32_t j = 0; j < k; ++j)
        if (l[it[j]] > m) m = l[it[j]];
      double den = 0.0;
      if (renormalize) {
        for (int32_t j = 0; j < k; ++j) den += exp((double)l[it[j]] - m);
      } else {
        for (int32_t e = 0; e < E; ++e)
          if ((double)l[e] > m) m = l[e];
        for (int32_t e = 0; e < E; ++e) den += exp((double)l[e] - m);
      }
      for (int32_t j = 0; j < k; ++j) w[t * k + j] = (float)(exp((double)l[it[j]] - m) / den);
    }
  }
  free(taken);
  return MOE_REF_OK;
}

/* ------------------------------------------------------------ permutation */

/* Group the T*k (token, slot) rows by expert, tokens ascending inside a group:
 * a counting sort that walks the rows in (t, j) order. */
int moe_ref_permute(const int32_t* idx, int64_t T, int32_t k, int32_t E, int32_t* counts,
                    int32_t* offsets, int32_t* perm) {
  if (!idx || !counts || !offsets || !perm || T < 0 || k < 1 || E < 1) return MOE_REF_ERR_ARG;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t r = 0; r < T * k; ++r) {
    if (idx[r] < 0 || idx[r] >= E) return MOE_REF_ERR_ARG;
    counts[idx[r]] += 1;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* cur = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  if (!cur) return MOE_REF_ERR_ARG;
  for (int32_t e = 0; e < E; ++e) cur[e] = offsets[e];
  for (int64_t r = 0; r < T * k; ++r) perm[cur[idx[r]]++] = (int32_t)r;
  free(cur);
  return MOE_REF_OK;
}

/* ------------------------------------------------------------ dense parts */

/* kimi-k3-mlx digest, architecture: the latent projections 7168 -> 3584 and
 * back are bf16 matrices; sum in fp64, round once to bf16. */
int moe_ref_linear_bf16(const uint16_t* in, const uint16_t* W, int64_t T, int32_t n_in, int32_t n_out,
                        uint16_t* out) {
  if (!in || !W || !out || T < 0 || n_in <= 0 || n_out <= 0) return MOE_REF_ERR_ARG;
  for (int64_t t = 0; t < T; ++t)
    for (int32_t o = 0; o < n_out; ++o) {
      double s = 0.0;
      for (int32_t i = 0; i < n_in; ++i)
        s += bf16_to_f64(in[t * n_in + i]) * bf16_to_f64(W[(int64_t)o * n_in + i]);
      out[t * n_out + o] = moe_ref_bf16_from_f64(s);
    }
  return MOE_REF_OK;
}

/* ---------------------------------------------------------------- experts */

double moe_ref_silu(double g) { return g / (1.0 + exp(-g)); }

/* One routed expert, GLU form implied by 3 matrices of 3584 x 3072 per expert
 * (kimi-k3-in-c post, MXFP4 section: 33,030,144 = 3 * 3584 * 3072), with the
 * activation in fp32 or better (kimi-k3-mlx digest, SiTU-GLU bullet):
 *   g = RN32(W_g h), u = RN32(W_u h), a = bf16(act(g) * u), y = RN32(W_dn a). */
/* ------------------------------------------------- MXFP8 activations (OCP MX) */

/* E4M3 (OCP FP8, bias 7, no infinities): sign bit 7, exponent bits 6..3, mantissa
 * bits 2..0; exponent field 0 holds the subnormals m * 2^-9; S.1111.111 is NaN, so
 * the largest finite magnitude is 1.75 * 2^8 = 448. */
double moe_ref_e4m3_value(int32_t code) {
  const int sign = (code >> 7) & 1, ef = (code >> 3) & 15, m = code & 7;
  double v;
  if (ef == 15 && m == 7) return NAN;
  if (ef == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, ef - 7);
  return sign ? -v : v;
}

/* the e4m3 code of |q| rounded to nearest, ties to the even mantissa, saturated to 448 */
static int32_t e4m3_code_of(double q) {
  const int sign = signbit(q) ? 0x80 : 0;
  double a = fabs(q);
  if (a >= 448.0) return sign | 0x7E;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);                 /* a = f 2^e, f in [0.5, 1): the binade is 2^(e-1) */
  int b = e - 1;
  if (b < -6) b = -6;           /* the subnormal range shares the spacing of 2^-6 */
  const double step = ldexp(1.0, b - 3);
  const double r = nearbyint(a / step) * step;  /* default rounding: ties to even */
  if (r == 0.0) return sign;
  if (r < ldexp(1.0, -6)) return sign | (int32_t)(r / ldexp(1.0, -9));  /* subnormal */
  frexp(r, &e);
  const int rb = e - 1;         /* r may have moved up to the next binade */
  const int m = (int)((r / ldexp(1.0, rb) - 1.0) * 8.0);
  return sign | ((rb + 7) << 3) | m;
}

/* One block of 32 values as MXFP8 (OCP Microscaling v1.0 convention, E4M3 elements):
 * shared exponent X = floor(log2(max |v|)) - 8 (8 = E4M3's largest normal exponent),
 * the maximum taken over the finite values and X limited to the e8m0 range [-127, 127];
 * element codes = v / 2^X rounded to nearest even E4M3, saturated to +-448; scale byte
 * X + 127.  A block of zeros gets scale byte 0 and zero codes (signs kept).  E4M3 has no
 * infinity: NaN and +-inf elements get the NaN code 0x7F (the convention as read here). */
int moe_ref_mxfp8_block(const double* v, uint8_t* codes, uint8_t* scale) {
  if (!v || !codes || !scale) return MOE_REF_ERR_ARG;
  double amax = 0.0;
  for (int i = 0; i < 32; ++i)
    if (isfinite(v[i]) && fabs(v[i]) > amax) amax = fabs(v[i]);
  int X = -127;
  if (amax > 0.0) {
    int e;
    frexp(amax, &e);
    X = (e - 1) - 8;
    if (X < -127) X = -127;
    if (X > 127) X = 127;
  }
  for (int i = 0; i < 32; ++i)
    codes[i] = isfinite(v[i]) ? (uint8_t)e4m3_code_of(ldexp(v[i], -X)) : (uint8_t)0x7F;
  *scale = (uint8_t)(X + 127);
  return MOE_REF_OK;
}

/* the values a row of n (multiple of 32) takes after MXFP8 quantisation */
static void mxfp8_row(const double* v, int64_t n, double* out) {
  uint8_t codes[32], sc;
  for (int64_t b = 0; b < n; b += 32) {
    moe_ref_mxfp8_block(v + b, codes, &sc);
    for (int i = 0; i < 32; ++i) out[b + i] = ldexp(moe_ref_e4m3_value(codes[i]), (int)sc - 127);
  }
}

int moe_ref_expert_fmt(const uint16_t* h, const uint8_t* record, int32_t L, int32_t F, int32_t act,
                       int32_t act_format, uint16_t* a_out, float* y) {
  if (!h || !record || !y || L <= 0 || F <= 0 || L % 32 || F % 32) return MOE_REF_ERR_ARG;
  if (act_format != MOE_REF_ACT_BF16 && act_format != MOE_REF_ACT_MXFP8) return MOE_REF_ERR_ARG;
  if (act != MOE_REF_ACT_SILU) return MOE_REF_ERR_UNSUPPORTED;
  const int64_t ncode = (int64_t)F * L / 2, mat = ncode + (int64_t)F * L / 32;
  const uint8_t* gate = record;
  const uint8_t* up = record + mat;
  const uint8_t* down = record + 2 * mat;
  const int32_t wmax = L > F ? L : F;
  uint16_t* a = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)F);
  double* wg = (double*)malloc(sizeof(double) * (size_t)wmax);
  double* wu = (double*)malloc(sizeof(double) * (size_t)wmax);
  double* hv = (double*)malloc(sizeof(double) * (size_t)wmax);  /* the GEMM inputs as used */
  double* tmp = (double*)malloc(sizeof(double) * (size_t)wmax);
  if (!a || !wg || !wu || !hv || !tmp) { free(a); free(wg); free(wu); free(hv); free(tmp); return MOE_REF_ERR_ARG; }
  /* h as the gate/up input: the bf16 values, or their MXFP8 quantisation */
  for (int32_t l = 0; l < L; ++l) tmp[l] = bf16_to_f64(h[l]);
  if (act_format == MOE_REF_ACT_MXFP8)
    mxfp8_row(tmp, L, hv);
  else
    memcpy(hv, tmp, sizeof(double) * (size_t)L);
  for (int32_t f = 0; f < F; ++f) {
    mx_row(gate, gate + ncode, L, f, wg);
    mx_row(up, up + ncode, L, f, wu);
    double sg = 0.0, su = 0.0;
    for (int32_t l = 0; l < L; ++l) {
      sg += hv[l] * wg[l];
      su += hv[l] * wu[l];
    }
    float g = (float)sg, u = (float)su;
    a[f] = moe_ref_bf16_from_f64(moe_ref_silu((double)g) * (double)u);
  }
  /* a as the down input, likewise */
  for (int32_t f = 0; f < F; ++f) tmp[f] = bf16_to_f64(a[f]);
  if (act_format == MOE_REF_ACT_MXFP8)
    mxfp8_row(tmp, F, hv);
  else
    memcpy(hv, tmp, sizeof(double) * (size_t)F);
  for (int32_t l = 0; l < L; ++l) {
    mx_row(down, down + ncode, F, l, wg);
    double s = 0.0;
    for (int32_t f = 0; f < F; ++f) s += hv[f] * wg[f];
    y[l] = (float)s;
  }
  if (a_out) memcpy(a_out, a, sizeof(uint16_t) * (size_t)F);
  free(a); free(wg); free(wu); free(hv); free(tmp);
  return MOE_REF_OK;
}

int moe_ref_expert(const uint16_t* h, const uint8_t* record, int32_t L, int32_t F, int32_t act,
                   uint16_t* a_out, float* y) {
  return moe_ref_expert_fmt(h, record, L, F, act, MOE_REF_ACT_BF16, a_out, y);
}

/* weighted combine of the k expert outputs of each token, in latent space */
int moe_ref_combine(const float* y, const float* w, int64_t T, int32_t k, int32_t L, uint16_t* z) {
  if (!y || !w || !z || T < 0 || k < 1 || L <= 0) return MOE_REF_ERR_ARG;
  for (int64_t t = 0; t < T; ++t)
    for (int32_t l = 0; l < L; ++l) {
      double s = 0.0;
      for (int32_t j = 0; j < k; ++j) s += (double)w[t * k + j] * (double)y[(t * k + j) * L + l];
      z[t * L + l] = moe_ref_bf16_from_f64(s);
    }
  return MOE_REF_OK;
}

/* ------------------------------------------------------------- REAP saliency */

/* The REAP score's sum (kimi-k3-mlx digest, REAP section): for each token t and slot j,
 * the router weight w[t][j] times the 2-norm of that expert's output y[t*k+j] is added
 * to s[idx[t][j]], in token order; squares and sums in fp64. */
int moe_ref_reap_saliency(const float* y, const float* w, const int32_t* idx, int64_t T, int32_t k, int32_t L,
                          int32_t E, double* s) {
  if (!y || !w || !idx || !s || T < 0 || k < 1 || L <= 0 || E < 1) return MOE_REF_ERR_ARG;
  for (int64_t t = 0; t < T; ++t)
    for (int32_t j = 0; j < k; ++j) {
      const int32_t e = idx[t * k + j];
      if (e < 0 || e >= E) return MOE_REF_ERR_ARG;
      const float* row = y + (t * k + j) * (int64_t)L;
      double sq = 0.0;
      for (int32_t l = 0; l < L; ++l) sq += (double)row[l] * (double)row[l];
      s[e] += (double)w[t * k + j] * sqrt(sq);
    }
  return MOE_REF_OK;
}

/* ------------------------------------------------------------ whole layer */

/* The layer with num_shared always-on shared experts (kimi-k3-mlx digest, architecture
 * table and LatentMoE bullet: two per token, and they work at the full width, not in
 * the latent).  Reading: each is a SiLU-GLU expert on the token x itself, an MXFP4 record
 * of the routed format with (L, F) = (d, F_s), weight 1; its fp32 output joins the
 * latent-up product before the one bf16 rounding of out. */
int moe_ref_layer_forward_shared(int32_t d, int32_t L, int32_t F, int32_t E, int32_t k, int32_t act,
                                 int32_t act_format, int32_t renormalize, const uint16_t* x, const uint16_t* router_w,
                          const float* bias, int64_t bias_stride, const uint16_t* latent_down,
                          const uint16_t* latent_up, const uint8_t* blob, const int32_t* tokens,
                          int64_t n_tokens, uint16_t* out, int32_t* idx, float* w, float* logits,
                          uint16_t* h_out, uint16_t* z_out, const uint8_t* shared_blob, int32_t num_shared,
                          int32_t F_s) {
  if (!x || !router_w || !latent_down || !latent_up || !blob || !out || d <= 0 || L <= 0 ||
      F <= 0 || E <= 0 || k < 1 || k > E || n_tokens < 0 || L % 32 || F % 32)
    return MOE_REF_ERR_ARG;
  if (act != MOE_REF_ACT_SILU) return MOE_REF_ERR_UNSUPPORTED;
  const size_t rec = moe_ref_expert_bytes(L, F);
  float* lg = (float*)malloc(sizeof(float) * (size_t)E);
  int32_t* id = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  float* wt = (float*)malloc(sizeof(float) * (size_t)k);
  uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)L);
  float* y = (float*)malloc(sizeof(float) * (size_t)k * (size_t)L);
  uint16_t* z = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)L);
  float* ys = num_shared > 0 ? (float*)malloc(sizeof(float) * (size_t)num_shared * (size_t)d) : NULL;
  int rc = MOE_REF_OK;
  if (!lg || !id || !wt || !h || !y || !z || (num_shared > 0 && (!ys || !shared_blob || F_s <= 0 || F_s % 32)))
    rc = MOE_REF_ERR_ARG;
  for (int64_t i = 0; i < n_tokens && rc == MOE_REF_OK; ++i) {
    int64_t t = tokens ? tokens[i] : i;
    const uint16_t* xt = x + t * d;
    const float* bt = bias ? bias + t * bias_stride : NULL;
    moe_ref_router_logits(xt, router_w, bt, 0, 1, d, E, lg);
    moe_ref_select(lg, 1, E, k, renormalize, id, wt);
    moe_ref_linear_bf16(xt, latent_down, 1, d, L, h);
    for (int32_t j = 0; j < k && rc == MOE_REF_OK; ++j)
      rc = moe_ref_expert_fmt(h, blob + (size_t)id[j] * rec, L, F, act, act_format, NULL, y + (size_t)j * L);
    moe_ref_combine(y, wt, 1, k, L, z);
    if (num_shared == 0) {
      moe_ref_linear_bf16(z, latent_up, 1, L, d, out + i * d);
    } else {
      const size_t srec = moe_ref_expert_bytes(d, F_s);
      for (int32_t sx = 0; sx < num_shared && rc == MOE_REF_OK; ++sx)
        rc = moe_ref_expert_fmt(xt, shared_blob + (size_t)sx * srec, d, F_s, act, act_format, NULL,
                                ys + (size_t)sx * d);
      for (int32_t m = 0; m < d; ++m) {
        double acc = 0.0;
        for (int32_t l = 0; l < L; ++l) acc += bf16_to_f64(z[l]) * bf16_to_f64(latent_up[(int64_t)m * L + l]);
        for (int32_t sx = 0; sx < num_shared; ++sx) acc += (double)ys[(size_t)sx * d + m];
        out[i * d + m] = moe_ref_bf16_from_f64(acc);
      }
    }
    if (idx) memcpy(idx + i * k, id, sizeof(int32_t) * (size_t)k);
    if (w) memcpy(w + i * k, wt, sizeof(float) * (size_t)k);
    if (logits) memcpy(logits + i * E, lg, sizeof(float) * (size_t)E);
    if (h_out) memcpy(h_out + i * L, h, sizeof(uint16_t) * (size_t)L);
    if (z_out) memcpy(z_out + i * L, z, sizeof(uint16_t) * (size_t)L);
  }
  free(lg); free(id); free(wt); free(h); free(y); free(z); free(ys);
  return rc;
}

int moe_ref_layer_forward_fmt(int32_t d, int32_t L, int32_t F, int32_t E, int32_t k, int32_t act,
                              int32_t act_format, int32_t renormalize, const uint16_t* x, const uint16_t* router_w,
                              const float* bias, int64_t bias_stride, const uint16_t* latent_down,
                              const uint16_t* latent_up, const uint8_t* blob, const int32_t* tokens,
                              int64_t n_tokens, uint16_t* out, int32_t* idx, float* w, float* logits,
                              uint16_t* h_out, uint16_t* z_out) {
  return moe_ref_layer_forward_shared(d, L, F, E, k, act, act_format, renormalize, x, router_w, bias, bias_stride,
                                      latent_down, latent_up, blob, tokens, n_tokens, out, idx, w, logits, h_out,
                                      z_out, NULL, 0, 0);
}

int moe_ref_layer_forward(int32_t d, int32_t L, int32_t F, int32_t E, int32_t k, int32_t act,
                          int32_t renormalize, const uint16_t* x, const uint16_t* router_w,
                          const float* bias, int64_t bias_stride, const uint16_t* latent_down,
                          const uint16_t* latent_up, const uint8_t* blob, const int32_t* tokens,
                          int64_t n_tokens, uint16_t* out, int32_t* idx, float* w, float* logits,
                          uint16_t* h_out, uint16_t* z_out) {
  return moe_ref_layer_forward_fmt(d, L, F, E, k, act, MOE_REF_ACT_BF16, renormalize, x, router_w, bias,
                                   bias_stride, latent_down, latent_up, blob, tokens, n_tokens, out, idx, w,
                                   logits, h_out, z_out);
}
