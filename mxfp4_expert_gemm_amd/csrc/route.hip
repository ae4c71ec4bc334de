// Router top-k with certified, exact selection (one wavefront per token).
//
// The router picks the top-k of E experts per token (kimi-k3-mlx digest,
// architecture table: top-16 of 896) and its weights are probabilities renormalised
// over the kept experts (same digest, REAP section).  The selection is defined on
// the correctly rounded fp32 logit of the exact bf16 dot product, plus the bias in
// one fp32 add, ordered by (logit descending, expert index ascending).
//
// The fast logits come with a per-logit error radius r_e = gamma |x_t| |w_e| plus
// rounding padding, so the exact biased logit lies in [c_e - r_e, c_e + r_e].  With
// S the k best by centre, M = min over S of the lower ends and m = max over the rest
// of the upper ends: if M > m the set is certain.  Otherwise an expert whose lower
// end exceeds m is certainly in, one whose upper end is below M certainly out, and
// the ambiguous rest A (lo <= m, hi >= M) is recomputed exactly and ranked.
//
// Exact recompute of one logit: the wave sums the exact fp64 products with a
// rigorous error bound; when both ends of the bound round to the same fp32 that is
// the correctly rounded value.  Otherwise the products are accumulated exactly in a
// fixed-point integer (least significant bit 2^-266, 20 signed 64-bit digits of 32
// bits in LDS, updated with 64-bit LDS atomics, so the order of additions cannot
// matter) and rounded to nearest even once.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int ROUTE_MAXI = 16;  // experts per lane: E <= 1024
constexpr int KDIG = 20;
constexpr int KLSB = 266;

struct WaveScratch {
  unsigned long long acc[KDIG];
  int special;  // bit 0 NaN, bit 1 +inf, bit 2 -inf
};

// ---- ordering: larger value first, NaN last, ties to the lower index
__device__ __forceinline__ bool ranks_before(double va, int ia, double vb, int ib) {
  bool na = va != va, nb = vb != vb;
  if (na != nb) return nb;
  if (!na && va != vb) return va > vb;
  return ia < ib;
}

__device__ __forceinline__ void wave_best(double& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    double ov = __shfl_xor(v, o);
    int oi = __shfl_xor(i, o);
    if (ranks_before(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

__device__ __forceinline__ double wave_min_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmin(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}

// ---- exact dot product of two bf16 rows, correctly rounded to fp32

__device__ void kulisch_add(WaveScratch* ws, uint32_t a, uint32_t b) {
  uint32_t sa = a >> 15, sb = b >> 15;
  uint32_t ea = (a >> 7) & 0xFFu, eb = (b >> 7) & 0xFFu;
  uint32_t fa = a & 0x7Fu, fb = b & 0x7Fu;
  bool a_nan = ea == 255 && fa, b_nan = eb == 255 && fb;
  bool a_inf = ea == 255 && !fa, b_inf = eb == 255 && !fb;
  bool a_zero = ea == 0 && !fa, b_zero = eb == 0 && !fb;
  if (a_nan || b_nan || (a_inf && b_zero) || (b_inf && a_zero)) {
    atomicOr(&ws->special, 1);
    return;
  }
  if (a_inf || b_inf) {
    atomicOr(&ws->special, (sa ^ sb) ? 4 : 2);
    return;
  }
  if (a_zero || b_zero) return;
  uint64_t ma = ea ? 128u + fa : fa, mb = eb ? 128u + fb : fb;
  int qa = ea ? (int)ea - 134 : -133, qb = eb ? (int)eb - 134 : -133;
  int o = qa + qb + KLSB;
  uint64_t v = (ma * mb) << (o & 31);
  uint64_t lo = v & 0xFFFFFFFFull, hi = v >> 32;
  if (sa ^ sb) {
    lo = 0ull - lo;
    hi = 0ull - hi;
  }
  atomicAdd(&ws->acc[o >> 5], lo);
  if (hi) atomicAdd(&ws->acc[(o >> 5) + 1], hi);
}

// digits (signed, lazy carries) -> correctly rounded fp32; run by one lane
__device__ float kulisch_round(const WaveScratch* ws) {
  if ((ws->special & 1) || (ws->special & 6) == 6) return __uint_as_float(0x7FC00000u);
  if (ws->special & 2) return __uint_as_float(0x7F800000u);
  if (ws->special & 4) return __uint_as_float(0xFF800000u);
  uint32_t dig[KDIG];
  long long carry = 0;
  for (int i = 0; i < KDIG; ++i) {
    long long v = (long long)ws->acc[i] + carry;
    dig[i] = (uint32_t)v;
    carry = (v - (long long)dig[i]) >> 32;  // exact: a multiple of 2^32
  }
  bool neg = carry < 0;
  if (neg) {
    uint64_t c = 1;
    for (int i = 0; i < KDIG; ++i) {
      uint64_t v = (uint64_t)(~dig[i]) + c;
      dig[i] = (uint32_t)v;
      c = v >> 32;
    }
  }
  int top = -1;
  for (int i = KDIG - 1; i >= 0 && top < 0; --i)
    if (dig[i]) top = 32 * i + 31 - __clz(dig[i]);
  if (top < 0) return 0.f;
  int lsb = top - 23;
  if (lsb < KLSB - 149) lsb = KLSB - 149;  // fp32 subnormal spacing 2^-149
  auto bit = [&](int i) -> uint32_t { return i < 0 ? 0u : (dig[i >> 5] >> (i & 31)) & 1u; };
  uint32_t mant = 0;
  for (int i = top; i >= lsb; --i) mant = (mant << 1) | bit(i);
  uint32_t rb = bit(lsb - 1);
  bool sticky = false;
  for (int i = lsb - 2; i >= 0 && !sticky; --i) sticky = bit(i);
  if (rb && (sticky || (mant & 1u))) mant += 1;
  float r = ldexpf((float)mant, lsb - KLSB);
  return neg ? -r : r;
}

__device__ float exact_dot_wave(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int d,
                                WaveScratch* ws, int32_t* stats) {
  const int lane = lane_id();
  double s = 0.0, sa = 0.0;
  int nterm = 0;
  for (int c = lane; c < d / 8; c += WAVE) {
    uint4 xv = *reinterpret_cast<const uint4*>(x + 8 * c);
    uint4 wv = *reinterpret_cast<const uint4*>(w + 8 * c);
    uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w}, wsv[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      double p0 = (double)bf16lo(xs[q]) * (double)bf16lo(wsv[q]);
      double p1 = (double)bf16hi(xs[q]) * (double)bf16hi(wsv[q]);
      s += p0;
      s += p1;
      sa += fabs(p0);
      sa += fabs(p1);
    }
    nterm += 8;
  }
  s = wave_sum(s);
  sa = wave_sum(sa);
  int nmax = __shfl(nterm, 0);  // lane 0 has the most terms
  // each lane: nterm additions; tree: 6 more; products are exact in fp64
  double err = (double)(nmax + 8) * 0x1p-53 * sa * (1.0 + 0x1p-40) + 0x1p-1022;
  if (__builtin_isfinite(s) && __builtin_isfinite(sa)) {
    double e2 = err + 0x1p-52 * fabs(s);
    float lo = (float)(s - e2), hi = (float)(s + e2);
    if (lo == hi && __builtin_signbit(lo) == __builtin_signbit(hi)) return lo;  // a zero of unknown sign goes on
  }
  // fixed-point fallback
  if (stats && lane == 0) atomicAdd(&stats[2], 1);
  if (lane < KDIG) ws->acc[lane] = 0ull;
  if (lane == 0) ws->special = 0;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  for (int c = lane; c < d / 8; c += WAVE) {
    uint4 xv = *reinterpret_cast<const uint4*>(x + 8 * c);
    uint4 wv = *reinterpret_cast<const uint4*>(w + 8 * c);
    uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w}, wsv[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      kulisch_add(ws, xs[q] & 0xFFFFu, wsv[q] & 0xFFFFu);
      kulisch_add(ws, xs[q] >> 16, wsv[q] >> 16);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  float r = 0.f;
  if (lane == 0) r = kulisch_round(ws);
  return __shfl(r, 0);
}

// ---- the routing kernel

__global__ void __launch_bounds__(256) route_kernel(RouteArgs a) {
  __shared__ WaveScratch scratch[4];
  const int lane = lane_id();
  const int wave = threadIdx.x / WAVE;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= a.T) return;
  const int E = a.E, k = a.k;
  const int NI = (E + WAVE - 1) / WAVE;
  const bool topk_mode = a.exact_logits != nullptr;
  WaveScratch* ws = &scratch[wave];

  double cen[ROUTE_MAXI], rad[ROUTE_MAXI];
  float val[ROUTE_MAXI];  // the logit used for weights and export
  double xn = topk_mode ? 0.0 : sqrt((double)a.xnorm2[t]);
  const double abs_pad = (double)a.d * 0x1p-125;
#pragma unroll
  for (int i = 0; i < ROUTE_MAXI; ++i) {
    int e = i * WAVE + lane;
    cen[i] = -__builtin_inf();
    rad[i] = 0.0;
    val[i] = -__builtin_inff();
    if (i < NI && e < E) {
      if (topk_mode) {
        float v = a.exact_logits[t * E + e];
        val[i] = v;
        cen[i] = (double)v;  // NaN handled by ranks_before
      } else {
        float lf = a.logits_fast[t * E + e];
        float b = a.bias ? a.bias[t * a.bias_stride + e] : 0.f;
        val[i] = lf + b;  // the fast biased logit, one fp32 rounding
        double beta = a.gamma * xn * sqrt((double)a.wnorm2[e]) * (1.0 + 0x1p-20) + abs_pad;
        double r = beta + 0x1p-21 * ((double)fabsf(lf) + (double)fabsf(b));
        if (__builtin_isfinite(lf) && __builtin_isfinite(b) && __builtin_isfinite(r)) {
          cen[i] = (double)lf + (double)b;
          rad[i] = r;
        } else {
          cen[i] = -__builtin_inf();
          rad[i] = __builtin_inf();
        }
      }
    }
  }

  uint32_t sel = 0;
  if (topk_mode) {
    for (int j = 0; j < k; ++j) {
      double bv = __builtin_nan("");
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < ROUTE_MAXI; ++i) {
        int e = i * WAVE + lane;
        if (i < NI && e < E && !(sel >> i & 1u) && ranks_before(cen[i], e, bv, bi)) {
          bv = cen[i];
          bi = e;
        }
      }
      wave_best(bv, bi);
      if (bi < E && (bi & (WAVE - 1)) == lane) sel |= 1u << (bi / WAVE);
    }
  } else {
    // tentative top-k by centre
    for (int j = 0; j < k; ++j) {
      double bv = __builtin_nan("");
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < ROUTE_MAXI; ++i) {
        int e = i * WAVE + lane;
        if (i < NI && e < E && !(sel >> i & 1u) && ranks_before(cen[i], e, bv, bi)) {
          bv = cen[i];
          bi = e;
        }
      }
      wave_best(bv, bi);
      if (bi < E && (bi & (WAVE - 1)) == lane) sel |= 1u << (bi / WAVE);
    }
    double Mloc = __builtin_inf(), mloc = -__builtin_inf();
#pragma unroll
    for (int i = 0; i < ROUTE_MAXI; ++i) {
      int e = i * WAVE + lane;
      if (i < NI && e < E) {
        double lo = rad[i] == __builtin_inf() ? -__builtin_inf() : cen[i] - rad[i];
        double hi = rad[i] == __builtin_inf() ? __builtin_inf() : cen[i] + rad[i];
        if (sel >> i & 1u) Mloc = fmin(Mloc, lo);
        else mloc = fmax(mloc, hi);
      }
    }
    const double M = wave_min_d(Mloc), m = wave_max_d(mloc);
    const bool all = (a.flags & MOE_ROUTE_EXACT_ALL) != 0;
    if (all || (k < E && !(M > m))) {
      // certainly-in experts keep their place; the ambiguous ones are recomputed
      uint32_t amb = 0, cin = 0;
#pragma unroll
      for (int i = 0; i < ROUTE_MAXI; ++i) {
        int e = i * WAVE + lane;
        if (i < NI && e < E) {
          double lo = rad[i] == __builtin_inf() ? -__builtin_inf() : cen[i] - rad[i];
          double hi = rad[i] == __builtin_inf() ? __builtin_inf() : cen[i] + rad[i];
          if (all) amb |= 1u << i;
          else if ((sel >> i & 1u) && lo > m) cin |= 1u << i;
          else if (lo <= m && hi >= M) amb |= 1u << i;
        }
      }
      int n_in = 0;
#pragma unroll
      for (int i = 0; i < ROUTE_MAXI; ++i) n_in += __popcll(__ballot((cin >> i) & 1u));
      int n_amb = 0;
#pragma unroll
      for (int i = 0; i < ROUTE_MAXI; ++i) {
        unsigned long long bal = __ballot((amb >> i) & 1u);
        n_amb += __popcll(bal);
        while (bal) {
          int l = __ffsll((long long)bal) - 1;
          bal &= bal - 1;
          int e = i * WAVE + l;
          float v = exact_dot_wave(a.x + t * a.d, a.router_w + (int64_t)e * a.d, a.d, ws, a.stats);
          if (a.bias) v = v + a.bias[t * a.bias_stride + e];
          if (lane == l) val[i] = v;
        }
      }
      if (a.stats && lane == 0) {
        atomicAdd(&a.stats[0], 1);
        atomicAdd(&a.stats[1], n_amb);
      }
      // final set: certainly-in plus the best (k - n_in) of the ambiguous by exact value
      sel = cin;
      for (int j = n_in; j < k; ++j) {
        double bv = __builtin_nan("");
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < ROUTE_MAXI; ++i) {
          int e = i * WAVE + lane;
          if ((amb >> i & 1u) && !(sel >> i & 1u) && ranks_before((double)val[i], e, bv, bi)) {
            bv = (double)val[i];
            bi = e;
          }
        }
        wave_best(bv, bi);
        if (bi < E && (bi & (WAVE - 1)) == lane) sel |= 1u << (bi / WAVE);
      }
    }
  }

  // weights over the selected logits (or all when not renormalising)
  float mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < ROUTE_MAXI; ++i) {
    int e = i * WAVE + lane;
    bool use = a.renormalize ? (sel >> i & 1u) : (i < NI && e < E);
    if (use) mx = fmaxf(mx, val[i]);
  }
  mx = wave_max(mx);
  float den = 0.f;
#pragma unroll
  for (int i = 0; i < ROUTE_MAXI; ++i) {
    int e = i * WAVE + lane;
    bool use = a.renormalize ? (sel >> i & 1u) : (i < NI && e < E);
    if (use) den += expf(val[i] - mx);
  }
  den = wave_sum(den);

  // ascending ids, then weights; export logits
  int base = 0;
#pragma unroll
  for (int i = 0; i < ROUTE_MAXI; ++i) {
    unsigned long long bal = __ballot((sel >> i) & 1u);
    if ((sel >> i) & 1u) {
      int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
      a.idx[t * k + pos] = i * WAVE + lane;
      a.w[t * k + pos] = expf(val[i] - mx) / den;
    }
    base += __popcll(bal);
    int e = i * WAVE + lane;
    if (a.logits_out && i < NI && e < E) a.logits_out[t * E + e] = val[i];
  }
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  if (a.E > ROUTE_MAXI * WAVE) return hipErrorInvalidValue;
  hipLaunchKernelGGL(route_kernel, dim3((unsigned)ceil_div(a.T, 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
