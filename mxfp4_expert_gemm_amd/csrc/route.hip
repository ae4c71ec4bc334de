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

__device__ __forceinline__ void kulisch_add(WaveScratch* ws, uint32_t a, uint32_t b) {
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
__device__ __forceinline__ float kulisch_round(const WaveScratch* ws) {
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

__device__ __forceinline__ float exact_dot_wave(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int d,
                                WaveScratch* ws, int32_t* stats) {
  const int lane = lane_id();
  double s = 0.0, sa = 0.0;
  int nterm = 0;
  // EXU chunks of 8 products per lane are loaded before any is used, so the row costs
  // d / (8 WAVE EXU) memory round trips (two at d = 7168) rather than one per chunk
  constexpr int EXU = 7;
  const int nch = d / 8;
  for (int c0 = lane; c0 < nch; c0 += WAVE * EXU) {
    uint4 xv[EXU], wv[EXU];
#pragma unroll
    for (int u = 0; u < EXU; ++u) {
      const int c = c0 + WAVE * u;
      if (c < nch) {
        xv[u] = *reinterpret_cast<const uint4*>(x + 8 * c);
        wv[u] = *reinterpret_cast<const uint4*>(w + 8 * c);
      } else {
        xv[u] = wv[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < EXU; ++u) {
      if (c0 + WAVE * u >= nch) continue;
      uint32_t xs[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w}, wsv[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
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

// ---- selection by keys

// neighbouring floats (finite inputs; the infinities stay put)
__device__ __forceinline__ float next_down(float f) {
  if (f != f || f == -__builtin_inff()) return f;
  if (f == 0.f) return -__uint_as_float(1u);
  uint32_t u = __float_as_uint(f);
  return __uint_as_float(f > 0.f ? u - 1u : u + 1u);
}
__device__ __forceinline__ float next_up(float f) { return -next_down(-f); }

// order-preserving 32-bit key of a float: larger value -> larger key; -0 == +0;
// NaN maps to 1, below every number (every number's key is >= 0x007FFFFF); 0 is
// reserved for "not a candidate".
__device__ __forceinline__ uint32_t order_key(float v) {
  if (v != v) return 1u;
  uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Marks in `sel` the kk largest keys of the wave (ties to the lower expert index,
// e = 64 i + lane).  Keys of 0 are never taken when at least kk keys are nonzero.
// Radix select on the key bits with ballot counts: no cross-lane data movement.
__device__ __forceinline__ uint32_t select_top(const uint32_t (&key)[ROUTE_MAXI], int kk) {
  uint32_t tau = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < ROUTE_MAXI; ++i) cnt += __popcll(__ballot(key[i] >= cand));
    if (cnt >= kk) tau = cand;
  }
  uint32_t sel = 0;
  int need = kk;
#pragma unroll
  for (int i = 0; i < ROUTE_MAXI; ++i) {
    const bool gt = key[i] > tau;
    need -= __popcll(__ballot(gt));
    if (gt) sel |= 1u << i;
  }
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < ROUTE_MAXI; ++i) {
    unsigned long long m = __ballot(key[i] == tau && tau != 0u);
    unsigned long long take = 0;
    while (need > 0 && m) {
      unsigned long long low = m & (0ull - m);
      take |= low;
      m ^= low;
      --need;
    }
    if ((take >> lane) & 1ull) sel |= 1u << i;
  }
  return sel;
}

// ---- routing of one token by one wave


// Per-wave LDS of the routing: Kulisch digits, the candidate list of the fast path and
// the selected (expert, logit) pairs in output order.
constexpr int ROUTE_CAND = WAVE;
struct RouteLds {
  WaveScratch ks;
  uint32_t ckey[ROUTE_CAND];
  int cidx[ROUTE_CAND];
  float cval[ROUTE_CAND], crad[ROUTE_CAND];
  alignas(16) int oidx[WAVE];
  float oval[WAVE];
};

// Writes idx/w of token t from the k selected (expert, logit) pairs in L->oidx/oval,
// ascending expert order.  Renormalised weights: softmax over the k logits (max and a
// fixed DPP tree, the same in every path).  Otherwise: over all E logits, whose
// max and sum over experts the caller passes in.
__device__ __forceinline__ void emit_topk(const RouteArgs& a, int64_t t, const RouteLds* L, float mx_all,
                                          float den_all) {
  const int lane = lane_id(), k = a.k;
  const bool mine = lane < k;
  const float v = mine ? L->oval[lane] : -__builtin_inff();
  float mx = mx_all, den = den_all;
  float ex;
  if (a.renormalize) {
    mx = wave_max_dpp(v);
    ex = mine ? expf(v - mx) : 0.f;
    den = wave_sum_dpp(ex);
  } else {
    ex = expf(v - mx);
  }
  if (mine) {
    a.idx[t * k + lane] = L->oidx[lane];
    a.w[t * k + lane] = ex / den;
  }
}

// max and sum of exp(v - max) over all experts of the lane arrays (softmax over E)
__device__ __forceinline__ void softmax_all(const float (&val)[ROUTE_MAXI], int E, float& mx, float& den) {
  const int lane = lane_id();
  mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < ROUTE_MAXI; ++i)
    if (i * WAVE + lane < E) mx = fmaxf(mx, val[i]);
  mx = wave_max_dpp(mx);
  den = 0.f;
#pragma unroll
  for (int i = 0; i < ROUTE_MAXI; ++i)
    if (i * WAVE + lane < E) den += expf(val[i] - mx);
  den = wave_sum_dpp(den);
}

// General path: selection over every expert by radix select on the keys, certification,
// exact recompute of the ambiguous logits.  Kept out of line: it runs only when the
// fast path below cannot decide (many ties, an uncertain boundary, MOE_ROUTE_EXACT_ALL).
__device__ __forceinline__ void route_token_general(const RouteArgs& a, int64_t t, RouteLds* L) {
  const int lane = lane_id();
  const int E = a.E, k = a.k;
  const bool topk_mode = a.exact_logits != nullptr;
  float val[ROUTE_MAXI];      // logit used for weights and export (exact where recomputed)
  float lo[ROUTE_MAXI], hi[ROUTE_MAXI];
  uint32_t key[ROUTE_MAXI];
  const double xn = topk_mode ? 0.0 : (double)a.xnorm[t];
  const double abs_pad = (double)a.d * 0x1p-125;
#pragma unroll
  for (int i = 0; i < ROUTE_MAXI; ++i) {
    const int e = i * WAVE + lane;
    val[i] = -__builtin_inff();
    lo[i] = -__builtin_inff();
    hi[i] = -__builtin_inff();
    key[i] = 0u;
    if (e < E) {
      if (topk_mode) {
        val[i] = a.exact_logits[t * E + e];
        key[i] = order_key(val[i]);
      } else {
        const float lf = a.logits_fast[t * E + e];
        const float b = a.bias ? a.bias[t * a.bias_stride + e] : 0.f;
        val[i] = lf + b;  // the fast biased logit, one fp32 rounding
        const double r = a.gamma * xn * (double)a.wnorm[e] * (1.0 + 0x1p-20) + abs_pad +
                         0x1p-21 * ((double)fabsf(lf) + (double)fabsf(b));
        const double c = (double)lf + (double)b;
        if (b == -__builtin_inff() && __builtin_isfinite(lf) && __builtin_isfinite(r) &&
            fabs((double)lf) + r < 0x1.fffffep127) {
          // a bias of -inf (an expert pruned away): the exact logit is finite, so the
          // biased logit is exactly -inf and never needs recomputing
          val[i] = lo[i] = hi[i] = -__builtin_inff();
          key[i] = order_key(-__builtin_inff());
        } else if (__builtin_isfinite(lf) && __builtin_isfinite(b) && __builtin_isfinite(r)) {
          // outward-rounded fp32 ends of the interval holding the exact biased logit
          float l32 = (float)(c - r), h32 = (float)(c + r);
          if ((double)l32 > c - r) l32 = next_down(l32);
          if ((double)h32 < c + r) h32 = next_up(h32);
          lo[i] = l32;
          hi[i] = h32;
          key[i] = order_key((float)c);
        } else {  // unknown: must be recomputed if it can matter
          lo[i] = -__builtin_inff();
          hi[i] = __builtin_inff();
          key[i] = order_key(-__builtin_inff());
        }
      }
    }
  }

  uint32_t sel = select_top(key, k);
  if (!topk_mode) {
    float mloc = -__builtin_inff(), Mloc = __builtin_inff();
#pragma unroll
    for (int i = 0; i < ROUTE_MAXI; ++i) {
      const int e = i * WAVE + lane;
      if (e < E) {
        if ((sel >> i) & 1u) Mloc = fminf(Mloc, lo[i]);
        else mloc = fmaxf(mloc, hi[i]);
      }
    }
    const float M = wave_min_dpp(Mloc), m = wave_max_dpp(mloc);
    const bool all = (a.flags & MOE_ROUTE_EXACT_ALL) != 0;
    if (all || (k < E && !(M > m))) {
      // amb: undecided experts, ranked below on exact values; known: those among them
      // whose interval is a point (a pruned expert's exact -inf), already in val
      uint32_t amb = 0, cin = 0, known = 0;
#pragma unroll
      for (int i = 0; i < ROUTE_MAXI; ++i) {
        const int e = i * WAVE + lane;
        if (e < E) {
          if (all) amb |= 1u << i;
          else if (((sel >> i) & 1u) && lo[i] > m) cin |= 1u << i;
          else if (lo[i] <= m && hi[i] >= M) {
            amb |= 1u << i;
            if (lo[i] == hi[i]) known |= 1u << i;
          }
        }
      }
      int n_in = 0, n_amb = 0;
#pragma unroll
      for (int i = 0; i < ROUTE_MAXI; ++i) {
        n_in += __popcll(__ballot((cin >> i) & 1u));
        unsigned long long bal = __ballot(((amb & ~known) >> i) & 1u);
        n_amb += __popcll(bal);
        while (bal) {
          const int l = __ffsll((long long)bal) - 1;
          bal &= bal - 1;
          const int e = i * WAVE + l;
          float v = exact_dot_wave(a.x + t * a.d, a.router_w + (int64_t)e * a.d, a.d, &L->ks, a.stats);
          if (a.bias) v = v + a.bias[t * a.bias_stride + e];
          if (lane == l) val[i] = v;
        }
      }
      if (a.stats && lane == 0) {
        atomicAdd(&a.stats[0], 1);
        atomicAdd(&a.stats[1], n_amb);
      }
      uint32_t ekey[ROUTE_MAXI];
#pragma unroll
      for (int i = 0; i < ROUTE_MAXI; ++i) ekey[i] = ((amb >> i) & 1u) ? order_key(val[i]) : 0u;
      sel = cin | select_top(ekey, k - n_in);
    }
  }

  // selected pairs in ascending expert order, then the weights
  int base = 0;
#pragma unroll
  for (int i = 0; i < ROUTE_MAXI; ++i) {
    const unsigned long long bal = __ballot((sel >> i) & 1u);
    if ((sel >> i) & 1u) {
      const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
      L->oidx[pos] = i * WAVE + lane;
      L->oval[pos] = val[i];
    }
    base += __popcll(bal);
    const int e = i * WAVE + lane;
    if (a.logits_out && e < E) a.logits_out[t * E + e] = val[i];
  }
  float mx_all = 0.f, den_all = 1.f;
  if (!a.renormalize) softmax_all(val, E, mx_all, den_all);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  emit_topk(a, t, L, mx_all, den_all);
}

// k-th largest of one key per lane (radix select with ballots), k <= WAVE
__device__ __forceinline__ uint32_t kth_of_lanes(uint32_t v, int k) {
  uint32_t tau = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    if (__popcll(__ballot(v >= cand)) >= k) tau = cand;
  }
  return tau;
}

// Routing of token t (fills idx/w, ascending ids, and optionally logits_out).
//
// Fast path.  The keys of the fast biased logits c_e are cut at tau, the k-th largest
// of the 64 per-lane maxima: at least k keys reach tau, so the k best are among the
// candidates (key >= tau), usually a few dozen.  The candidates are ranked against
// each other, one per lane, and the selection is certified as in the general path
// with fp32 interval ends: radius R_e = gamma' |x||w_e| + pad' + 2^-20 (|lf| + |b|),
// with gamma' = gamma (1 + 2^-18) and pad' = d 2^-124, covers the radius of the
// general path plus the roundings of c_e = lf + b and of R_e itself (a few ulp of
// 2^-24 each), and the ends c - R and c + R are pushed one ulp outwards.  More than 64
// candidates or an uncertified boundary go to the general path, which starts over.
__device__ __forceinline__ void route_token(const RouteArgs& a, int64_t t, RouteLds* L) {
  const int lane = lane_id();
  const int E = a.E, k = a.k;
  const bool topk_mode = a.exact_logits != nullptr;
  if (a.flags & MOE_ROUTE_EXACT_ALL) {
    route_token_general(a, t, L);
    return;
  }
  float c[ROUTE_MAXI], R[ROUTE_MAXI];
  uint32_t key[ROUTE_MAXI];
  const float xn = topk_mode ? 0.f : a.xnorm[t];
  const float gam = (float)a.gamma * (1.f + 0x1p-18f) * xn;
  const float pad = (float)a.d * 0x1p-124f;
  // every load unconditional and from a pointer chosen once (lanes past E read the last
  // expert and are masked after; a missing operand reads the logits and is not used), so
  // no branch splits them and all are in flight together: one memory round trip
  const float* pl = (topk_mode ? a.exact_logits : a.logits_fast) + t * E;
  const bool has_bias = !topk_mode && a.bias != nullptr;
  const float* pb = has_bias ? a.bias + t * a.bias_stride : pl;
  const float* pw = topk_mode ? pl : a.wnorm;
  float lf[ROUTE_MAXI], bv[ROUTE_MAXI], wn[ROUTE_MAXI];
#pragma unroll
  for (int i = 0; i < ROUTE_MAXI; ++i) {
    const int e = i * WAVE + lane < E ? i * WAVE + lane : E - 1;
    lf[i] = pl[e];
    bv[i] = pb[e];
    wn[i] = pw[e];
  }
#pragma unroll
  for (int i = 0; i < ROUTE_MAXI; ++i) bv[i] = has_bias ? bv[i] : 0.f;
  uint32_t kmax = 0;
#pragma unroll
  for (int i = 0; i < ROUTE_MAXI; ++i) {
    const int e = i * WAVE + lane;
    c[i] = -__builtin_inff();
    R[i] = 0.f;
    key[i] = 0u;
    if (e < E) {
      if (topk_mode) {
        c[i] = lf[i];
      } else {
        c[i] = lf[i] + bv[i];
        R[i] = gam * wn[i] + pad + 0x1p-20f * (fabsf(lf[i]) + fabsf(bv[i]));
        if (bv[i] == -__builtin_inff()) {
          // pruned expert (bias -inf): exactly -inf when the exact logit is finite, which
          // the radius shows; else unknown
          const float rr = gam * wn[i] + pad + 0x1p-20f * fabsf(lf[i]);
          const bool known = __builtin_isfinite(lf[i]) && __builtin_isfinite(rr) && fabsf(lf[i]) + rr < 0x1p127f;
          c[i] = -__builtin_inff();
          R[i] = known ? 0.f : __builtin_inff();
        } else if (!(__builtin_isfinite(c[i]) && __builtin_isfinite(R[i]))) {
          c[i] = -__builtin_inff();  // unknown: the general path recomputes it if it can matter
          R[i] = __builtin_inff();
        }
      }
      key[i] = order_key(c[i]);
      kmax = key[i] > kmax ? key[i] : kmax;
    }
  }
  const uint32_t tau = kth_of_lanes(kmax, k);
  // candidates: keys >= tau, compacted in (lane, i) order
  int mine = 0;
#pragma unroll
  for (int i = 0; i < ROUTE_MAXI; ++i) mine += (key[i] != 0u && key[i] >= tau);
  int n_c = 0;
  int pos = wave_excl_scan(mine, n_c);
  if (n_c > ROUTE_CAND) {
    route_token_general(a, t, L);
    return;
  }
#pragma unroll
  for (int i = 0; i < ROUTE_MAXI; ++i)
    if (key[i] != 0u && key[i] >= tau) {
      L->ckey[pos] = key[i];
      L->cidx[pos] = i * WAVE + lane;
      L->cval[pos] = c[i];
      L->crad[pos] = R[i];
      ++pos;
    }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // rank of this lane's candidate: (key descending, expert ascending)
  const bool live = lane < n_c;
  const uint32_t mk = live ? L->ckey[lane] : 0u;
  const int me = live ? L->cidx[lane] : 0x7FFFFFFF;
  int rank = 0;
  for (int j = 0; j < n_c; ++j) {  // register broadcasts: no memory round trip per step
    const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)mk, j);
    const int ej = __builtin_amdgcn_readlane(me, j);
    rank += (kj > mk) || (kj == mk && ej < me);
  }
  const bool sel = live && rank < k;
  const float mc = live ? L->cval[lane] : 0.f, mr = live ? L->crad[lane] : 0.f;
  if (!topk_mode && k < E) {
    // certification: min lower end over the selected, max upper end over the rest
    float Mloc = __builtin_inff(), mloc = -__builtin_inff();
    if (sel) Mloc = mr == __builtin_inff() ? -__builtin_inff() : next_down(mc - mr);
    if (live && !sel) mloc = mr == __builtin_inff() ? __builtin_inff() : next_up(mc + mr);
#pragma unroll
    for (int i = 0; i < ROUTE_MAXI; ++i)
      if (key[i] != 0u && key[i] < tau) mloc = fmaxf(mloc, R[i] == __builtin_inff() ? __builtin_inff() : next_up(c[i] + R[i]));
    const float M = wave_min_dpp(Mloc), m = wave_max_dpp(mloc);
    if (!(M > m)) {
      route_token_general(a, t, L);
      return;
    }
  }
  // output order: ascending expert id among the selected
  int op = 0;
  for (unsigned long long sm = __ballot(sel); sm; sm &= sm - 1)
    op += __builtin_amdgcn_readlane(me, __ffsll((long long)sm) - 1) < me;
  if (sel) {
    L->oidx[op] = me;
    L->oval[op] = mc;
  }
  if (a.logits_out) {
#pragma unroll
    for (int i = 0; i < ROUTE_MAXI; ++i) {
      const int e = i * WAVE + lane;
      if (e < E) a.logits_out[t * E + e] = c[i];
    }
  }
  float mx_all = 0.f, den_all = 1.f;
  if (!a.renormalize) softmax_all(c, E, mx_all, den_all);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  emit_topk(a, t, L, mx_all, den_all);
}

// the 8 values of group j of a latent row, quantised (the quad of lanes holding the four
// groups of a scale block is active together)
__device__ __forceinline__ void quantize_group8(const uint4 raw, const QRows& q, int64_t j, bool mxfp8) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16lo(w[i]);
    v[2 * i + 1] = bf16hi(w[i]);
  }
  uint32_t hi[2], lo[2], shi, slo;
  quantize_quad8_fmt(v, hi, lo, shi, slo, mxfp8);
  *reinterpret_cast<uint2*>(q.hi + 8 * j) = make_uint2(hi[0], hi[1]);
  *reinterpret_cast<uint2*>(q.lo + 8 * j) = make_uint2(lo[0], lo[1]);
  if ((j & 3) == 0) {
    q.shi[j >> 2] = (uint8_t)shi;
    q.slo[j >> 2] = (uint8_t)slo;
  }
}

// the token's latent row h as two e4m3 terms for the expert kernels, eight values per
// lane and group: for L <= 8 * 64 * QH_GROUPS every group's load is issued before the
// first is used (one memory round trip per row instead of one per two groups)
constexpr int QH_GROUPS = 8;
__device__ __forceinline__ void quantize_token_h(const RouteArgs& a, int64_t t) {
  if (!a.h) return;
  const QRows q{a.hq.hi + t * a.L, a.hq.lo + t * a.L, a.hq.shi + t * (a.L / 32), a.hq.slo + t * (a.L / 32)};
  const uint16_t* h = a.h + t * a.L;
  const int ng = a.L / 8, lane = lane_id();
  if (ng > QH_GROUPS * WAVE) {
    quantize_quads(h, q, a.L, lane, WAVE, a.mxfp8 != 0);
    return;
  }
  uint4 raw[QH_GROUPS];
#pragma unroll
  for (int u = 0; u < QH_GROUPS; ++u) {
    const int j = lane + WAVE * u;
    raw[u] = j < ng ? *reinterpret_cast<const uint4*>(h + 8 * j) : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int u = 0; u < QH_GROUPS; ++u)
    if (lane + WAVE * u < ng) quantize_group8(raw[u], q, lane + WAVE * u, a.mxfp8 != 0);
}

// MINB blocks per CU: 4 caps the kernel at 128 registers a lane, spilling in the general
// path; for large batches the doubled occupancy over the 2 blocks of the uncapped build
// (172 registers) pays (prefill32k: 0.49 -> 0.33 ms), while a few dozen tokens, whose
// slowest token sets the kernel's length, run faster uncapped (decode64: 63 us against 71).
constexpr int64_t ROUTE_WIDE_TOKENS = 2048;  // 512 blocks: two per CU at the uncapped occupancy

template <int MINB>
__global__ void __launch_bounds__(256, MINB) route_kernel(RouteArgs a) {
  __shared__ RouteLds scratch[4];
  const int wave = threadIdx.x / WAVE;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= a.T) return;
  route_token(a, t, &scratch[wave]);
  quantize_token_h(a, t);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  if (a.E > ROUTE_MAXI * WAVE) return hipErrorInvalidValue;
  const dim3 grid((unsigned)ceil_div(a.T, 4));
  if (a.T >= ROUTE_WIDE_TOKENS)
    hipLaunchKernelGGL(route_kernel<4>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(route_kernel<1>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---- small batches: the grouping of routed rows by expert

// Block-wide grouping of the T*k routed rows r = t*k + j (expert sidx[r]; the k experts
// of a token are distinct and valid; T <= 64) by expert: counts, offsets, perm with
// tokens ascending inside each group, and the tile list.  Per expert, LDS holds the row
// count, the 64-bit mask of its tokens and its first row, all built with integer
// atomics (order-free); a row's place inside its group is the number of lower tokens in
// the mask.  One packed prefix sum over the experts gives offsets (low 16 bits) and tile
// slots (high 16 bits) together.
constexpr int PLACE_MAX_TOKENS = ROUTE_PLACE_TOKENS;
struct PlaceLds {
  int cnt[ROUTE_MAXI * WAVE];
  unsigned long long tmask[ROUTE_MAXI * WAVE];
  int first[ROUTE_MAXI * WAVE];
  int wsum[16];
};

__device__ void place_rows_block(const int* sidx, int T, int k, int E, PlaceLds* S, const PermOut& p) {
  const int tid = threadIdx.x, nt = blockDim.x, nw = nt / WAVE, wave = tid / WAVE, lane = lane_id();
  for (int e = tid; e < E; e += nt) {
    S->cnt[e] = 0;
    S->tmask[e] = 0ull;
    S->first[e] = 0x7FFFFFFF;
  }
  __syncthreads();
  const int rows = T * k;
  for (int r = tid; r < rows; r += nt) {
    const int e = sidx[r];
    atomicAdd(&S->cnt[e], 1);
    atomicOr(&S->tmask[e], 1ull << (r / k));
    atomicMin(&S->first[e], r);
  }
  __syncthreads();
  const int per = (E + nt - 1) / nt;  // consecutive experts per thread
  int loc = 0;
  for (int q = 0; q < per; ++q) {
    const int e = tid * per + q;
    if (e < E) loc += S->cnt[e] | ((S->cnt[e] > 0) << 16);
  }
  int wtot = 0;
  const int wex = wave_excl_scan(loc, wtot);
  if (lane == 0) S->wsum[wave] = wtot;
  __syncthreads();
  int run = wex, totals = 0;
  for (int w = 0; w < nw; ++w) {
    run += w < wave ? S->wsum[w] : 0;
    totals += S->wsum[w];
  }
  for (int q = 0; q < per; ++q) {
    const int e = tid * per + q;
    if (e < E) {
      const int c = S->cnt[e], off = run & 0xFFFF;
      p.counts[e] = c;
      p.offsets[e] = off;
      if (c > 0) p.tiles[run >> 16] = make_int4(e, off, c, S->first[e]);
      run += c | ((c > 0) << 16);
      S->cnt[e] = off;  // from here on: the group's first position
    }
  }
  const int nact = totals >> 16;
  if (tid == 0) {
    p.offsets[E] = totals & 0xFFFF;
    *p.n_active = nact;
  }
  for (int sl = nact + tid; sl < p.max_tiles; sl += nt) p.tiles[sl] = make_int4(-1, 0, 0, -1);
  __syncthreads();
  for (int r = tid; r < rows; r += nt) {
    const int e = sidx[r], t = r / k;
    p.perm[S->cnt[e] + __popcll(S->tmask[e] & ((1ull << t) - 1ull))] = r;
  }
}

// Routing of T <= ROUTE_FUSED_TOKENS tokens, the quantisation of their latent rows and
// the grouping by expert in one block.
__global__ void __launch_bounds__(512) route_permute_small_kernel(RouteArgs a, PermOut p) {
  __shared__ RouteLds scratch[8];
  __shared__ int sidx[ROUTE_FUSED_TOKENS * WAVE];
  __shared__ PlaceLds pl;
  const int wave = threadIdx.x / WAVE, nw = blockDim.x / WAVE;
  const int k = a.k, T = (int)a.T;
  for (int t = wave; t < T; t += nw) route_token(a, t, &scratch[wave]);
  // eight latent values per thread: by the waves that route no token when there are
  // some (they start at once), else by every thread, counted from the last one down so
  // that the waves with fewer tokens to route take the first ones
  if (a.h) {
    if (T < nw) {
      if (wave >= T)
        quantize_quads(a.h, a.hq, (int64_t)T * a.L, threadIdx.x - T * WAVE, blockDim.x - T * WAVE, a.mxfp8 != 0);
    } else {
      quantize_quads(a.h, a.hq, (int64_t)T * a.L, blockDim.x - 1 - threadIdx.x, blockDim.x, a.mxfp8 != 0);
    }
  }
  __syncthreads();  // token t's selection, ascending, is in scratch[t].oidx (one wave per token)
  if (T == 1) {
    // one token: its k distinct experts in ascending order are the k groups, one row
    // each.  Thread experts e = tid + i nt (i < NE, NE nt > E): offsets[e] = selections
    // below e, counts[e] = 1 if e is selected; each selection is read once.
    constexpr int NE = (ROUTE_MAXI * WAVE + 1 + 4 * WAVE - 1) / (4 * WAVE);
    const int* sel = scratch[0].oidx;
    const int nt = blockDim.x;
    int below[NE], upto[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) below[i] = upto[i] = 0;
    for (int j = 0; j < k; ++j) {
      const int sj = sel[j];
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        const int e = threadIdx.x + i * nt;
        below[i] += sj < e;
        upto[i] += sj <= e;
      }
    }
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const int e = threadIdx.x + i * nt;
      if (e <= a.E) p.offsets[e] = below[i];
      if (e < a.E) p.counts[e] = upto[i] - below[i];
    }
    for (int j = threadIdx.x; j < k; j += blockDim.x) {
      p.perm[j] = j;
      p.tiles[j] = make_int4(sel[j], j, 1, j);
    }
    for (int sl = k + threadIdx.x; sl < p.max_tiles; sl += blockDim.x) p.tiles[sl] = make_int4(-1, 0, 0, -1);
    if (threadIdx.x == 0) *p.n_active = k;
    return;
  }
  for (int r = threadIdx.x; r < T * k; r += blockDim.x) sidx[r] = scratch[r / k].oidx[r % k];
  __syncthreads();
  place_rows_block(sidx, T, k, a.E, &pl, p);
}

// One token (decode) routed by a whole block, one expert per thread.  A single wave
// holding 14 experts per lane spends most of its time in dependent instruction chains;
// here the fast logits, radii and keys of route_token are computed once per thread
// (the same fp32 values), the cut tau is the k-th largest of the maxima of 64 groups of
// consecutive experts (at least k keys reach it, so the k best are candidates), and the
// candidates are compacted in expert order and ranked by all waves (four each).  Wave 0
// certifies the boundary against every other expert's upper end and writes the
// selection, the same values route_token writes when its fast path decides; when this
// one cannot decide (more than ROUTE_CAND candidates, an uncertain boundary, weights
// over all experts) wave 0 runs route_token instead.  The other waves quantise the
// latent row meanwhile (its loads are issued with the logits'); then every thread
// writes the grouping entries of its expert.
constexpr int RB_THREADS = 1024;
constexpr int RB_WAVES = RB_THREADS / WAVE;
constexpr int RB_GROUP = RB_THREADS / WAVE;  // experts per group: one group maximum per lane
constexpr int RB_QT = RB_THREADS - WAVE;     // threads of the latent row's quantisation
static_assert(ROUTE_CAND == WAVE && ROUTE_CAND <= 4 * RB_WAVES, "four candidates ranked per wave");

struct RouteBlockLds {
  RouteLds rl;  // wave 0's candidates, output pairs and fallback scratch
  unsigned long long cpk[ROUTE_CAND];  // candidate (key, ~expert): larger ranks first
  int crank[ROUTE_CAND];
  int selpre[ROUTE_CAND + 1];  // selected candidates before candidate i
  uint32_t gmax[WAVE];
  int wcnt[RB_WAVES];
  float wup[RB_WAVES];
  uint32_t tau;
  int decided;
};

// route_token as a call: its registers are not reserved in the block kernel, where it
// runs only when the block's selection cannot decide
__attribute__((noinline)) __device__ void route_token_call(RouteArgs a, RouteLds* L) { route_token(a, 0, L); }

__global__ void __launch_bounds__(RB_THREADS) route_permute_one_kernel(RouteArgs a, PermOut p) {
  __shared__ RouteBlockLds S;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
  const int E = a.E, k = a.k;
  const int e = tid;
  const bool have = e < E;
  const int ec = have ? e : E - 1;
  const float lf = a.logits_fast[ec];
  const float bv = a.bias ? a.bias[ec] : 0.f;
  const float wn = a.wnorm[ec];
  const float xn = a.xnorm[0];
  // the first group of the latent row this thread quantises
  const int64_t ng = a.h ? a.L / 8 : 0;
  const int64_t jq = tid - WAVE;
  const bool qg = wave > 0 && jq < ng;
  const uint4 hraw = qg ? *reinterpret_cast<const uint4*>(a.h + 8 * jq) : make_uint4(0u, 0u, 0u, 0u);

  const float gam = (float)a.gamma * (1.f + 0x1p-18f) * xn;
  const float pad = (float)a.d * 0x1p-124f;
  float c = -__builtin_inff(), R = 0.f;
  uint32_t key = 0u;
  if (have) {
    c = lf + bv;
    R = gam * wn + pad + 0x1p-20f * (fabsf(lf) + fabsf(bv));
    if (bv == -__builtin_inff()) {
      const float rr = gam * wn + pad + 0x1p-20f * fabsf(lf);
      const bool known = __builtin_isfinite(lf) && __builtin_isfinite(rr) && fabsf(lf) + rr < 0x1p127f;
      c = -__builtin_inff();
      R = known ? 0.f : __builtin_inff();
    } else if (!(__builtin_isfinite(c) && __builtin_isfinite(R))) {
      c = -__builtin_inff();
      R = __builtin_inff();
    }
    key = order_key(c);
  }
  // the maximum of each 16-lane row (a group), by DPP within the row
  static_assert(RB_GROUP == 16, "a group is one DPP row");
  uint32_t gm = key;
  gm = max(gm, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)gm, DPP_QUAD_1032, 0xF, 0xF, false));
  gm = max(gm, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)gm, DPP_QUAD_2301, 0xF, 0xF, false));
  gm = max(gm, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)gm, DPP_ROW_ROR4, 0xF, 0xF, false));
  gm = max(gm, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)gm, DPP_ROW_ROR8, 0xF, 0xF, false));
  if ((lane & (RB_GROUP - 1)) == 0) S.gmax[tid / RB_GROUP] = gm;
  lds_barrier();
  if (wave == 0) {
    const uint32_t t0 = kth_of_lanes(S.gmax[lane], k);
    if (lane == 0) S.tau = t0;
  }
  lds_barrier();
  const uint32_t tau = S.tau;
  const bool cand = key != 0u && key >= tau;
  const unsigned long long cb = __ballot(cand);
  float up = -__builtin_inff();
  if (have && !cand) up = R == __builtin_inff() ? __builtin_inff() : next_up(c + R);
  up = wave_max_dpp(up);
  if (lane == 0) {
    S.wcnt[wave] = __popcll(cb);
    S.wup[wave] = up;
  }
  lds_barrier();
  int base = 0, n_c = 0;
#pragma unroll
  for (int w = 0; w < RB_WAVES; ++w) {
    const int cw = S.wcnt[w];
    base += w < wave ? cw : 0;
    n_c += cw;
  }
  // this expert's place in the candidate list (for a non-candidate: the candidates below it)
  const int pos = base + __popcll(cb & ((1ull << lane) - 1ull));
  const bool fits = n_c <= ROUTE_CAND;
  if (fits && cand) {
    S.cpk[pos] = ((unsigned long long)key << 32) | (uint32_t)~(uint32_t)e;
    S.rl.cidx[pos] = e;
    S.rl.cval[pos] = c;
    S.rl.crad[pos] = R;
  }
  lds_barrier();
  if (fits) {
    // wave w ranks candidates 4w..4w+3 against all: rank = candidates ahead of it
    const unsigned long long pj = lane < n_c ? S.cpk[lane] : 0ull;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = 4 * wave + u;
      const unsigned long long pi = __shfl(pj, i);
      const int r = __popcll(__ballot(lane < n_c && pj > pi));
      if (lane == 0 && i < n_c) S.crank[i] = r;
    }
  }
  lds_barrier();
  if (wave == 0) {
    bool fast = fits && a.renormalize && !(a.flags & MOE_ROUTE_EXACT_ALL);
    if (fast) {
      const bool live = lane < n_c;
      const bool sel = live && S.crank[lane] < k;
      const float mc = live ? S.rl.cval[lane] : 0.f, mr = live ? S.rl.crad[lane] : 0.f;
      if (k < E) {
        float Mloc = __builtin_inff(), mloc = -__builtin_inff();
        if (sel) Mloc = mr == __builtin_inff() ? -__builtin_inff() : next_down(mc - mr);
        if (live && !sel) mloc = mr == __builtin_inff() ? __builtin_inff() : next_up(mc + mr);
        if (lane < RB_WAVES) mloc = fmaxf(mloc, S.wup[lane]);
        fast = wave_min_dpp(Mloc) > wave_max_dpp(mloc);
      }
      if (fast) {
        // candidates are in expert order, so the output place is the count of selected below
        const unsigned long long sb = __ballot(sel);
        const int op = __popcll(sb & ((1ull << lane) - 1ull));
        S.selpre[lane] = op;
        if (lane == 0) S.selpre[ROUTE_CAND] = __popcll(sb);
        if (sel) {
          S.rl.oidx[op] = S.rl.cidx[lane];
          S.rl.oval[op] = mc;
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        emit_topk(a, 0, &S.rl, 0.f, 1.f);
      }
    }
    if (!fast) route_token_call(a, &S.rl);
    if (lane == 0) S.decided = fast;
  } else {
    if (qg) quantize_group8(hraw, a.hq, jq, a.mxfp8 != 0);
    if (ng > RB_QT) quantize_quads(a.h, a.hq, a.L, jq + RB_QT, RB_QT, a.mxfp8 != 0);
  }
  lds_barrier();  // the k selected experts, ascending, are in S.rl.oidx
  const bool decided = S.decided;
  if (decided && a.logits_out && have) a.logits_out[e] = c;
  // one row per selected expert: offsets[e] = selected experts below e
  int below = 0, upto = 0;
  if (decided) {
    below = S.selpre[pos < n_c ? pos : ROUTE_CAND];
    upto = below + (cand && S.crank[pos] < k);
  } else {
    for (int j = 0; j < k; ++j) {
      const int sj = S.rl.oidx[j];
      below += sj < e;
      upto += sj <= e;
    }
  }
  if (e <= E) p.offsets[e] = below;
  if (tid == 0 && E == RB_THREADS) p.offsets[E] = k;
  if (have) p.counts[e] = upto - below;
  if (tid < k) {
    p.perm[tid] = tid;
    p.tiles[tid] = make_int4(S.rl.oidx[tid], tid, 1, tid);
  }
  for (int sl = k + tid; sl < p.max_tiles; sl += RB_THREADS) p.tiles[sl] = make_int4(-1, 0, 0, -1);
  if (tid == 0) *p.n_active = k;
}

// Grouping of the rows of routed tokens (distinct, valid experts per token) for
// T <= PLACE_MAX_TOKENS and T*k <= ROUTE_SMALL_ROWS, after route_kernel.
__global__ void __launch_bounds__(1024) place_rows_kernel(const int32_t* __restrict__ idx, int T, int k, int E,
                                                          PermOut p) {
  __shared__ int sidx[ROUTE_SMALL_ROWS];
  __shared__ PlaceLds pl;
  for (int r = threadIdx.x; r < T * k; r += blockDim.x) sidx[r] = idx[r];
  __syncthreads();
  place_rows_block(sidx, T, k, E, &pl, p);
}

hipError_t launch_place_rows(const int32_t* idx, int64_t T, int32_t k, int32_t E, const PermOut& p,
                             hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (E > ROUTE_MAXI * WAVE || T > PLACE_MAX_TOKENS || T * k > ROUTE_SMALL_ROWS || k > WAVE)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(place_rows_kernel, dim3(1), dim3(1024), 0, st, idx, (int)T, k, E, p);
  return hipGetLastError();
}

hipError_t launch_route_permute_small(const RouteArgs& a, const PermOut& p, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  if (a.E > ROUTE_MAXI * WAVE || a.T > ROUTE_FUSED_TOKENS || a.k > WAVE) return hipErrorInvalidValue;
  if (a.T == 1 && a.E <= RB_THREADS && a.exact_logits == nullptr) {
    hipLaunchKernelGGL(route_permute_one_kernel, dim3(1), dim3(RB_THREADS), 0, st, a, p);
    return hipGetLastError();
  }
  // a wave per token, and at least one wave more that quantises the latent rows meanwhile
  // for T < 8
  const int nw = a.T < 4 ? 4 : 8;
  hipLaunchKernelGGL(route_permute_small_kernel, dim3(1), dim3(nw * WAVE), 0, st, a, p);
  return hipGetLastError();
}

}  // namespace moe
