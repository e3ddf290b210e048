// l1norm.hpp — the normalisers of a (draft, target) row pair and the L1
// distance of their softmaxes, accurate relative to L1 itself where the two
// rows nearly agree ("DSpark Speculative Decoding (Draft Training) Design",
// "Acceptance and confidence": a = clamp(1 - L1 / 2, 0, 1) with the raw L1).
//
// When the rows nearly agree, L1 = sum_v |P_v - T_v| is far below the
// rounding of either normaliser (a few 1e-7 relative in fp32), so neither
// 2 (1 - sum_v min(P_v, T_v)) nor a sum of |P_v - T_v| with separately
// normalised terms keeps relative accuracy.  Here:
//  * both rows of a part are exponentiated against ONE power-of-two shift
//    (when their maxima are within kCommonGap): D_v = 2^(d_v log2e - A),
//    T_v = 2^(t_v log2e - A), so equal logits give bit-equal terms;
//  * the normalisers are carried as Sd = sum D_v and DS = St - Sd, with DS
//    summed from per-element differences T_v - D_v, each formed without
//    cancellation: D_v expm1(t_v - d_v) by its series where
//    |t_v - d_v| < kSeriesBand (t - d is exact there for bf16 logits, and
//    rounded once for fp32), T_v - D_v otherwise (at least 1/16 apart, so
//    its relative error stays near 1e-5);
//  * with kappa = DS / Sd, P_v - T_v = (D_v kappa - (T_v - D_v)) / St, a term
//    that keeps its relative accuracy, so sum_v |.| does too.
// Softmax ignores a constant added to a row, so rows may nearly agree up to
// an offset (t_v ~ d_v + K); the target row is first moved by the pair's
// reference offset K (ref_offset: where the middle three of t_v - d_v over
// the row's first five tokens agree to 1/16, their median on a grid of
// 2^-10 so that t_v - K is exact; else, or below 2^-7, 0), and everything
// here reads t_v for t_v - K.
// Rows whose maxima are more than kCommonGap apart cannot nearly agree
// (unless they differ by an almost constant offset, where L1 is then accurate
// to about 1e-7 absolute); one shift could underflow the lower row, so each
// row takes its own shift.  Parts of a row pair (segments, workgroup slices)
// carry their own shifts and are merged exactly (power-of-two rescaling).
// The second look takes that form only for pairs that may nearly agree.  A
// part also carries AD = sum |T_v - D_v|, and for a pair
//   L1 >= (AD - |DS|) / min(Sd, St)
// (replace P by D / Sd, or T by T / Sd, and count what the replacement
// moves); where that bound reaches kFarL1 the plain overlap form
// L1 = 2 (1 - sum_v min(P_v, T_v)), one exponential per element pair, is
// accurate to about 1e-5 relative (and exactly 2 for disjoint supports).
#pragma once

#include "common.hpp"

namespace dspark {

constexpr float kCommonGap = 64.0f;     // maxima further apart: separate shifts
constexpr float kSeriesBand = 0.03125f;  // |t - d| below this: expm1 by its series
constexpr float kFarL1 = 0.125f;         // L1 bound from which the overlap form is used

// The reference offset of a pair from t_v - d_v of its first five tokens
// (non-finite values skipped; 0 unless three or more are finite and the
// middle three agree to 1/16).
__device__ __forceinline__ float ref_offset(float r0, float r1, float r2, float r3, float r4) {
  float v[5] = {r0, r1, r2, r3, r4};
  int n = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const bool ok = fabsf(v[i]) < pos_inf();  // false for +-inf and NaN
    n += ok ? 1 : 0;
    v[i] = ok ? v[i] : pos_inf();
  }
  // sort ascending (non-finite last): odd-even transposition, five rounds
#pragma unroll
  for (int rd = 0; rd < 5; ++rd)
#pragma unroll
    for (int i = rd & 1; i + 1 < 5; i += 2) {
      const float a = fminf(v[i], v[i + 1]), b = fmaxf(v[i], v[i + 1]);
      v[i] = a;
      v[i + 1] = b;
    }
  float k = 0.0f, lo = 0.0f, hi = pos_inf();
  const int m = (n - 1) / 2;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    k = i == m ? v[i] : k;
    lo = i == m - 1 ? v[i] : lo;
    hi = i == m + 1 ? v[i] : hi;
  }
  k = rintf(k * 1024.0f) * (1.0f / 1024.0f);
  return (n >= 3 && hi - lo <= 0.0625f && fabsf(k) >= 0.0078125f && fabsf(k) <= 4096.0f) ? k : 0.0f;
}

// A part of a row pair: its maxima, sd = sum D_v, x = sum (T_v - D_v) and
// ad = sum |T_v - D_v| (common shift) or x = sum T_v (separate shifts, ad
// unused).  An empty part has maxima -inf and zero sums.
struct NormPart {
  float md, mt, sd, x, ad;
};

__device__ __forceinline__ NormPart np_empty() { return NormPart{neg_inf(), neg_inf(), 0.0f, 0.0f, 0.0f}; }

__device__ __forceinline__ bool np_common(float md, float mt) {
  return md > neg_inf() && mt > neg_inf() && fabsf(md - mt) <= kCommonGap;
}

// The power-of-two shift (in log2 units, an integer) of a maximum; 0 for -inf.
__device__ __forceinline__ float shift2(float m) { return m > neg_inf() ? floorf(m * kLog2e) : 0.0f; }

__device__ __forceinline__ void np_shifts(float md, float mt, float& a2d, float& a2t) {
  if (np_common(md, mt)) {
    a2d = a2t = shift2(fmaxf(md, mt));
  } else {
    a2d = shift2(md);
    a2t = shift2(mt);
  }
}

// expm1(r) for |r| < kSeriesBand: r (1 + r/2 + r^2/6), relative error below
// r^3 / 24 (1.3e-6).
__device__ __forceinline__ float expm1_series(float r) { return r * fmaf(r, fmaf(r, 1.0f / 6.0f, 0.5f), 1.0f); }

// T - D of one element pair under a common shift; d = t = -inf gives 0.
// SELECT: both forms computed and one selected (no branch); otherwise the
// compiler may branch and form T - D only where it is taken.  Same value.
template <bool SELECT>
__device__ __forceinline__ float np_diff(float d, float t, float D, float T) {
  const float r = t - d;
  if constexpr (SELECT) {
    const float near = D * expm1_series(r), far = T - D;
    return fabsf(r) < kSeriesBand ? near : far;
  } else {
    return fabsf(r) < kSeriesBand ? D * expm1_series(r) : T - D;
  }
}

// Accumulate one element pair into a part's sums under shifts (a2d, a2t);
// COMMON: a2d == a2t, x collects T - D and ad |T - D|; else x collects T.
template <bool COMMON>
__device__ __forceinline__ void np_elem(float d, float t, float a2d, float a2t, float& sd, float& x, float& ad) {
  const float D = __builtin_amdgcn_exp2f(fmaf(d, kLog2e, -a2d));
  const float T = __builtin_amdgcn_exp2f(fmaf(t, kLog2e, -a2t));
  sd += D;
  if constexpr (COMMON) {
    const float e = np_diff<true>(d, t, D, T);
    x += e;
    ad += fabsf(e);
  } else {
    x += T;
  }
}

// A part's sums at a common shift a2 (>= the part's own shifts): (sd, ds, ad).
// A part with separate shifts has one row above the other by e^64 or more,
// so its sum |T - D| is its sum T + D.
__device__ __forceinline__ void np_at_common(const NormPart& p, float a2, float& sd, float& ds, float& ad) {
  float pd, pt;
  np_shifts(p.md, p.mt, pd, pt);
  sd = ldexpf(p.sd, static_cast<int>(pd - a2));
  if (np_common(p.md, p.mt)) {
    ds = ldexpf(p.x, static_cast<int>(pd - a2));
    ad = ldexpf(p.ad, static_cast<int>(pd - a2));
  } else {
    const float st = ldexpf(p.x, static_cast<int>(pt - a2));
    ds = st - sd;
    ad = st + sd;
  }
}

// A part's sums at separate shifts (a2d, a2t) (>= the part's own): (sd, st).
__device__ __forceinline__ void np_at_separate(const NormPart& p, float a2d, float a2t, float& sd, float& st) {
  float pd, pt;
  np_shifts(p.md, p.mt, pd, pt);
  sd = ldexpf(p.sd, static_cast<int>(pd - a2d));
  st = ldexpf(np_common(p.md, p.mt) ? p.sd + p.x : p.x, static_cast<int>(pt - a2t));
}

// Merge of parts held one per lane (lanes past n hold np_empty()): the
// combined part, on every lane (fixed reduction order).
__device__ __forceinline__ NormPart np_wave_merge(const NormPart& p) {
  const float md = wave_max(p.md), mt = wave_max(p.mt);
  float a2d, a2t, sd, x, ad = 0.0f;
  np_shifts(md, mt, a2d, a2t);
  if (np_common(md, mt)) {
    np_at_common(p, a2d, sd, x, ad);
  } else {
    np_at_separate(p, a2d, a2t, sd, x);
  }
  return NormPart{md, mt, wave_sum(sd), wave_sum(x), wave_sum(ad)};
}

// Merge of two parts (any shifts).
__device__ __forceinline__ NormPart np_merge(const NormPart& a, const NormPart& b) {
  const float md = fmaxf(a.md, b.md), mt = fmaxf(a.mt, b.mt);
  float a2d, a2t, sa, xa, sb, xb, da = 0.0f, db = 0.0f;
  np_shifts(md, mt, a2d, a2t);
  if (np_common(md, mt)) {
    np_at_common(a, a2d, sa, xa, da);
    np_at_common(b, a2d, sb, xb, db);
  } else {
    np_at_separate(a, a2d, a2t, sa, xa);
    np_at_separate(b, a2d, a2t, sb, xb);
  }
  return NormPart{md, mt, sa + sb, xa + xb, da + db};
}

// A row pair's constants for the L1 look, from its merged part:
//   a2d, a2t  the shifts of D_v and T_v
//   far       L1 >= kFarL1 (or separate shifts): the overlap form, with
//             lam2 = log2(Sd / St): min(P_v, T_v) Sd = 2^min(ud_v, ut_v + lam2)
//   kappa     DS / Sd (0 when a row is empty): the near form
//             |P_v - T_v| St = |D_v kappa - (T_v - D_v)|
//   inv_st    1 / St, isd = 1 / Sd (0 for an empty row)
//   lse_d     the draft row's log-sum-exp
//   K         the reference offset (the caller sets it)
//   empty     bit 0: draft row empty, bit 1: target row empty
struct PairK {
  float a2d, a2t, kappa, lam2;
  float inv_st, isd, lse_d, K;
  uint32_t empty, far;
};

__device__ __forceinline__ PairK pair_k(const NormPart& p) {
  PairK k;
  np_shifts(p.md, p.mt, k.a2d, k.a2t);
  const bool common = np_common(p.md, p.mt);
  const float Sd = p.sd, St = common ? p.sd + p.x : p.x;
  const float DS = common ? p.x : p.x - p.sd;
  k.empty = (Sd > 0.0f ? 0u : 1u) | (St > 0.0f ? 0u : 2u);
  k.kappa = k.empty ? 0.0f : DS / Sd;
  k.far = (!common || p.ad - fabsf(DS) >= kFarL1 * fminf(Sd, St)) ? 1u : 0u;
  k.lam2 = k.empty ? 0.0f : __log2f(Sd) - __log2f(St);
  k.inv_st = St > 0.0f ? 1.0f / St : 0.0f;
  k.isd = Sd > 0.0f ? 1.0f / Sd : 0.0f;
  k.lse_d = (k.a2d + __log2f(Sd)) * kLn2;
  k.K = 0.0f;
  return k;
}

// Near form: one element pair's |P_v - T_v| St.
__device__ __forceinline__ float l1_near(float d, float t, float a2, float kappa) {
  const float D = __builtin_amdgcn_exp2f(fmaf(d, kLog2e, -a2));
  const float T = __builtin_amdgcn_exp2f(fmaf(t, kLog2e, -a2));
  return fabsf(fmaf(D, kappa, -np_diff<false>(d, t, D, T)));
}

// Far form: one element pair's min(P_v, T_v) Sd.
__device__ __forceinline__ float l1_far(float d, float t, float a2d, float a2t, float lam2) {
  return __builtin_amdgcn_exp2f(fminf(fmaf(d, kLog2e, -a2d), fmaf(t, kLog2e, -a2t) + lam2));
}

// L1 of the pair from the summed l1_near (times St) or l1_far (times Sd).
__device__ __forceinline__ float l1_final(uint32_t empty, uint32_t far, float inv_st, float isd, float acc) {
  if (empty) return empty == 3u ? 0.0f : 1.0f;  // one row empty: L1 = the other's mass
  const float l1 = far ? 2.0f * (1.0f - acc * isd) : acc * inv_st;
  return fminf(2.0f, fmaxf(0.0f, l1));
}
__device__ __forceinline__ float l1_final(const PairK& k, float acc) {
  return l1_final(k.empty, k.far, k.inv_st, k.isd, acc);
}

}  // namespace dspark
