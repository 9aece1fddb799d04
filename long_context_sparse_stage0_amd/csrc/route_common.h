// alpha-entmax threshold solver shared by the Stage 1 kernels.
//
// alpha-entmax (Peters, Niculae and Martins 2019; used for chunk routing in arXiv
// 2605.18753, gist.science "Stufe 1: Entmax-Chunk-Routing"):
//   p_c = [y_c - tau]_+^(1/(alpha-1)),  y = (alpha-1) * gamma * s * <q, k_bar_c>,
//   tau fixed by sum_c p_c = 1.
// F(tau) = sum_c [y_c - tau]_+^(1/(alpha-1)) - 1 is convex and decreasing, and
// tau* lies in [max y - 1, max y - n^(1-alpha)].
//
// Solver (own design): start at the left end tau_0 = max y - 1 (F >= 0) and step right,
// never past tau*, so the current support S = {y > tau} always contains the true one.
// Each pass reduces, over S, the count, sum d, sum d^2 (or the needed powers) and the
// smallest d = y - tau; from these:
//   alpha = 2  : the root of the linear piece, delta = (sum d - 1)/|S|; exact and final
//                if delta < min d, otherwise a Newton step (which it equals).
//   alpha = 1.5: the smaller root of |S| delta^2 - 2 delta sum d + sum d^2 - 1 = 0 is the
//                exact answer if it stays below min d (the support does not change);
//                otherwise tau* > tau + min d, and the step is max(Newton, min d).
//   other alpha: safeguarded Newton steps until the step is below fp32 resolution.
// Every step is a valid lower bound (Newton from the left on a convex function, or a
// point where F is still positive), so the iteration is monotone and each pass that does
// not finish drops at least one element.
// For alpha = 1.5 and at least kEntmaxModelMinN entries, the starting point comes from a
// Gaussian model of the entries' moments instead (see gauss_sq_tail_offset); it is used only
// after a pass confirms F >= 0 there, so the same invariants hold.
#pragma once
#include "dash_internal.h"

namespace dash {

enum { kAlphaGeneral = 0, kAlpha15 = 1, kAlpha2 = 2, kTopK = 3 };  // kTopK: comparison router

__device__ __forceinline__ float pow_pos(float d, float e) {  // d > 0
  return fast_exp2(e * fast_log2(d));
}

// Cross-lane reduction hooks: the generic kernel reduces over a whole wave; the MFMA
// kernel supplies its own combination over lanes and waves.
struct WaveReduce {
  __device__ __forceinline__ float sum(float v) const { return wave_sum(v); }
  __device__ __forceinline__ float min(float v) const { return wave_min(v); }
  __device__ __forceinline__ float max(float v) const { return wave_max(v); }
};

// smallest unsigned value over the wave (DPP steps inside each 16-lane row, then the row
// swaps); used on the bit patterns of non-negative floats, which order like the floats
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  v = ::min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = ::min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = ::min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = ::min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = ::min(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return ::min(b[0], b[1]);
}

// Start point from the first pass's moments (own design, alpha = 1.5).  With the scores
// modelled as Gaussian with the mean and variance v of the current support (n entries),
// sum_c [y_c - tau]_+^2 at tau = mean + a sqrt(v) is n v g(a), g(a) = E[(Z - a)_+^2]
// = (1 + a^2) Q(a) - a phi(a) for a standard normal Z (Q its upper tail, phi its density).
// Returns the a solving n v g(a) = target by Newton steps from a = 0 (g is decreasing and
// convex, g' = -2 (phi(a) - a Q(a))).  A target above 1 leans the estimate left of tau*;
// the caller still checks that the point is a lower bound before relying on it.
// Q comes from the rational erfc approximation 7.1.26 of Abramowitz and Stegun (absolute
// error below 1.5e-7), which shares the factor exp(-a^2 / 2) with phi, so a step costs one
// exp2 and two reciprocals.
__device__ __forceinline__ float gauss_sq_tail_offset(float nv, float target) {
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const float e = fast_exp2(-0.72134752f * a * a);              // exp(-a^2 / 2)
    const float tt = __builtin_amdgcn_rcpf(fmaf(0.23164189f, fabsf(a), 1.f));  // p / sqrt 2
    const float poly =
        tt * fmaf(tt, fmaf(tt, fmaf(tt, fmaf(tt, 1.061405429f, -1.453152027f), 1.421413741f),
                           -0.284496736f), 0.254829592f);
    const float qh = 0.5f * poly * e;                             // Q(|a|)
    const float Q = a >= 0.f ? qh : 1.f - qh;
    const float ph = 0.39894228f * e;
    const float g = fmaf(a, a, 1.f) * Q - a * ph;
    const float h = ph - a * Q;
    a += (nv * g - target) * __builtin_amdgcn_rcpf(2.f * nv * h);
  }
  return a;
}

// Moment-based start (alpha = 1.5) from this many entries on, aiming at a squared-excess
// sum of kEntmaxModelTarget, i.e. a little left of tau*.
constexpr int kEntmaxModelMinN = 256;
constexpr float kEntmaxModelTarget = 1.25f;

// y[NR]: this lane's scores ((alpha-1)-scaled), -inf for absent entries.
// Returns tau; *zsum receives sum_c [y_c - tau]_+^(1/(alpha-1)) (the normaliser).
// Called with every lane of the wave active: the reductions and the support count (a popcount
// of the wave's comparison mask) span all 64 lanes.
template <int MODE, int NR, class Red>
__device__ float entmax_threshold(const float (&y)[NR], int n, float alpha, const Red& red,
                                  float* zsum) {
  // alpha = 1.5 with many entries starts from a point given by the moments of all entries
  // (gauss_sq_tail_offset), gathered with the max; the first pass checks it is still a lower
  // bound of tau*, else the solver resumes at the tangent of F there, which lies at or below
  // tau* (F is convex), or at max - 1
  const bool model = MODE == kAlpha15 && n >= kEntmaxModelMinN;
  float m = -INFINITY, sy = 0.f, syy = 0.f;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    m = fmaxf(m, y[r]);
    if (model) {
      const float v = y[r] > -INFINITY ? y[r] : 0.f;   // absent entries are -inf
      sy += v;
      syy = fmaf(v, v, syy);
    }
  }
  m = red.max(m);
  float tau = m - 1.0f;
  const float inv = 1.0f / (alpha - 1.0f);
  const float hi = m - ((MODE == kAlpha15) ? rsqrtf((float)n)
                                            : (MODE == kAlpha2 ? 1.0f / (float)n
                                                               : pow_pos((float)n, 1.0f - alpha)));
  bool probe = false;
  float lo = tau;
  if (model) {
    const float nf = (float)n;
    const float mean = red.sum(sy) / nf;
    const float var = fmaxf(fmaf(-mean, mean, red.sum(syy) / nf), 0.f);
    const float est = mean + gauss_sq_tail_offset(nf * var, kEntmaxModelTarget) * sqrtf(var);
    if (est > tau) {                              // false for a NaN estimate
      tau = fminf(est, hi);
      probe = true;
    }
  }
  for (int it = 0; it < 96; ++it) {
    float s1 = 0.f, s2 = 0.f, mn = INFINITY, cnt;
    if constexpr (MODE == kAlpha15 || MODE == kAlpha2) {
      // branch-free: entries outside the support add +0 (and fma(0, 0, s2) = s2), the
      // count is the popcount of the wave's comparison mask, and the support's smallest
      // excess is an unsigned min over the bit patterns (positive floats order like them)
      uint32_t mnb = 0x7f800000u;                   // +inf
      int cw = 0;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float d = y[r] - tau;
        const bool in = d > 0.f;
        cw += __builtin_popcountll(__builtin_amdgcn_ballot_w64(in));
        const float dp = in ? d : 0.f;
        s1 += dp;
        if (MODE == kAlpha15) s2 = fmaf(dp, dp, s2);
        mnb = ::min(mnb, in ? __float_as_uint(d) : 0x7f800000u);
      }
      cnt = (float)cw;
      s1 = red.sum(s1);
      if (MODE == kAlpha15) s2 = red.sum(s2);
      mn = __uint_as_float(wave_umin(mnb));
    } else {
      int icnt = 0;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float d = y[r] - tau;
        if (d > 0.f) {
          ++icnt;
          mn = fminf(mn, d);
          const float dp1 = pow_pos(d, inv - 1.0f);  // d^(p-1)
          s1 += dp1;                                 // for F'
          s2 = fmaf(dp1, d, s2);                     // d^p, for F
        }
      }
      cnt = red.sum((float)icnt);
      s1 = red.sum(s1);
      s2 = red.sum(s2);
      mn = red.min(mn);
    }
    if (MODE == kAlpha2) {
      const float delta = (s1 - 1.0f) / cnt;
      if (delta < mn) {
        tau += delta;
        break;
      }
      tau = fminf(tau + fmaxf(delta, mn), hi);
    } else if (MODE == kAlpha15) {
      const float F = s2 - 1.0f;
      if (probe && F < 0.f) {
        probe = false;
        tau = fmaxf(lo, tau + F / (2.0f * s1));
        continue;
      }
      probe = false;
      const float disc = fmaf(s1, s1, -cnt * F);
      if (disc >= 0.f) {
        const float delta = (s1 - sqrtf(disc)) / cnt;
        if (delta < mn) {
          tau += fmaxf(delta, 0.f);
          break;
        }
      }
      tau = fminf(tau + fmaxf(F / (2.0f * s1), mn), hi);
    } else {
      const float F = s2 - 1.0f;
      const float step = F / (inv * s1);
      tau = fminf(tau + fmaxf(step, 0.f), hi);
      if (step <= 3e-7f * fmaxf(1.0f, fabsf(tau))) break;
    }
  }
  float z = 0.f;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float d = y[r] - tau;
    if constexpr (MODE == kAlpha15) {
      const float dp = d > 0.f ? d : 0.f;        // +0 outside the support
      z += dp * dp;
    } else if constexpr (MODE == kAlpha2) {
      z += d > 0.f ? d : 0.f;
    } else {
      if (d > 0.f) z += pow_pos(d, inv);
    }
  }
  *zsum = red.sum(z);
  return tau;
}

template <int MODE>
__device__ __forceinline__ float entmax_weight(float y, float tau, float inv, float rz) {
  const float d = y - tau;
  if (!(d > 0.f)) return 0.f;
  const float p = (MODE == kAlpha15) ? d * d : (MODE == kAlpha2 ? d : pow_pos(d, inv));
  return p * rz;
}

// The same weight without a branch, for bulk use: max(d, 0) gives +0 outside the support.
template <int MODE>
__device__ __forceinline__ float entmax_weight_nonneg(float y, float tau, float inv, float rz) {
  const float d = fmaxf(y - tau, 0.f);
  if (MODE == kAlpha15) return d * (d * rz);
  if (MODE == kAlpha2) return d * rz;
  return d > 0.f ? pow_pos(d, inv) * rz : 0.f;
}

}  // namespace dash
