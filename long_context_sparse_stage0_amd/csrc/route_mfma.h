// Stage 1 routing on bf16 MFMA for bf16 queries: chunk scores, alpha-entmax threshold,
// GQA average, bit-packed mask and the averaged weights at set bits.
//
// Method: gist.science summary of arXiv 2605.18753, "Stufe 1: Entmax-Chunk-Routing"
// (w_hat = alpha-entmax(gamma z_bar) over chunk-summary logits; the probabilities of the
// query heads sharing a KV head are averaged into one shared sparse support); aixai.ru
// blog, "Трёхстадийная архитектура" (active chunks packed in 64-bit words).  The entmax
// definition is that of Peters, Niculae and Martins (2019).
//
// Work unit: one workgroup (1 to 8 waves) per (b, kv head, R = 32/G or 16/G rows of one 64-row
// block): 32 query vectors that all route over the same chunks c < i_t.  Chunk tiles of 16
// are dealt to the waves round-robin (tile w, w + NW, ...), and every score stays in
// registers (at most 8 tiles x 2 query tiles x 4 = 64 values per lane; 16 waves cover
// 2048 chunks).
//
// estimate_diagonal (aiexpert.news, interface paragraph): the own chunk's score of each
// query vector, precomputed by k_diag_scores, is one more entry of the max, of every solver
// pass and of the normaliser; it never gets a weight or a mask bit.
//
// Scores: S^T = K_bar Q^T on v_mfma_f32_16x16x32_bf16.  Q is bf16 exactly; the fp32
// summaries are split once (by Stage 0) into bf16 hi + lo planes and both products are
// accumulated in fp32, so a score carries about 16 mantissa bits of the summary instead
// of 8 -- enough for mask bits to agree with a float64 reference outside a 1e-4 margin.
//
// Threshold solver (own design, see route_common.h): monotone steps from max y - 1 with an
// exact closed-form finish for alpha = 1.5 and 2; for alpha = 1.5 on long rows the second
// point comes from a Gaussian model of the first pass's moments, checked to be a lower
// bound of tau* before the iteration continues from it (about half the passes).  Per pass each lane reduces its own
// values, the four 16-lane groups combine by lane shuffles, and the eight waves combine
// through a double-buffered LDS table (one barrier per pass); every wave then holds the
// same totals for all 32 queries and takes the same decision.
// GQA average: the G heads of a row are G adjacent columns of a 16-lane row, summed with
// DPP (quad permutes, half-row and row mirrors) in a fixed order.
// Top-k comparison router (topk > 0, not the method): the same scores summed over the
// heads first, then a k-th-largest search by bits of an order-preserving key; the
// selected chunks get weight 1 (no prior).
#pragma once
#include <algorithm>
#include <utility>

#include "route_common.h"

namespace dash {

namespace {

// 64-bit mask words per row that can hold routed chunks (plus one spare)
constexpr int kRouteMaskWords = (kMaxRouted + 63) / 64 + 1;
// dword 3 of a raw buffer descriptor (32-bit data, byte offsets, bounds checked against the
// record count), and a byte offset beyond any record count used here
constexpr int kWbarRsrcWord3 = 0x00020000;
constexpr int kDropOffset = 0x7ffffff0;

__device__ __forceinline__ floatx4 mfma16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// one butterfly step of the sum over the G adjacent lanes of a 16-lane row that hold the
// heads of one row, applied to every value of query tile qt; the steps for G = 2, 4, 8, 16
// are the DPP moves quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
template <int CTRL, int MT, int QTR>
__device__ __forceinline__ void head_step(float (&v)[MT][QTR][4], int qt) {
#pragma unroll
  for (int j = 0; j < MT; ++j)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) v[j][qt][jj] += dpp<CTRL>(v[j][qt][jj]);
}

// reductions over the four 16-lane groups (lanes l, l^16, l^32, l^48) with the gfx950
// row-swap moves: permlane16_swap(v, v) gives each lane the values of rows {2i, 2i+1} of
// its row pair, permlane32_swap(v, v) those of the lower and the upper half-wave
template <typename Op>
__device__ __forceinline__ float xg_reduce(float v, Op op) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xg_sum(float v) {
  return xg_reduce(v, [](float x, float y) { return x + y; });
}
__device__ __forceinline__ float xg_min(float v) {
  return xg_reduce(v, [](float x, float y) { return fminf(x, y); });
}
__device__ __forceinline__ float xg_max(float v) {
  return xg_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}

}  // namespace

// One workgroup's routing with MT chunk tiles per wave (MT = ceil(ntile / NW), chosen per
// workgroup so short rows do not pay for the longest row's tile count).
template <int D, int NW, int MT, int QTR, int MODE, bool KEEP>
__device__ __forceinline__ void route_rows(const RouteArgs& a, const bf16* __restrict__ ssplit,
                                           float (&part)[2][QTR][4][16][NW],
                                           uint16_t (&mbits16)[16 * QTR][4 * kRouteMaskWords],
                                           int bk, int row0, int it, int ntile) {
  constexpr int KS = D / 32;
  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int b = bk / a.Hkv, kvh = bk % a.Hkv;
  const int T = a.Tq;

  // queries of this lane: column l16 of query tiles 0 and 1
  bf16x8 qop[QTR][KS];
  int qrow[QTR];
  // estimate_diagonal: the own chunk's score of each query vector joins the normalisation as
  // one more entry, held by the lanes of wave 0's first 16-lane group only
  const bool dsel = a.ydiag != nullptr && wv == 0 && lg == 0;
  float yd[QTR];
#pragma unroll
  for (int qt = 0; qt < QTR; ++qt) {
    const int n = 16 * qt + l16;
    const int r = n / G, g = n % G;
    qrow[qt] = r;
    const int t = min(row0 + r, T - 1);
    yd[qt] = dsel ? a.ydiag[(size_t)(b * a.Hq + kvh * G + g) * T + t] : -INFINITY;
    const bf16* qp = (const bf16*)a.q + ((size_t)(b * a.Hq + kvh * G + g) * T + t) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[qt][ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks + 8 * lg);
  }

  // scores
  const bf16* sp = ssplit + (size_t)bk * split_bk_stride(a.nc_alloc, D);
  float y[MT][QTR][4];
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int ct = wv + NW * j;
    floatx4 acc[QTR];
#pragma unroll
    for (int qt = 0; qt < QTR; ++qt) acc[qt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (ct < ntile) {  // wave-uniform
      // the tile's 16 chunk rows are allocated even past nc; rows past it are zeroed
      const int crow = 16 * ct + l16;
      const bool cok = crow < it;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 hi = *reinterpret_cast<const bf16x8*>(sp + split_offset(crow, 0, 32 * ks + 8 * lg, D));
        bf16x8 lo = *reinterpret_cast<const bf16x8*>(sp + split_offset(crow, 1, 32 * ks + 8 * lg, D));
        if (!cok) { hi = bf16x8{}; lo = bf16x8{}; }
#pragma unroll
        for (int qt = 0; qt < QTR; ++qt) acc[qt] = mfma16(hi, qop[qt][ks], acc[qt]);
#pragma unroll
        for (int qt = 0; qt < QTR; ++qt) acc[qt] = mfma16(lo, qop[qt][ks], acc[qt]);
      }
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int c = 16 * ct + 4 * lg + jj;
      const bool ok = (ct < ntile) && (c < it);
#pragma unroll
      for (int qt = 0; qt < QTR; ++qt) y[j][qt][jj] = ok ? a.zscale * acc[qt][jj] : -INFINITY;
    }
  }

  // tiles owned by this wave: wv, wv + NW, ... below ntile (wave-uniform)
  const int nj = ntile > wv ? (ntile - wv + NW - 1) / NW : 0;

  // ---- threshold solver for the 32 queries
  float tau[QTR], hi[QTR], zs[QTR], lo[QTR];
  bool done[QTR], probe[QTR];
#pragma unroll
  for (int qt = 0; qt < QTR; ++qt) {
    tau[qt] = 0.f;
    hi[qt] = 0.f;
    zs[qt] = 1.f;
    lo[qt] = 0.f;
    done[qt] = true;
    probe[qt] = false;
  }
  // long rows (alpha = 1.5) take a moment-based start after the first pass
  const int nent = a.ydiag != nullptr ? it + 1 : it;   // entries of the normalisation
  const bool model_start = MODE == kAlpha15 && nent >= kEntmaxModelMinN;
  const float inv = 1.0f / (a.alpha - 1.0f);
  int buf = 0;
  if (MODE == kTopK && it > 0) {
    // ---- top-k comparison router: group score = sum of the G heads' scores of a row (the
    // same order as their mean, G being a power of two); every chunk whose group score is
    // at least the k-th largest is selected with weight 1.  The k-th largest is the largest
    // order-preserving 32-bit key u with count(key >= u) >= k, built from the top bit down
    // with one count per bit over the workgroup; it stops as soon as that count is exactly
    // k, which already fixes the selected set.
#pragma unroll
    for (int qt = 0; qt < QTR; ++qt) {
      if (G >= 2) head_step<0xB1>(y, qt);
      if (G >= 4) head_step<0x4E>(y, qt);
      if (G >= 8) head_step<0x141>(y, qt);
      if (G >= 16) head_step<0x140>(y, qt);
    }
    // the scores become their keys in place (bit patterns only, never used as floats); an
    // absent chunk (-inf) gets a key below that of every finite score, kKeyFinite
    constexpr uint32_t kKeyFinite = 0x00800000u;
#pragma unroll
    for (int qt = 0; qt < QTR; ++qt)
#pragma unroll
      for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const uint32_t u = __float_as_uint(y[j][qt][jj]);
          y[j][qt][jj] = __uint_as_float((u & 0x80000000u) ? ~u : (u | 0x80000000u));
        }
    const int kk = a.topk;
    uint32_t thr[QTR];
    float have[QTR];                                // count(key >= thr)
#pragma unroll
    for (int qt = 0; qt < QTR; ++qt) {
      thr[qt] = 0u;
      have[qt] = (float)it;
    }
    if (it > kk) {
      for (int bit = 31; bit >= 0; --bit) {
#pragma unroll
        for (int qt = 0; qt < QTR; ++qt) {
          const uint32_t cand = max(thr[qt] | (1u << bit), kKeyFinite);
          float cnt = 0.f;
#pragma unroll
          for (int j = 0; j < MT; ++j) {
            if (j >= nj) continue;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) cnt += __float_as_uint(y[j][qt][jj]) >= cand ? 1.f : 0.f;
          }
          cnt = xg_sum(cnt);
          if (lg == 0) part[buf][qt][0][l16][wv] = cnt;
        }
        __syncthreads();
        bool settled = true;
#pragma unroll
        for (int qt = 0; qt < QTR; ++qt) {
          float tot = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) tot += part[buf][qt][0][l16][w];
          if (have[qt] != (float)kk && tot >= (float)kk) {
            thr[qt] |= 1u << bit;
            have[qt] = tot;
          }
          settled = settled && have[qt] == (float)kk;
        }
        buf ^= 1;
        // every wave read the same totals, so the exit is uniform over the workgroup
        if (__ballot(!settled) == 0ull) break;
      }
    }
#pragma unroll
    for (int qt = 0; qt < QTR; ++qt) {
      const uint32_t lim = max(thr[qt], kKeyFinite);
#pragma unroll
      for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) y[j][qt][jj] = __float_as_uint(y[j][qt][jj]) >= lim ? 1.f : 0.f;
    }
  }
  if (MODE != kTopK && it > 0) {
    // pass 0: max
#pragma unroll
    for (int qt = 0; qt < QTR; ++qt) {
      float m = yd[qt];
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        if (j < nj) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) m = fmaxf(m, y[j][qt][jj]);
        }
      }
      m = xg_max(m);
      if (lg == 0) part[buf][qt][0][l16][wv] = m;
    }
    __syncthreads();
    const float n = (float)nent;
    const float hoff = (MODE == kAlpha15) ? rsqrtf(n) : (MODE == kAlpha2 ? 1.0f / n : pow_pos(n, 1.0f - a.alpha));
#pragma unroll
    for (int qt = 0; qt < QTR; ++qt) {
      float m = part[buf][qt][0][l16][0];
#pragma unroll
      for (int w = 1; w < NW; ++w) m = fmaxf(m, part[buf][qt][0][l16][w]);
      tau[qt] = m - 1.0f;
      hi[qt] = m - hoff;
      done[qt] = false;
    }
    buf ^= 1;
    for (int pass = 0; pass < 96; ++pass) {
#pragma unroll
      for (int qt = 0; qt < QTR; ++qt) {
        float cnt = 0.f, s1 = 0.f, s2 = 0.f, mn = INFINITY;
#pragma unroll
        for (int j = -1; j < MT; ++j) {
          if (j >= nj) continue;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            if (j < 0 && jj > 0) continue;
            const float d = (j < 0 ? yd[qt] : y[j][qt][jj]) - tau[qt];
            const bool in = d > 0.f;
            const float dp = fmaxf(d, 0.f);
            cnt += in ? 1.f : 0.f;
            mn = fminf(mn, in ? d : INFINITY);
            if (MODE == kAlpha15) {
              s1 += dp;
              s2 = fmaf(dp, dp, s2);
            } else if (MODE == kAlpha2) {
              s1 += dp;
            } else if (in) {
              const float dp1 = pow_pos(d, inv - 1.0f);
              s1 += dp1;
              s2 = fmaf(dp1, d, s2);
            }
          }
        }
        cnt = xg_sum(cnt);
        s1 = xg_sum(s1);
        s2 = xg_sum(s2);
        mn = xg_min(mn);
        if (lg == 0) {
          part[buf][qt][0][l16][wv] = cnt;
          part[buf][qt][1][l16][wv] = s1;
          part[buf][qt][2][l16][wv] = s2;
          part[buf][qt][3][l16][wv] = mn;
        }
      }
      __syncthreads();
#pragma unroll
      for (int qt = 0; qt < QTR; ++qt) {
        float cnt = 0.f, s1 = 0.f, s2 = 0.f, mn = INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          cnt += part[buf][qt][0][l16][w];
          s1 += part[buf][qt][1][l16][w];
          s2 += part[buf][qt][2][l16][w];
          mn = fminf(mn, part[buf][qt][3][l16][w]);
        }
        if (done[qt]) continue;
        if (MODE == kAlpha2) {
          const float delta = (s1 - 1.0f) / cnt;
          if (delta < mn) {
            tau[qt] += delta;
            done[qt] = true;
          } else {
            tau[qt] = fminf(tau[qt] + fmaxf(delta, mn), hi[qt]);
          }
        } else if (MODE == kAlpha15) {
          const float F = s2 - 1.0f;
          if (probe[qt] && F < 0.f) {
            // the moment-based point lies past tau*.  F is convex, so its tangent there
            // meets zero at or below tau*: resume from that point or the plain step
            probe[qt] = false;
            tau[qt] = fmaxf(lo[qt], tau[qt] + F / (2.0f * s1));
            continue;
          }
          probe[qt] = false;
          const float disc = fmaf(s1, s1, -cnt * F);
          bool fin = false;
          if (disc >= 0.f) {
            const float delta = (s1 - sqrtf(disc)) / cnt;
            if (delta < mn) {
              tau[qt] += fmaxf(delta, 0.f);
              done[qt] = fin = true;
            }
          }
          if (!fin) {
            float nt = fminf(tau[qt] + fmaxf(F / (2.0f * s1), mn), hi[qt]);
            if (model_start && pass == 0) {
              const float mean = s1 / cnt, var = fmaxf(fmaf(-mean, mean, s2 / cnt), 0.f);
              const float est =
                  tau[qt] + mean + gauss_sq_tail_offset(cnt * var, kEntmaxModelTarget) * sqrtf(var);
              if (est > nt) {               // false for a NaN estimate
                lo[qt] = nt;
                nt = fminf(est, hi[qt]);
                probe[qt] = true;
              }
            }
            tau[qt] = nt;
          }
        } else {
          const float F = s2 - 1.0f;
          const float step = F / (inv * s1);
          tau[qt] = fminf(tau[qt] + fmaxf(step, 0.f), hi[qt]);
          if (step <= 3e-7f * fmaxf(1.0f, fabsf(tau[qt]))) done[qt] = true;
        }
      }
      buf ^= 1;
      bool all_done = true;
#pragma unroll
      for (int qt = 0; qt < QTR; ++qt) all_done = all_done && done[qt];
      if (__ballot(!all_done) == 0ull) break;
    }
    // normaliser
#pragma unroll
    for (int qt = 0; qt < QTR; ++qt) {
      float z = 0.f;
#pragma unroll
      for (int j = -1; j < MT; ++j) {
        if (j >= nj) continue;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          if (j < 0 && jj > 0) continue;
          const float d = (j < 0 ? yd[qt] : y[j][qt][jj]) - tau[qt];
          if (d > 0.f) z += (MODE == kAlpha15) ? d * d : (MODE == kAlpha2 ? d : pow_pos(d, inv));
        }
      }
      z = xg_sum(z);
      if (lg == 0) part[buf][qt][0][l16][wv] = z;
    }
    __syncthreads();
#pragma unroll
    for (int qt = 0; qt < QTR; ++qt) {
      float z = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) z += part[buf][qt][0][l16][w];
      zs[qt] = z;
    }
    // thresholds and normalisers kept for the backward pass (one lane per query vector);
    // compiled only into the instances the backward's recompute launches
    if (KEEP && wv == 0 && lg == 0) {
#pragma unroll
      for (int qt = 0; qt < QTR; ++qt) {
        const int n = 16 * qt + l16, t = row0 + n / G;
        if (t < T) {
          const size_t hi = (size_t)(b * a.Hq + kvh * G + n % G) * T + t;
          a.tau_out[hi] = tau[qt];
          a.z_out[hi] = zs[qt];
        }
      }
    }
  }

  // ---- weights, GQA average, w_bar at active chunks, mask bits.  After the head sum all
  // G lanes of a row hold the same averaged weights; lane g of the row stores chunk slots
  // jj = g, g + G, ... (coalesced 16-chunk runs), and each row's 16 mask bits of a tile are
  // gathered from the four 16-lane groups and stored as one 16-bit word.
  if (it > 0) {
    const int g = l16 % G;
#pragma unroll
    for (int qt = 0; qt < QTR; ++qt) {
      // 1/G of the GQA mean folded into each head's normaliser; the weights replace the
      // scores in place (chunks past it hold y = -inf, so their weight and bit are 0)
      if (MODE != kTopK) {
        const float rz = 1.0f / (zs[qt] * (float)G);
#pragma unroll
        for (int j = 0; j < MT; ++j)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            y[j][qt][jj] = entmax_weight_nonneg<MODE>(y[j][qt][jj], tau[qt], inv, rz);
        // GQA sum over the G adjacent lanes of a row, one (wave-uniform) test of G per step
        // for all of the lane's weights
        if (G >= 2) head_step<0xB1>(y, qt);
        if (G >= 4) head_step<0x4E>(y, qt);
        if (G >= 8) head_step<0x141>(y, qt);
        if (G >= 16) head_step<0x140>(y, qt);
      }
      // w_bar stores go through a buffer descriptor over this workgroup's rows that ends at
      // the last row below T: a lane with nothing to store uses an offset past the end, which
      // the hardware drops, so the stores need no branches
      const int r = qrow[qt];
      const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
          a.wbar + ((size_t)bk * a.rows + row0) * a.wbar_ld, (short)0,
          min(16 * QTR / G, T - row0) * a.wbar_ld * 4, kWbarRsrcWord3);
      const int rbase = r * a.wbar_ld;
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        if (j >= nj) continue;
        const int ct = wv + NW * j;
        const int c0 = 16 * ct + 4 * lg;
        const float* wb = y[j][qt];
        unsigned nib = 0;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) nib |= (wb[jj] > 0.f ? 1u : 0u) << jj;
        // w_bar stores at set bits: this lane's slots are jj = g + G s < 4 (G a power of two)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (s > 0 && G * s >= 4) break;      // wave-uniform
          const int jj = g + G * s;
          const float v = jj == 0 ? wb[0] : jj == 1 ? wb[1] : jj == 2 ? wb[2] : wb[3];
          const bool st = jj < 4 && ((nib >> jj) & 1u);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), wrsrc,
                                                st ? (rbase + c0 + jj) * 4 : kDropOffset, 0, 0);
        }
        // mask bits of the row for chunks 16 ct + [0, 16)
        unsigned f = nib << (4 * lg);
        {
          const auto x = __builtin_amdgcn_permlane16_swap(f, f, false, false);
          f = x[0] | x[1];
          const auto y2 = __builtin_amdgcn_permlane32_swap(f, f, false, false);
          f = y2[0] | y2[1];
        }
        mbits16[r][ct] = (uint16_t)f;           // the same word from every lane of row r
      }
    }
  }
}

// one-tile shapes are held to 4 waves per SIMD (128 registers) so that two 8-wave
// workgroups share a CU
template <int D, int NW, int MT, int QTR, int MODE, bool KEEP>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(QTR == 1 ? 4 : 1)))
void k_route_mfma(RouteArgs a, const bf16* __restrict__ ssplit, int rt_lo) {
  constexpr int NT = NW * 64;
  __shared__ float part[2][QTR][4][16][NW];
  __shared__ uint16_t mbits16[16 * QTR][4 * kRouteMaskWords];

  const int G = a.Hq / a.Hkv;
  const int R = 16 * QTR / G;                       // rows per workgroup
  const int tid = threadIdx.x;
  const int tile = gridDim.x - 1 - blockIdx.x;      // late (heavy) rows first
  const int BH = a.B * a.Hkv;
  const int rt = rt_lo + tile / BH, bk = tile % BH;
  const int row0 = rt * R;
  const int it = row0 / kChunk;                     // routed chunks c < it for every row
  const int T = a.Tq;
  const int W = a.W;
  const int ntile = (it + 15) / 16;

  uint32_t* m32 = reinterpret_cast<uint32_t*>(&mbits16[0][0]);
  for (int i = tid; i < 16 * QTR * 2 * kRouteMaskWords; i += NT) m32[i] = 0u;
  __syncthreads();
  route_rows<D, NW, MT, QTR, MODE, KEEP>(a, ssplit, part, mbits16, bk, row0, it, ntile);
  __syncthreads();
  const uint64_t* mrow = reinterpret_cast<const uint64_t*>(&mbits16[0][0]);
  for (int idx = tid; idx < R * W; idx += NT) {
    const int r = idx / W, w = idx % W;
    if (row0 + r < T)
      a.mask[((size_t)bk * a.rows + row0 + r) * W + w] =
          (w < kRouteMaskWords) ? mrow[r * kRouteMaskWords + w] : 0ull;
  }
}

template <int D, int NW, int MT, int QTR, bool KEEP>
static void launch_mt(const RouteArgs& a, const bf16* ss, int rt_lo, int rt_n, hipStream_t s) {
  dim3 grid(rt_n * a.B * a.Hkv);
  if (!KEEP && a.topk > 0)
    k_route_mfma<D, NW, MT, QTR, kTopK, false><<<grid, NW * 64, 0, s>>>(a, ss, rt_lo);
  else if (a.alpha == 1.5f)
    k_route_mfma<D, NW, MT, QTR, kAlpha15, KEEP><<<grid, NW * 64, 0, s>>>(a, ss, rt_lo);
  else if (a.alpha == 2.0f)
    k_route_mfma<D, NW, MT, QTR, kAlpha2, KEEP><<<grid, NW * 64, 0, s>>>(a, ss, rt_lo);
  else
    k_route_mfma<D, NW, MT, QTR, kAlphaGeneral, KEEP><<<grid, NW * 64, 0, s>>>(a, ss, rt_lo);
}

// Workgroup shapes by the number of 16-chunk tiles a row tile routes over.  Up to 64 tiles
// (1024 routed chunks): 32 query vectors per workgroup (two query tiles) on the fewest
// waves (NW) that hold every tile at no more than 8 tiles per wave, MT = ceil(ntile / NW).
// Beyond: one query tile (16 query vectors) on 8 waves of up to 16 tiles each, which fits
// the same registers, so every shape runs at least two workgroups per CU; they hide each
// other's barrier and memory latency (one 16-wave workgroup per CU cannot).  Rows are
// contiguous per shape (i_t grows with the row), one launch each, heaviest first.
struct RouteShape { int nw, mt, qtr; };
constexpr RouteShape kRouteShapes[] = {
    {1, 1, 2}, {1, 2, 2}, {1, 3, 2}, {1, 4, 2}, {1, 5, 2}, {1, 6, 2}, {1, 7, 2}, {1, 8, 2},
    {2, 5, 2}, {2, 6, 2}, {2, 7, 2}, {2, 8, 2}, {4, 5, 2}, {4, 6, 2}, {4, 7, 2}, {4, 8, 2},
    {8, 5, 2}, {8, 6, 2}, {8, 7, 2}, {8, 8, 2},
    {8, 9, 1}, {8, 10, 1}, {8, 11, 1}, {8, 12, 1}, {8, 13, 1}, {8, 14, 1}, {8, 15, 1},
    {8, 16, 1}};

template <int D, bool KEEP, int I>
static void launch_shape(const RouteArgs& a, const bf16* ss, int lo, int n, hipStream_t s) {
  launch_mt<D, kRouteShapes[I].nw, kRouteShapes[I].mt, kRouteShapes[I].qtr, KEEP>(a, ss, lo, n, s);
}

template <int D, bool KEEP, int... I>
static void launch_all(const RouteArgs& a, const bf16* ss, hipStream_t s,
                       std::integer_sequence<int, I...>) {
  constexpr int NS = sizeof...(I);
  using Fn = void (*)(const RouteArgs&, const bf16*, int, int, hipStream_t);
  static const Fn fns[NS] = {launch_shape<D, KEEP, I>...};
  const int G = a.Hq / a.Hkv;
  // rows [row_hi(i-1), row_hi(i)) go to shape i: i_t <= 16 cap, i.e. row < 64 (16 cap + 1)
  long long row_hi[NS];
  for (int i = 0; i < NS; ++i) {
    const long long cap = (long long)kRouteShapes[i].nw * kRouteShapes[i].mt;
    row_hi[i] = std::min<long long>(a.Tq, 64LL * (16LL * cap + 1));
  }
  row_hi[NS - 1] = a.Tq;
  for (int i = NS - 1; i >= 0; --i) {
    const long long r0 = i > 0 ? row_hi[i - 1] : 0, r1 = row_hi[i];
    if (r1 <= r0) continue;
    const int R = 16 * kRouteShapes[i].qtr / G;     // rows per workgroup (divides 64)
    const int lo = (int)(r0 / R), hi = (int)((r1 + R - 1) / R);
    fns[i](a, ss, lo, hi - lo, s);
  }
}

template <int D, bool KEEP>
static void launch_d(const RouteArgs& a, const bf16* ss, hipStream_t s) {
  constexpr int NS = sizeof(kRouteShapes) / sizeof(kRouteShapes[0]);
  launch_all<D, KEEP>(a, ss, s, std::make_integer_sequence<int, NS>{});
}

}  // namespace dash
