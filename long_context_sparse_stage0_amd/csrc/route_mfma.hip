// Stage 1 routing on bf16 MFMA for bf16 queries: chunk scores, alpha-entmax threshold,
// GQA average, bit-packed mask and the averaged weights at set bits.
//
// Method: gist.science summary of arXiv 2605.18753, "Stufe 1: Entmax-Chunk-Routing"
// (w_hat = alpha-entmax(gamma z_bar) over chunk-summary logits; the probabilities of the
// query heads sharing a KV head are averaged into one shared sparse support); aixai.ru
// blog, "Трёхстадийная архитектура" (active chunks packed in 64-bit words).  The entmax
// definition is that of Peters, Niculae and Martins (2019).
//
// Work unit: one workgroup (8 or 16 waves) per (b, kv head, R = 32/G rows of one 64-row
// block): 32 query vectors that all route over the same chunks c < i_t.  Chunk tiles of 16
// are dealt to the waves round-robin (tile w, w + NW, ...), and every score stays in
// registers (at most 8 tiles x 2 query tiles x 4 = 64 values per lane; 16 waves cover
// 2048 chunks).
//
// Scores: S^T = K_bar Q^T on v_mfma_f32_16x16x32_bf16.  Q is bf16 exactly; the fp32
// summaries are split once (by Stage 0) into bf16 hi + lo planes and both products are
// accumulated in fp32, so a score carries about 16 mantissa bits of the summary instead
// of 8 -- enough for mask bits to agree with a float64 reference outside a 1e-4 margin.
//
// Threshold solver (own design, see route_common.h): monotone steps from max y - 1 with an
// exact closed-form finish for alpha = 1.5 and 2.  Per pass each lane reduces its own
// values, the four 16-lane groups combine by lane shuffles, and the eight waves combine
// through a double-buffered LDS table (one barrier per pass); every wave then holds the
// same totals for all 32 queries and takes the same decision.
// GQA average: the G heads of a row are G adjacent columns of a 16-lane row, summed with
// DPP (quad permutes, half-row and row mirrors) in a fixed order.
#include "route_common.h"

namespace dash {

namespace {

__device__ __forceinline__ floatx4 mfma16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// sum over the G adjacent lanes of a 16-lane row that hold the heads of one row
__device__ __forceinline__ float head_sum(float v, int G) {
  if (G >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  if (G >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  if (G >= 8) v += dpp<0x141>(v);   // row_half_mirror
  if (G >= 16) v += dpp<0x140>(v);  // row_mirror
  return v;
}

__device__ __forceinline__ float xg_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}
__device__ __forceinline__ float xg_min(float v) {
  v = fminf(v, __shfl_xor(v, 16, 64));
  return fminf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float xg_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}

}  // namespace

template <int D, int NW, int MT, int MODE>
__global__ __launch_bounds__(NW * 64) void k_route_mfma(RouteArgs a, const bf16* __restrict__ ssplit) {
  constexpr int NT = NW * 64, KS = D / 32, NQ = 4;  // NQ reduced quantities per pass
  constexpr int MAXW = (kMaxRouted + 63) / 64 + 1;
  __shared__ float part[2][2][NQ][16][NW];
  __shared__ unsigned long long mbits[32][MAXW];

  const int G = a.Hq / a.Hkv;
  const int R = 32 / G;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int tile = gridDim.x - 1 - blockIdx.x;      // late (heavy) rows first
  const int BH = a.B * a.Hkv;
  const int rt = tile / BH, bk = tile % BH;
  const int b = bk / a.Hkv, kvh = bk % a.Hkv;
  const int row0 = rt * R;
  const int it = row0 / kChunk;                     // routed chunks c < it for every row
  const int T = a.Tq;
  const int W = a.W;

  for (int i = tid; i < 32 * MAXW; i += NT) (&mbits[0][0])[i] = 0ull;

  // queries of this lane: column l16 of query tiles 0 and 1
  bf16x8 qop[2][KS];
  int qrow[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int n = 16 * qt + l16;
    const int r = n / G, g = n % G;
    qrow[qt] = r;
    const int t = min(row0 + r, T - 1);
    const bf16* qp = (const bf16*)a.q + ((size_t)(b * a.Hq + kvh * G + g) * T + t) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[qt][ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks + 8 * lg);
  }

  // scores
  const int ntile = (it + 15) / 16;
  const bf16* sp = ssplit + (size_t)bk * a.nc_alloc * 2 * D;
  float y[MT][2][4];
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int ct = wv + NW * j;
    floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    if (ct < ntile) {  // wave-uniform
      const int crow = 16 * ct + l16;
      const bool cok = crow < it;
      const bf16* srow = sp + (size_t)(cok ? crow : 0) * 2 * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 hi = *reinterpret_cast<const bf16x8*>(srow + 32 * ks + 8 * lg);
        bf16x8 lo = *reinterpret_cast<const bf16x8*>(srow + D + 32 * ks + 8 * lg);
        if (!cok) { hi = bf16x8{}; lo = bf16x8{}; }
        acc0 = mfma16(hi, qop[0][ks], acc0);
        acc1 = mfma16(hi, qop[1][ks], acc1);
        acc0 = mfma16(lo, qop[0][ks], acc0);
        acc1 = mfma16(lo, qop[1][ks], acc1);
      }
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int c = 16 * ct + 4 * lg + jj;
      const bool ok = (ct < ntile) && (c < it);
      y[j][0][jj] = ok ? a.zscale * acc0[jj] : -INFINITY;
      y[j][1][jj] = ok ? a.zscale * acc1[jj] : -INFINITY;
    }
  }

  // tiles owned by this wave: wv, wv + 8, ... below ntile (wave-uniform, so the per-tile
  // blocks below are skipped by scalar branches)
  const int nj = ntile > wv ? (ntile - wv + NW - 1) / NW : 0;

  // ---- threshold solver for the 32 queries
  float tau[2] = {0.f, 0.f}, hi[2] = {0.f, 0.f}, zs[2] = {1.f, 1.f};
  bool done[2] = {true, true};
  const float inv = 1.0f / (a.alpha - 1.0f);
  int buf = 0;
  if (it > 0) {
    // pass 0: max
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float m = -INFINITY;
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
    const float n = (float)it;
    const float hoff = (MODE == kAlpha15) ? rsqrtf(n) : (MODE == kAlpha2 ? 1.0f / n : pow_pos(n, 1.0f - a.alpha));
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
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
      for (int qt = 0; qt < 2; ++qt) {
        float cnt = 0.f, s1 = 0.f, s2 = 0.f, mn = INFINITY;
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          if (j >= nj) continue;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float d = y[j][qt][jj] - tau[qt];
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
      for (int qt = 0; qt < 2; ++qt) {
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
          const float disc = fmaf(s1, s1, -cnt * F);
          bool fin = false;
          if (disc >= 0.f) {
            const float delta = (s1 - sqrtf(disc)) / cnt;
            if (delta < mn) {
              tau[qt] += fmaxf(delta, 0.f);
              done[qt] = fin = true;
            }
          }
          if (!fin) tau[qt] = fminf(tau[qt] + fmaxf(F / (2.0f * s1), mn), hi[qt]);
        } else {
          const float F = s2 - 1.0f;
          const float step = F / (inv * s1);
          tau[qt] = fminf(tau[qt] + fmaxf(step, 0.f), hi[qt]);
          if (step <= 3e-7f * fmaxf(1.0f, fabsf(tau[qt]))) done[qt] = true;
        }
      }
      buf ^= 1;
      if (__ballot(!(done[0] && done[1])) == 0ull) break;
    }
    // normaliser
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float z = 0.f;
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        if (j >= nj) continue;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float d = y[j][qt][jj] - tau[qt];
          if (d > 0.f) z += (MODE == kAlpha15) ? d * d : (MODE == kAlpha2 ? d : pow_pos(d, inv));
        }
      }
      z = xg_sum(z);
      if (lg == 0) part[buf][qt][0][l16][wv] = z;
    }
    __syncthreads();
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float z = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) z += part[buf][qt][0][l16][w];
      zs[qt] = z;
    }
  }

  // ---- weights, GQA average, mask bits, w_bar at set bits
  if (it > 0) {
    const float rG = 1.0f / (float)G;
    const size_t rbase = (size_t)bk * a.rows + row0;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float rz = 1.0f / zs[qt];
      const bool writer = (l16 % G) == 0 && (row0 + qrow[qt]) < T;
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const int ct = wv + NW * j;
        if (j >= nj) continue;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float p = entmax_weight<MODE>(y[j][qt][jj], tau[qt], inv, rz);
          const float wb = head_sum(p, G) * rG;
          const int c = 16 * ct + 4 * lg + jj;
          if (writer && wb > 0.f && c < it) {
            a.wbar[(rbase + qrow[qt]) * a.wbar_ld + c] = wb;
            atomicOr(&mbits[qrow[qt]][c >> 6], 1ull << (c & 63));
          }
        }
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < R * W; idx += NT) {
    const int r = idx / W, w = idx % W;
    if (row0 + r < T) a.mask[((size_t)bk * a.rows + row0 + r) * W + w] = (w < MAXW) ? mbits[r][w] : 0ull;
  }
}

template <int D, int NW, int MT>
static void launch_mt(const RouteArgs& a, const bf16* ss, dim3 grid, hipStream_t s) {
  if (a.alpha == 1.5f)
    k_route_mfma<D, NW, MT, kAlpha15><<<grid, NW * 64, 0, s>>>(a, ss);
  else if (a.alpha == 2.0f)
    k_route_mfma<D, NW, MT, kAlpha2><<<grid, NW * 64, 0, s>>>(a, ss);
  else
    k_route_mfma<D, NW, MT, kAlphaGeneral><<<grid, NW * 64, 0, s>>>(a, ss);
}

template <int D>
static void launch_d(const RouteArgs& a, const bf16* ss, dim3 grid, hipStream_t s) {
  const int max_it = (a.Tq - 1) / kChunk;
  const int tiles = (max_it + 15) / 16;
  if (tiles <= 8) launch_mt<D, 8, 1>(a, ss, grid, s);
  else if (tiles <= 16) launch_mt<D, 8, 2>(a, ss, grid, s);
  else if (tiles <= 32) launch_mt<D, 8, 4>(a, ss, grid, s);
  else if (tiles <= 64) launch_mt<D, 8, 8>(a, ss, grid, s);
  else launch_mt<D, 16, 8>(a, ss, grid, s);
}

hipError_t launch_route_mfma(const RouteArgs& a, const void* summ_split, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int R = 32 / G;
  dim3 grid(((a.Tq + R - 1) / R) * a.B * a.Hkv);
  if (a.D == 128) launch_d<128>(a, (const bf16*)summ_split, grid, s);
  else launch_d<64>(a, (const bf16*)summ_split, grid, s);
  return hipGetLastError();
}

}  // namespace dash
