// Stage 1 routing, generic kernel (any dtype, any alpha): used for fp32 inputs and for
// decode (one query row per sequence).
//
// One workgroup per (b, kv head, query row) with one wave per query head of the group.
// Lane l of a wave holds the scores of chunks l, l + 64, ... (up to 2048 chunks in 32
// registers), so every reduction of the threshold solver is one wave reduction.  The G
// heads' weights are averaged in LDS in a fixed head order (deterministic), then one
// ballot per 64 chunks packs the mask word (bit c % 64 of word c / 64, LSB first) and the
// averaged weights are written where the bit is set.
//
// Method: gist.science summary of arXiv 2605.18753, "Stufe 1: Entmax-Chunk-Routing"
// (w_hat = alpha-entmax(gamma z_bar); in GQA the probabilities of the heads that share a
// KV head are averaged into one shared sparse support); aixai.ru blog,
// "Трёхстадийная архитектура" (mask packed in 64-bit words).  estimate_diagonal follows the
// aiexpert.news interface paragraph (a diagonal correction of the entmax normalisation),
// read as the own chunk's partial summary joining each head's normalisation.
#include "route_common.h"

namespace dash {

template <typename TIn, int D, int MODE>
__global__ __launch_bounds__(1024) void k_route_valu(RouteArgs a) {
  constexpr int NR = kMaxRoutedRegs;
  __shared__ float qs[16][D];
  __shared__ float wsum[kMaxRouted];
  __shared__ float kdg[D];
  const int G = a.Hq / a.Hkv;
  const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int row = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  int t = row;
  bool valid = true;
  if (a.seq_lens) {
    t = a.seq_lens[b] - 1;
    valid = (t >= 0) && (t < a.tcap);
  }
  const int it = valid ? (t / kChunk) : 0;
  const int h = kvh * G + g;
  const int tq = a.seq_lens ? 0 : t;
  const TIn* qp = (const TIn*)a.q + ((size_t)(b * a.Hq + h) * a.Tq + tq) * D;
  for (int d = lane; d < D; d += 64) qs[g][d] = to_f32(qp[d]);
  for (int c = threadIdx.x; c < kMaxRouted; c += blockDim.x) wsum[c] = 0.f;
  // estimate_diagonal: the own chunk (keys i_t C .. t) gets a summary by Stage 0's formula
  // over the keys seen so far and joins the normalisation as entry i_t.  Wave 0 builds it:
  // lane j scores key j against head_cls, softmax across lanes, then lane l accumulates
  // columns l, l + 64, ... over the keys (coalesced row reads).
  const bool diag = a.kdiag != nullptr && valid && it > 0 && it < NR * 64;
  if (diag && g == 0) {
    const TIn* kb =
        (const TIn*)a.kdiag + ((size_t)(b * a.Hkv + kvh) * a.kdiag_ld + (size_t)it * kChunk) * D;
    const TIn* hc = (const TIn*)a.head_cls + (size_t)kvh * D;
    const int nk = t - it * kChunk + 1;
    float lg = -INFINITY;
    if (lane < nk) {
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = fmaf(to_f32(hc[d]), to_f32(kb[(size_t)lane * D + d]), acc);
      lg = acc * a.s0_scale_log2;
    }
    const float m = wave_max(lg);
    const float e = lane < nk ? fast_exp2(lg - m) : 0.f;
    const float pj = e / wave_sum(e);
    for (int d = lane; d < D; d += 64) {
      float acc = 0.f;
      for (int j = 0; j < nk; ++j) acc = fmaf(__shfl(pj, j), to_f32(kb[(size_t)j * D + d]), acc);
      kdg[d] = acc;
    }
  }
  __syncthreads();
  float ydiag = -INFINITY;
  if (diag) {
    float acc = 0.f;
    for (int d = lane; d < D; d += 64) acc = fmaf(qs[g][d], kdg[d], acc);
    ydiag = a.zscale * wave_sum(acc);
  }

  float y[NR];
  const float* sb = a.summ + (size_t)(b * a.Hkv + kvh) * a.nc_alloc * D;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int c = lane + 64 * r;
    y[r] = -INFINITY;
    if (c < it) {
      const float4* srow = reinterpret_cast<const float4*>(sb + (size_t)c * D);
      float acc = 0.f;
#pragma unroll 8
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const float4 s4 = srow[d4];
        acc = fmaf(qs[g][4 * d4 + 0], s4.x, acc);
        acc = fmaf(qs[g][4 * d4 + 1], s4.y, acc);
        acc = fmaf(qs[g][4 * d4 + 2], s4.z, acc);
        acc = fmaf(qs[g][4 * d4 + 3], s4.w, acc);
      }
      y[r] = a.zscale * acc;
    } else if (c == it && diag) {
      y[r] = ydiag;
    }
  }
  float p[NR];
  if (it > 0) {
    float z;
    const float tau = entmax_threshold<MODE, NR>(y, diag ? it + 1 : it, a.alpha, WaveReduce(), &z);
    const float rz = 1.0f / z, inv = 1.0f / (a.alpha - 1.0f);
    if (a.tau_out != nullptr && lane == 0 && a.seq_lens == nullptr) {
      const size_t hi = (size_t)(b * a.Hq + h) * a.Tq + t;
      a.tau_out[hi] = tau;
      a.z_out[hi] = z;
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) p[r] = entmax_weight<MODE>(y[r], tau, inv, rz);
  } else {
#pragma unroll
    for (int r = 0; r < NR; ++r) p[r] = 0.f;
  }
  // fixed-order sum over the G heads (the own chunk's weight, at c = i_t, is dropped below:
  // it stays attended with log-prior 0)
  for (int gg = 0; gg < G; ++gg) {
    if (g == gg) {
#pragma unroll
      for (int r = 0; r < NR; ++r) wsum[lane + 64 * r] += p[r];
    }
    __syncthreads();
  }
  const float rG = 1.0f / (float)G;
  const size_t rowi = (size_t)(b * a.Hkv + kvh) * a.rows + (a.seq_lens ? 0 : t);
  for (int w = g; w < a.W; w += G) {
    const int c = lane + 64 * w;
    const float wb = (c < kMaxRouted) ? wsum[c] * rG : 0.f;
    const bool on = valid && (c < it) && (wb > 0.f);
    const uint64_t bits = __ballot(on);
    if (on) a.wbar[rowi * a.wbar_ld + c] = wb;
    if (lane == 0) a.mask[rowi * a.W + w] = bits;
  }
}

template <typename TIn, int D>
static hipError_t launch_route_valu_t(const RouteArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  dim3 grid(a.rows, a.Hkv, a.B), block(64 * G);
  if (a.alpha == 1.5f)
    k_route_valu<TIn, D, kAlpha15><<<grid, block, 0, s>>>(a);
  else if (a.alpha == 2.0f)
    k_route_valu<TIn, D, kAlpha2><<<grid, block, 0, s>>>(a);
  else
    k_route_valu<TIn, D, kAlphaGeneral><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_route_valu(const RouteArgs& a, hipStream_t s) {
  if (a.dtype == 0)
    return a.D == 128 ? launch_route_valu_t<bf16, 128>(a, s) : launch_route_valu_t<bf16, 64>(a, s);
  return a.D == 128 ? launch_route_valu_t<float, 128>(a, s) : launch_route_valu_t<float, 64>(a, s);
}

}  // namespace dash
