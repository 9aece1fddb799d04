// Backward pass, generic kernels (any dtype): gradients of a loss with respect to q, k, v
// and head_cls through all three stages, given dL/dout.
//
// Method: the pages' central claim is end-to-end differentiability -- alpha-entmax has a
// Jacobian almost everywhere, so the gradient flows from the token-level attention through
// the routing distribution back to the chunk summaries and Stage 0's classifier query
// (gist.science summary of arXiv 2605.18753, "Stufe 1: Entmax-Chunk-Routing", remark on
// differentiability, and "Hauptbeiträge").  The entmax Jacobian is that of Peters, Niculae
// and Martins (2019): with s = p^(2 - alpha) on the support, dx = s dp - s (s . dp) / sum s.
//
// Kernels, in launch order (the forward's mask, weights, thresholds tau / normalisers z and
// log-sum-exp are recomputed or passed in):
//   k_bwd_attend_row  one wave per (b, head, row): recomputes the row's probabilities from
//                     the saved log-sum-exp, dl = P (dP - <dO, O>); dq (fp32) stored,
//                     dk, dv accumulated by atomics, and dw_bar = sigma / w_bar * sum of dl
//                     over the chunk's keys, accumulated over the G heads by atomics.
//   k_bwd_route_row   one workgroup per (b, kv head, row), one wave per head: recomputes
//                     the head's entmax weights from its saved tau, z; dp = dw_bar / G,
//                     dx = s (dp - rho); dq += gamma scale dx k_bar (final dq written);
//                     d k_bar += gamma scale dx q by atomics.
//   k_bwd_stage0      one wave per (b, kv head, chunk): Stage 0's softmax backwards,
//                     dk = dk(Stage 2) + pi d k_bar + scale da head_cls (final dk, and dv
//                     from its fp32 accumulator when there is one), and the chunk's part of
//                     d head_cls.  Also run after the MFMA kernels (backward_mfma.hip).
//   k_bwd_reduce_hc   d head_cls summed over batch and chunks in a fixed order.
#include "route_common.h"

namespace dash {

template <typename TIn, int D>
__global__ __launch_bounds__(64) void k_bwd_attend_row(BackwardArgs a) {
  constexpr int E = D / 64;
  __shared__ float qs[D], dos[D];
  __shared__ float ps[64], dls[64];
  const int lane = threadIdx.x;
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.Hkv, kvh = h / G;
  const int T = a.T;
  const size_t qi = (size_t)(b * a.Hq + h) * T + t;
  const TIn* qp = (const TIn*)a.q + qi * D;
  const TIn* dop = (const TIn*)a.dout + qi * D;
  const TIn* op = (const TIn*)a.out + qi * D;
  float delta = 0.f;
  for (int d = lane; d < D; d += 64) {
    qs[d] = to_f32(qp[d]);
    const float g = to_f32(dop[d]);
    dos[d] = g;
    delta = fmaf(g, to_f32(op[d]), delta);
  }
  delta = wave_sum(delta);
  __syncthreads();
  const float sl2 = a.scale * 1.4426950408889634f;
  const float lse2 = a.lse[qi] * 1.4426950408889634f;
  const int it = t / kChunk;
  const size_t kvbase = (size_t)(b * a.Hkv + kvh) * T;
  const TIn* kb = (const TIn*)a.k + kvbase * D;
  const TIn* vb = (const TIn*)a.v + kvbase * D;
  float* dkb = a.dk32 + kvbase * D;
  float* dvb = a.dv32 + kvbase * D;
  const size_t rowi = (size_t)(b * a.Hkv + kvh) * T + t;
  float dq[E];
#pragma unroll
  for (int e = 0; e < E; ++e) dq[e] = 0.f;

  // one 64-key chunk: bias2 in base-2 units (sigma log2 w_bar, 0 on the diagonal)
  auto visit = [&](int c, float bias2, float wb) {
    const int j = c * kChunk + lane;
    float p = 0.f, dl = 0.f;
    if (j <= t) {
      const TIn* kr = kb + (size_t)j * D;
      const TIn* vr = vb + (size_t)j * D;
      float s = 0.f, dp = 0.f;
      for (int d = 0; d < D; ++d) {
        s = fmaf(qs[d], to_f32(kr[d]), s);
        dp = fmaf(dos[d], to_f32(vr[d]), dp);
      }
      p = fast_exp2(fmaf(s, sl2, bias2) - lse2);
      dl = p * (dp - delta);
    }
    ps[lane] = p;
    dls[lane] = dl;
    if (wb > 0.f) {                      // a routed chunk: its bias is sigma log w_bar
      const float sdl = wave_sum(dl);
      if (lane == 0) atomicAdd(a.dwb + rowi * a.nc + c, a.sigma * sdl / wb);
    }
    __syncthreads();
    const int jn = min(kChunk, t + 1 - c * kChunk);
    for (int jj = 0; jj < jn; ++jj) {
      const float pj = ps[jj], dlj = dls[jj];
      const size_t row = (size_t)(c * kChunk + jj) * D;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int d = lane * E + e;
        dq[e] = fmaf(dlj, to_f32(kb[row + d]), dq[e]);
        atomicAdd(dkb + row + d, a.scale * dlj * qs[d]);
        atomicAdd(dvb + row + d, pj * dos[d]);
      }
    }
    __syncthreads();
  };

  for (int w = 0; w * 64 < it; ++w) {
    uint64_t bits = a.mask[rowi * a.W + w];
    while (bits) {
      const int c = 64 * w + __builtin_ctzll(bits);
      bits &= bits - 1;
      const float wb = a.wbar[rowi * a.nc + c];
      visit(c, a.sigma * fast_log2(wb), wb);
    }
  }
  visit(it, 0.f, 0.f);
#pragma unroll
  for (int e = 0; e < E; ++e) a.dq32[qi * D + lane * E + e] = a.scale * dq[e];
}

// Stage 1 backwards for one row: wave g = head g of the kv head.
template <typename TIn, int D, int MODE>
__global__ __launch_bounds__(1024) void k_bwd_route_row(BackwardArgs a) {
  constexpr int NR = kMaxRoutedRegs;
  __shared__ float qs[16][D];
  __shared__ float dxs[16][kMaxRouted];
  const int G = a.Hq / a.Hkv;
  const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int t = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int T = a.T;
  const int it = t / kChunk;
  const int h = kvh * G + g;
  const size_t qi = (size_t)(b * a.Hq + h) * T + t;
  const TIn* qp = (const TIn*)a.q + qi * D;
  for (int d = lane; d < D; d += 64) qs[g][d] = to_f32(qp[d]);
  __syncthreads();
  const float* sb = a.summ + (size_t)(b * a.Hkv + kvh) * a.nc * D;
  const size_t rowi = (size_t)(b * a.Hkv + kvh) * T + t;
  const float gs = a.gamma * a.scale;                  // dL/d<q, k_bar> = gs * dL/dx
  if (it > 0) {
    const float zscale = (a.alpha - 1.0f) * gs;
    const float tau = a.tau[qi], rz = 1.0f / a.z[qi];
    const float inv = 1.0f / (a.alpha - 1.0f), rG = 1.0f / (float)G;
    float sv[NR], dp[NR];
    float ssum = 0.f, sdp = 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int c = lane + 64 * r;
      sv[r] = 0.f;
      dp[r] = 0.f;
      if (c < it) {
        const float4* srow = reinterpret_cast<const float4*>(sb + (size_t)c * D);
        float acc = 0.f;
        for (int d4 = 0; d4 < D / 4; ++d4) {
          const float4 s4 = srow[d4];
          acc = fmaf(qs[g][4 * d4 + 0], s4.x, acc);
          acc = fmaf(qs[g][4 * d4 + 1], s4.y, acc);
          acc = fmaf(qs[g][4 * d4 + 2], s4.z, acc);
          acc = fmaf(qs[g][4 * d4 + 3], s4.w, acc);
        }
        const float p = entmax_weight<MODE>(zscale * acc, tau, inv, rz);
        if (p > 0.f) {
          sv[r] = (MODE == kAlpha15) ? sqrtf(p) : (MODE == kAlpha2 ? 1.f : pow_pos(p, 2.0f - a.alpha));
          const bool on = (a.mask[rowi * a.W + (c >> 6)] >> (c & 63)) & 1ull;
          dp[r] = on ? a.dwb[rowi * a.nc + c] * rG : 0.f;
        }
        ssum += sv[r];
        sdp = fmaf(sv[r], dp[r], sdp);
      }
    }
    ssum = wave_sum(ssum);
    sdp = wave_sum(sdp);
    const float rho = ssum > 0.f ? sdp / ssum : 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int c = lane + 64 * r;
      if (c < it) dxs[g][c] = gs * sv[r] * (dp[r] - rho);
    }
  }
  __syncthreads();
  // dq = Stage 2's part + gs sum_c dx_c k_bar_c
  for (int d = lane; d < D; d += 64) {
    float acc = a.dq32[qi * D + d];
    for (int c = 0; c < it; ++c) acc = fmaf(dxs[g][c], sb[(size_t)c * D + d], acc);
    ((TIn*)a.dq)[qi * D + d] = from_f32<TIn>(acc);
  }
  // d k_bar_c += sum over the heads of dx_c q_h
  float* dsb = a.dsumm + (size_t)(b * a.Hkv + kvh) * a.nc * D;
  for (int idx = threadIdx.x; idx < it * D; idx += blockDim.x) {
    const int c = idx / D, d = idx % D;
    float acc = 0.f;
    for (int gg = 0; gg < G; ++gg) acc = fmaf(dxs[gg][c], qs[gg][d], acc);
    if (acc != 0.f) atomicAdd(dsb + (size_t)c * D + d, acc);
  }
}

// Stage 0 backwards, one wave per (b, kv head, chunk); lane l owns columns [l E, l E + E).
template <typename TIn, int D>
__global__ __launch_bounds__(64) void k_bwd_stage0(BackwardArgs a) {
  constexpr int E = D / 64;
  __shared__ float red[64][65];
  __shared__ float pis[64], das[64];
  const int lane = threadIdx.x;
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int T = a.T;
  const size_t base = ((size_t)(b * a.Hkv + kvh) * T + (size_t)c * kChunk) * D;
  const TIn* kc = (const TIn*)a.k + base;
  const int nrow = min(kChunk, T - c * kChunk);
  const bool full = nrow == kChunk;
  float* dhp = a.dhc_part + ((size_t)(b * a.Hkv + kvh) * a.nc + c) * D;
  if (!full) {
    for (int j = 0; j < nrow; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const size_t i = base + (size_t)j * D + lane * E + e;
        ((TIn*)a.dk)[i] = from_f32<TIn>(a.dk32[i]);
        if (a.dv32 != nullptr) ((TIn*)a.dv)[i] = from_f32<TIn>(a.dv32[i]);
      }
#pragma unroll
    for (int e = 0; e < E; ++e) dhp[lane * E + e] = 0.f;
    return;
  }
  const float sl2 = a.scale * 1.4426950408889634f;
  float hcv[E], gv[E], kbar[E];
  const float* gsrc = a.dsumm + ((size_t)(b * a.Hkv + kvh) * a.nc + c) * D;
  const float* ksrc = a.summ + ((size_t)(b * a.Hkv + kvh) * a.nc + c) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    hcv[e] = to_f32(((const TIn*)a.head_cls)[kvh * D + lane * E + e]);
    gv[e] = gsrc[lane * E + e];
    kbar[e] = ksrc[lane * E + e];
  }
  // logits and <d k_bar, k_j>, reduced across lanes through LDS (row j -> lane j)
  for (int j = 0; j < kChunk; ++j) {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) part = fmaf(hcv[e], to_f32(kc[(size_t)j * D + lane * E + e]), part);
    red[j][lane] = part;
  }
  __syncthreads();
  float alog = 0.f;
  for (int i = 0; i < 64; ++i) alog += red[lane][i];
  __syncthreads();
  for (int j = 0; j < kChunk; ++j) {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) part = fmaf(gv[e], to_f32(kc[(size_t)j * D + lane * E + e]), part);
    red[j][lane] = part;
  }
  __syncthreads();
  float gk = 0.f;
  for (int i = 0; i < 64; ++i) gk += red[lane][i];
  float gkbar = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) gkbar = fmaf(gv[e], kbar[e], gkbar);
  gkbar = wave_sum(gkbar);
  const float a2 = alog * sl2;
  const float mx = wave_max(a2);
  const float pe = fast_exp2(a2 - mx);
  const float pi = pe / wave_sum(pe);
  pis[lane] = pi;
  das[lane] = pi * (gk - gkbar);
  __syncthreads();
  float dh[E];
#pragma unroll
  for (int e = 0; e < E; ++e) dh[e] = 0.f;
  for (int j = 0; j < kChunk; ++j) {
    const float pj = pis[j], daj = das[j];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const size_t i = base + (size_t)j * D + lane * E + e;
      const float kv = to_f32(kc[(size_t)j * D + lane * E + e]);
      ((TIn*)a.dk)[i] = from_f32<TIn>(a.dk32[i] + pj * gv[e] + a.scale * daj * hcv[e]);
      if (a.dv32 != nullptr) ((TIn*)a.dv)[i] = from_f32<TIn>(a.dv32[i]);
      dh[e] = fmaf(daj, kv, dh[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) dhp[lane * E + e] = a.scale * dh[e];
}

// d head_cls [Hkv, D] = sum over b and chunks of the per-chunk parts (fixed order)
__global__ void k_bwd_reduce_hc(BackwardArgs a) {
  const int kvh = blockIdx.x;
  for (int d = threadIdx.x; d < a.D; d += blockDim.x) {
    float acc = 0.f;
    for (int b = 0; b < a.B; ++b)
      for (int c = 0; c < a.nc; ++c)
        acc += a.dhc_part[((size_t)(b * a.Hkv + kvh) * a.nc + c) * a.D + d];
    a.dhead_cls[kvh * a.D + d] = acc;
  }
}

template <typename TIn, int D>
static hipError_t launch_backward_valu_t(const BackwardArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  k_bwd_attend_row<TIn, D><<<dim3(a.T, a.Hq, a.B), 64, 0, s>>>(a);
  if (a.alpha == 1.5f)
    k_bwd_route_row<TIn, D, kAlpha15><<<dim3(a.T, a.Hkv, a.B), 64 * G, 0, s>>>(a);
  else if (a.alpha == 2.0f)
    k_bwd_route_row<TIn, D, kAlpha2><<<dim3(a.T, a.Hkv, a.B), 64 * G, 0, s>>>(a);
  else
    k_bwd_route_row<TIn, D, kAlphaGeneral><<<dim3(a.T, a.Hkv, a.B), 64 * G, 0, s>>>(a);
  return hipGetLastError();
}

template <typename TIn, int D>
static hipError_t launch_backward_stage0_t(const BackwardArgs& a, hipStream_t s) {
  k_bwd_stage0<TIn, D><<<dim3(a.nc, a.Hkv, a.B), 64, 0, s>>>(a);
  k_bwd_reduce_hc<<<a.Hkv, 128, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_backward_valu(const BackwardArgs& a, hipStream_t s) {
  if (a.dtype == 0)
    return a.D == 128 ? launch_backward_valu_t<bf16, 128>(a, s) : launch_backward_valu_t<bf16, 64>(a, s);
  return a.D == 128 ? launch_backward_valu_t<float, 128>(a, s) : launch_backward_valu_t<float, 64>(a, s);
}

hipError_t launch_backward_stage0(const BackwardArgs& a, hipStream_t s) {
  if (a.dtype == 0)
    return a.D == 128 ? launch_backward_stage0_t<bf16, 128>(a, s) : launch_backward_stage0_t<bf16, 64>(a, s);
  return a.D == 128 ? launch_backward_stage0_t<float, 128>(a, s) : launch_backward_stage0_t<float, 64>(a, s);
}

}  // namespace dash
