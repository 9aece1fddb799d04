// Stage 2, generic kernel (any dtype): prior-induced sparse softmax attention, one wave
// per (b, query head, query row); used for fp32 inputs and for single-row decode.
//
// Method: gist.science summary of arXiv 2605.18753, "Stufe 2: Prior-induzierte spärliche
// Softmax" -- softmax with the uniform reference replaced by a prior g derived from the
// routing weights (g = 0 where w = 0), i.e. softmax(z + log g), run by a FlashAttention-
// style kernel that iterates over the active chunks of a bit-packed mask and adds the
// routing bias to the logits; the query's own chunk is a separate branch.
//
// Lane j of the wave owns key j of the current 64-key chunk for the logit and owns
// columns [l*E, l*E + E) of the output accumulator; the online-softmax state (running
// max and sum, base-2 logits) is wave-uniform.  The walk visits the set bits of the row's
// mask words in increasing chunk order, then the diagonal chunk.
#include "dash_internal.h"

namespace dash {

template <typename TIn, int D>
__global__ __launch_bounds__(64) void k_attend_valu(AttendArgs a) {
  constexpr int E = D / 64;
  __shared__ float qs[D];
  __shared__ float ps[64];
  const int lane = threadIdx.x;
  const int row = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.Hkv, kvh = h / G;
  int t = row;
  bool valid = true;
  if (a.seq_lens) {
    t = a.seq_lens[b] - 1;
    valid = (t >= 0) && (t < a.Tk);
  }
  const int tq = a.seq_lens ? 0 : t;
  TIn* op = (TIn*)a.out + ((size_t)(b * a.Hq + h) * a.Tq + tq) * D;
  if (!valid) {
#pragma unroll
    for (int e = 0; e < E; ++e) op[lane * E + e] = from_f32<TIn>(__builtin_nanf(""));
    return;
  }
  const TIn* qp = (const TIn*)a.q + ((size_t)(b * a.Hq + h) * a.Tq + tq) * D;
  for (int d = lane; d < D; d += 64) qs[d] = to_f32(qp[d]) * a.scale_log2;
  __syncthreads();
  const int it = t / kChunk;
  const size_t kvbase = (size_t)(b * a.Hkv + kvh) * a.Tk;
  const TIn* kb = (const TIn*)a.k + kvbase * D;
  const TIn* vb = (const TIn*)a.v + kvbase * D;
  const size_t rowi = (size_t)(b * a.Hkv + kvh) * a.rows + (a.seq_lens ? 0 : t);

  float m = -INFINITY, l = 0.f, o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;

  auto visit = [&](int c, float bias) {
    const int j = c * kChunk + lane;
    float logit = -INFINITY;
    if (j <= t) {
      const TIn* kr = kb + (size_t)j * D;
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = fmaf(qs[d], to_f32(kr[d]), acc);
      logit = acc + bias;
    }
    const float mn = fmaxf(m, wave_max(logit));
    const float corr = fast_exp2(m - mn);
    const float p = fast_exp2(logit - mn);
    l = l * corr + wave_sum(p);
    m = mn;
    ps[lane] = p;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= corr;
    const int jn = min(kChunk, t + 1 - c * kChunk);
    for (int jj = 0; jj < jn; ++jj) {
      const float pj = ps[jj];
      const TIn* vr = vb + (size_t)(c * kChunk + jj) * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = fmaf(pj, to_f32(vr[e]), o[e]);
    }
    __syncthreads();
  };

  for (int w = 0; w * 64 < it; ++w) {
    uint64_t bits;
    if (a.dense) {
      const int n = min(64, it - 64 * w);
      bits = n == 64 ? ~0ull : ((1ull << n) - 1ull);
    } else {
      bits = a.mask[rowi * a.W + w];
    }
    while (bits) {
      const int c = 64 * w + __builtin_ctzll(bits);
      bits &= bits - 1;
      const float bias = a.dense ? 0.f : a.sigma * fast_log2(a.wbar[rowi * a.wbar_ld + c]);
      visit(c, bias);
    }
  }
  visit(it, 0.f);
  const float rl = 1.0f / l;
#pragma unroll
  for (int e = 0; e < E; ++e) op[lane * E + e] = from_f32<TIn>(o[e] * rl);
  if (a.lse != nullptr && lane == 0 && a.seq_lens == nullptr)
    a.lse[(size_t)(b * a.Hq + h) * a.Tq + t] = (m + fast_log2(l)) * 0.69314718055994531f;
}

hipError_t launch_attend_valu(const AttendArgs& a, hipStream_t s) {
  dim3 grid(a.rows, a.Hq, a.B);
  if (a.dtype == 0) {
    if (a.D == 128) k_attend_valu<bf16, 128><<<grid, 64, 0, s>>>(a);
    else k_attend_valu<bf16, 64><<<grid, 64, 0, s>>>(a);
  } else {
    if (a.D == 128) k_attend_valu<float, 128><<<grid, 64, 0, s>>>(a);
    else k_attend_valu<float, 64><<<grid, 64, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace dash
