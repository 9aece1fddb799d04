// Stage 0: chunk summaries, and the chunk-transposed copy of V used by the MFMA Stage 2.
//
// Method (gist.science summary of arXiv 2605.18753, "Stufe 0: Lokale
// Chunk-Zusammenfassung"; aixai.ru blog, "Трёхстадийная архитектура"): a learned query
// attends by scaled dot-product attention over the 64 keys of a chunk; the attention-
// weighted key is the chunk's summary.  Once a chunk is complete its summary is frozen.
//
// Kernel shape: one 64-lane wave per (b, kv head, chunk).  A chunk of K is one
// contiguous 64 x D block (16 KiB at D = 128 bf16), read row by row so that each row is
// one fully coalesced 256-byte wave load; lane l owns columns [l*E, l*E + E), E = D/64.
// The 64 partial dot products of a lane are reduced across lanes through a padded LDS
// tile (lane j ends up with logit a_j), softmax runs across lanes, and the weighted sum
// of the rows (still in registers) is accumulated per lane in fp32.  HBM-bound: K is
// read once, fp32 summaries are written once.
#include "dash_internal.h"

namespace dash {

template <typename TIn, int D>
__global__ __launch_bounds__(64) void k_stage0(const TIn* __restrict__ k,
                                               const TIn* __restrict__ head_cls,
                                               float* __restrict__ summ,
                                               bf16* __restrict__ ssplit, int Hkv,
                                               int T_stride, int nc_alloc, int n_full,
                                               const int32_t* __restrict__ lo_b,
                                               const int32_t* __restrict__ seq_lens,
                                               float scale_log2,
                                               const int32_t* __restrict__ block_table,
                                               int bt_ld, int num_pages) {
  constexpr int E = D / 64;
  __shared__ float red[64][65];
  __shared__ float pis[64];
  const int lane = threadIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z;
  int lo = 0, hi = n_full;
  if (seq_lens != nullptr) {
    int sl = seq_lens[b];
    sl = sl < 0 ? 0 : (sl > T_stride ? T_stride : sl);
    hi = sl / kChunk;
    lo = lo_b ? lo_b[b] : 0;
    if (lo < 0) lo = 0;
  }
  float h[E];
#pragma unroll
  for (int e = 0; e < E; ++e) h[e] = to_f32(head_cls[kvh * D + lane * E + e]) * scale_log2;

  for (int c = lo + blockIdx.x; c < hi; c += gridDim.x) {
    const TIn* kc;
    if (block_table) {                       // paged: chunk c of sequence b lives in a page
      const int pg = block_table[(size_t)b * bt_ld + c];
      if (pg < 0 || pg >= num_pages) continue;   // (uniform over the wave)
      kc = k + ((size_t)pg * Hkv + kvh) * kChunk * D;
    } else {
      kc = k + ((size_t)(b * Hkv + kvh) * T_stride + (size_t)c * kChunk) * D;
    }
    float kr[64][E];
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        kr[j][e] = to_f32(kc[j * D + lane * E + e]);
        part += h[e] * kr[j][e];
      }
      red[j][lane] = part;
    }
    __syncthreads();
    float a = 0.f;  // logit of key `lane`, in log2 units
    for (int i = 0; i < 64; ++i) a += red[lane][i];
    const float m = wave_max(a);
    const float p = fast_exp2(a - m);
    const float s = wave_sum(p);
    pis[lane] = p / s;
    __syncthreads();
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const float pj = pis[j];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += pj * kr[j][e];
    }
    float* o = summ + ((size_t)(b * Hkv + kvh) * nc_alloc + c) * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = acc[e];
    if (ssplit != nullptr) {
      bf16* sp = ssplit + (size_t)(b * Hkv + kvh) * split_bk_stride(nc_alloc, D);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bf16 hi = (bf16)acc[e];
        sp[split_offset(c, 0, lane * E + e, D)] = hi;
        sp[split_offset(c, 1, lane * E + e, D)] = (bf16)(acc[e] - (float)hi);
      }
    }
    __syncthreads();
  }
}

// n_summarized[b] = max(n_summarized[b], complete chunks of the cache), with the length
// clamped to [0, T_stride] as k_stage0 clamps it, so the count never passes the chunks that
// were actually summarised
__global__ void k_update_nsum(int32_t* n_summarized, const int32_t* seq_lens, int B,
                              int T_stride) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) {
    int sl = seq_lens[b];
    sl = sl < 0 ? 0 : (sl > T_stride ? T_stride : sl);
    const int n = sl / kChunk;
    if (n > n_summarized[b]) n_summarized[b] = n;
  }
}

// V [B, Hkv, T, D] -> vt [B, Hkv, nc, D, 64]: each chunk becomes a D x 64 tile whose rows
// are 64 consecutive keys of one column; rows of a partial last chunk are zero-filled.
template <int D>
__global__ __launch_bounds__(256) void k_vtranspose(const uint16_t* __restrict__ v,
                                                    uint16_t* __restrict__ vt, int Hkv, int T,
                                                    int nc) {
  __shared__ uint16_t tile[64][D + 2];
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const uint16_t* src = v + ((size_t)(b * Hkv + kvh) * T + (size_t)c * kChunk) * D;
  constexpr int SEGS = 64 * D / 8;
  for (int seg = tid; seg < SEGS; seg += 256) {
    const int row = seg / (D / 8), col = (seg % (D / 8)) * 8;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (c * kChunk + row < T) val = *reinterpret_cast<const uint4*>(src + row * D + col);
    const uint16_t* pv = reinterpret_cast<const uint16_t*>(&val);
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[row][col + i] = pv[i];
  }
  __syncthreads();
  uint16_t* dst = vt + ((size_t)(b * Hkv + kvh) * nc + c) * (size_t)D * 64;
  for (int seg = tid; seg < D * 8; seg += 256) {
    const int d = seg / 8, j0 = (seg % 8) * 8;
    uint4 val;
    uint16_t* pv = reinterpret_cast<uint16_t*>(&val);
#pragma unroll
    for (int i = 0; i < 8; ++i) pv[i] = tile[j0 + i][d];
    *reinterpret_cast<uint4*>(dst + d * 64 + j0) = val;
  }
}

// estimate_diagonal on the MFMA router: the Stage 1 score of each row's own chunk,
// ydiag[b, h, t] = zscale <q_{h,t}, kbar_t>, where kbar_t is Stage 0's summary of the keys
// i_t C .. t (the chunk's keys seen so far).  One 256-thread workgroup per (b, kv head,
// chunk): the chunk's keys go to LDS in fp32 and wave 0 scores them against head_cls; thread
// (r, dq) = (tid / 4, tid % 4) then forms row r's prefix-softmax weights, accumulates its
// quarter of kbar_r in registers (column pairs 2 dq + 8 p, so the four threads of a row hit
// distinct LDS banks and read each query row contiguously together) and the G dot products
// are reduced over those four threads.
template <int D>
__global__ __launch_bounds__(256) void k_diag_scores(const bf16* __restrict__ k,
                                                     const bf16* __restrict__ head_cls,
                                                     const bf16* __restrict__ q,
                                                     float* __restrict__ ydiag, int Hq, int Hkv,
                                                     int T, float scale_log2, float zscale) {
  constexpr int NP = D / 8;                  // column pairs per thread
  __shared__ float kl[64][D + 1];
  __shared__ float al[64];
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int G = Hq / Hkv;
  const int t0 = c * kChunk;
  const int nrow = min(kChunk, T - t0);
  const bf16* kc = k + ((size_t)(b * Hkv + kvh) * T + t0) * D;
  for (int i = tid; i < 64 * D; i += 256) {
    const int j = i / D, d = i % D;
    kl[j][d] = j < nrow ? (float)kc[(size_t)j * D + d] : 0.f;
  }
  __syncthreads();
  if (tid < 64) {
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc = fmaf((float)head_cls[kvh * D + d], kl[tid][d], acc);
    al[tid] = acc * scale_log2;
  }
  __syncthreads();
  const int r = tid >> 2, dq = tid & 3;
  if (r >= nrow) return;                     // the four threads of a row leave together
  float m = -INFINITY;
  for (int j = 0; j <= r; ++j) m = fmaxf(m, al[j]);
  float acc[NP][2];
#pragma unroll
  for (int p = 0; p < NP; ++p) acc[p][0] = acc[p][1] = 0.f;
  float sum = 0.f;
  for (int j = 0; j <= r; ++j) {
    const float w = fast_exp2(al[j] - m);
    sum += w;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      acc[p][0] = fmaf(w, kl[j][2 * dq + 8 * p], acc[p][0]);
      acc[p][1] = fmaf(w, kl[j][2 * dq + 8 * p + 1], acc[p][1]);
    }
  }
  const float rs = zscale / sum;
  const int t = t0 + r;
  for (int g = 0; g < G; ++g) {
    const size_t qi = (size_t)(b * Hq + kvh * G + g) * T + t;
    const bf16* qp = q + qi * D + 2 * dq;
    float s = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      s = fmaf((float)qp[8 * p], acc[p][0], s);
      s = fmaf((float)qp[8 * p + 1], acc[p][1], s);
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (dq == 0) ydiag[qi] = s * rs;
  }
}

hipError_t launch_diag_scores(const void* k, const void* head_cls, const void* q, float* ydiag,
                              int B, int Hq, int Hkv, int T, int D, int nc, float scale,
                              float zscale, hipStream_t s) {
  dim3 grid(nc, Hkv, B);
  const float sl2 = scale * 1.4426950408889634f;
  if (D == 128)
    k_diag_scores<128><<<grid, 256, 0, s>>>((const bf16*)k, (const bf16*)head_cls, (const bf16*)q,
                                            ydiag, Hq, Hkv, T, sl2, zscale);
  else
    k_diag_scores<64><<<grid, 256, 0, s>>>((const bf16*)k, (const bf16*)head_cls, (const bf16*)q,
                                           ydiag, Hq, Hkv, T, sl2, zscale);
  return hipGetLastError();
}

hipError_t launch_stage0(const void* k, const void* head_cls, float* summ, void* summ_split,
                         int B, int Hkv, int T_stride, int D, int nc_alloc, int n_full,
                         const int32_t* lo_b, const int32_t* seq_lens, float scale,
                         int dtype, hipStream_t s, const int32_t* block_table, int bt_ld,
                         int num_pages) {
  bf16* ss = (bf16*)summ_split;
  const float sl2 = scale * 1.4426950408889634f;
  int gx = seq_lens ? 64 : n_full;
  if (gx < 1) gx = 1;
  dim3 grid(gx, Hkv, B);
  if (dtype == 0) {
    if (D == 128)
      k_stage0<bf16, 128><<<grid, 64, 0, s>>>((const bf16*)k, (const bf16*)head_cls, summ, ss, Hkv,
                                              T_stride, nc_alloc, n_full, lo_b, seq_lens, sl2,
                                              block_table, bt_ld, num_pages);
    else
      k_stage0<bf16, 64><<<grid, 64, 0, s>>>((const bf16*)k, (const bf16*)head_cls, summ, ss, Hkv,
                                             T_stride, nc_alloc, n_full, lo_b, seq_lens, sl2,
                                             block_table, bt_ld, num_pages);
  } else {
    if (D == 128)
      k_stage0<float, 128><<<grid, 64, 0, s>>>((const float*)k, (const float*)head_cls, summ,
                                               nullptr, Hkv, T_stride, nc_alloc, n_full, lo_b, seq_lens,
                                               sl2, nullptr, 0, 0);
    else
      k_stage0<float, 64><<<grid, 64, 0, s>>>((const float*)k, (const float*)head_cls, summ,
                                              nullptr, Hkv, T_stride, nc_alloc, n_full, lo_b, seq_lens,
                                              sl2, nullptr, 0, 0);
  }
  return hipGetLastError();
}

hipError_t launch_update_nsum(int32_t* n_summarized, const int32_t* seq_lens, int B,
                              int T_stride, hipStream_t s) {
  k_update_nsum<<<(B + 63) / 64, 64, 0, s>>>(n_summarized, seq_lens, B, T_stride);
  return hipGetLastError();
}

hipError_t launch_vtranspose(const void* v, void* vt, int B, int Hkv, int T, int D, int nc,
                             hipStream_t s) {
  dim3 grid(nc, Hkv, B);
  if (D == 128)
    k_vtranspose<128><<<grid, 256, 0, s>>>((const uint16_t*)v, (uint16_t*)vt, Hkv, T, nc);
  else
    k_vtranspose<64><<<grid, 256, 0, s>>>((const uint16_t*)v, (uint16_t*)vt, Hkv, T, nc);
  return hipGetLastError();
}

}  // namespace dash
