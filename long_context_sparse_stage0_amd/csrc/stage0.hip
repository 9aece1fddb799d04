// Stage 0: chunk summaries, and the chunk-transposed copy of V used by the MFMA Stage 2.
//
// Method (gist.science summary of arXiv 2605.18753, "Stufe 0: Lokale
// Chunk-Zusammenfassung"; aixai.ru blog, "Трёхстадийная архитектура"): a learned query
// attends by scaled dot-product attention over the 64 keys of a chunk; the attention-
// weighted key is the chunk's summary.  Once a chunk is complete its summary is frozen.
//
// Kernel shape: one 64-lane wave per (b, kv head, chunk).  A chunk of K is one
// contiguous 64 x D block (16 KiB at D = 128 bf16), read with 16-byte loads: a key row
// spans D / EPS lanes (EPS elements of 16 bytes each), so one wave-wide load covers
// 64 EPS / D consecutive rows and every lane issues 16-byte requests.  Logits are summed
// across the lanes of a row by xor butterflies, the softmax and the weighted sum across
// the row groups, all in registers in fp32.  HBM-bound: K is read once, fp32 summaries
// are written once.
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
  constexpr int EPS = 16 / (int)sizeof(TIn);     // elements per 16-byte load
  constexpr int LPR = D / EPS;                    // lanes per key row
  constexpr int RPI = 64 / LPR;                   // key rows per wave-wide load
  constexpr int NI = kChunk / RPI;                // loads per lane per chunk
  static_assert(LPR <= 64 && 64 % LPR == 0, "a key row must split evenly over the lanes");
  typedef TIn vec_t __attribute__((ext_vector_type(EPS)));
  const int lane = threadIdx.x;
  const int cg = lane % LPR, rg = lane / LPR;     // column group, row group
  const int kvh = blockIdx.y, b = blockIdx.z;
  int lo = 0, hi = n_full;
  if (seq_lens != nullptr) {
    int sl = seq_lens[b];
    sl = sl < 0 ? 0 : (sl > T_stride ? T_stride : sl);
    hi = sl / kChunk;
    lo = lo_b ? lo_b[b] : 0;
    if (lo < 0) lo = 0;
  }
  float h[EPS];
#pragma unroll
  for (int e = 0; e < EPS; ++e) h[e] = to_f32(head_cls[kvh * D + cg * EPS + e]) * scale_log2;

  for (int c = lo + blockIdx.x; c < hi; c += gridDim.x) {
    const TIn* kc;
    if (block_table) {                       // paged: chunk c of sequence b lives in a page
      const int pg = block_table[(size_t)b * bt_ld + c];
      if (pg < 0 || pg >= num_pages) continue;   // (uniform over the wave)
      kc = k + ((size_t)pg * Hkv + kvh) * kChunk * D;
    } else {
      kc = k + ((size_t)(b * Hkv + kvh) * T_stride + (size_t)c * kChunk) * D;
    }
    // lane (rg, cg) holds columns [cg EPS, + EPS) of rows i RPI + rg, one 16-byte load each
    // (rows stay packed in the input type until they are used: half the registers for bf16)
    vec_t kr[NI];
    float lgt[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i)
      kr[i] = *reinterpret_cast<const vec_t*>(kc + (size_t)(i * RPI + rg) * D + cg * EPS);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < EPS; ++e) part = fmaf(h[e], to_f32(kr[i][e]), part);
      lgt[i] = part;
    }
    // logits: sums over the LPR lanes of a row (xor butterflies stay inside the row group)
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1) lgt[i] += __shfl_xor(lgt[i], o, 64);
    // softmax over the 64 keys: each lane holds rows i RPI + rg; combine the row groups
    float mx = lgt[0];
#pragma unroll
    for (int i = 1; i < NI; ++i) mx = fmaxf(mx, lgt[i]);
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      lgt[i] = fast_exp2(lgt[i] - mx);
      sum += lgt[i];
    }
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) sum += __shfl_xor(sum, o, 64);
    const float rs = 1.0f / sum;
    float acc[EPS];
#pragma unroll
    for (int e = 0; e < EPS; ++e) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) a = fmaf(lgt[i], to_f32(kr[i][e]), a);
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) a += __shfl_xor(a, o, 64);
      acc[e] = a * rs;
    }
    if (rg == 0) {
      float* o = summ + ((size_t)(b * Hkv + kvh) * nc_alloc + c) * D + cg * EPS;
#pragma unroll
      for (int e = 0; e < EPS; ++e) o[e] = acc[e];
      if (ssplit != nullptr) {
        bf16* sp = ssplit + (size_t)(b * Hkv + kvh) * split_bk_stride(nc_alloc, D);
#pragma unroll
        for (int e = 0; e < EPS; ++e) {
          const bf16 hv = (bf16)acc[e];
          sp[split_offset(c, 0, cg * EPS + e, D)] = hv;
          sp[split_offset(c, 1, cg * EPS + e, D)] = (bf16)(acc[e] - (float)hv);
        }
      }
    }
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
