// Internal declarations shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dash {

// Tiled layout of the split summaries: tiles of 16 chunks per (b, kv head); in a tile, for
// plane p (0 hi, 1 lo), 32-element slice ks and chunk r, 32 consecutive bf16.
__host__ __device__ inline int split_tiles(int nc) { return (nc + 15) / 16; }
__host__ __device__ inline size_t split_bk_stride(int nc, int D) {
  return (size_t)split_tiles(nc) * 16 * 2 * D;
}
__host__ __device__ inline int split_offset(int c, int p, int e, int D) {
  return (c >> 4) * 32 * D + ((p * (D / 32) + (e >> 5)) * 16 + (c & 15)) * 32 + (e & 31);
}

constexpr int kChunk = 64;          // tokens per chunk (the pages' only chunk size)
constexpr int kMaxRouted = 2048;    // routed chunks per row held in registers (32 per lane)
constexpr int kMaxRoutedRegs = kMaxRouted / 64;
constexpr int kMaxRoutedWords = kMaxRouted / 64;   // mask words that can hold routed chunks

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ device helpers
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Whole-wave reductions without LDS round trips: DPP butterflies inside each 16-lane row
// (quad permutes, then the half-row and row mirrors), then the gfx950 row-swap moves across
// rows.  Every step combines a lane's value with its partner's and the partner does the
// same with the operands swapped, so all 64 lanes end with bit-identical results.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, dpp_f32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = op(v, dpp_f32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = op(v, dpp_f32<0x141>(v));   // row_half_mirror
  v = op(v, dpp_f32<0x140>(v));   // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ float wave_min(float v) {
  return wave_reduce(v, [](float x, float y) { return fminf(x, y); });
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float x, float y) { return x + y; });
}

// ------------------------------------------------------------------ launch-side API
// Every launcher enqueues on `stream` and returns hipGetLastError().

struct RouteArgs {
  const void* q;          // [B, Hq, Tq, D]
  const float* summ;      // [B, Hkv, nc_alloc, D]
  uint64_t* mask;         // [B, Hkv, rows, W]
  float* wbar;            // [B, Hkv, rows, wbar_ld] (written at set bits)
  const int32_t* seq_lens;  // decode: query row = seq_lens[b] - 1; prefill: nullptr
  int B, Hq, Hkv, D, Tq, rows, nc_alloc, W, wbar_ld;
  int tcap;               // prefill: T; decode: cache capacity (a query row must be < tcap)
  float alpha, zscale;    // zscale = (alpha - 1) * gamma * sm_scale
  int topk;               // > 0: top-k comparison router instead of entmax (MFMA prefill)
  int dtype;
  int32_t* list;          // decode: [B * Hkv][list_ld]: count, then the active chunks in
  int list_ld;            // increasing order followed by the diagonal chunk (or nullptr)
  float* sco;             // decode: [B * Hkv][G][sco_ld] scaled scores (or nullptr)
  int sco_ld;
  const void* kdiag;      // estimate_diagonal (generic router): keys [B, Hkv, kdiag_ld, D]
  const void* head_cls;   // and head_cls [Hkv, D] for the own chunk's summary, or nullptr
  int kdiag_ld;
  float s0_scale_log2;    // Stage 0 logit scale * log2(e)
  const float* ydiag;     // estimate_diagonal (MFMA router): [B, Hq, Tq] scaled score of each
                          // row's own chunk (k_diag_scores), or nullptr
  const int32_t* kdiag_bt;  // estimate_diagonal, paged decode: block table [B][kdiag_bt_ld] of
  int kdiag_bt_ld;          // kdiag's page pool [num_pages][Hkv][64][D] (nullptr: contiguous)
  int kdiag_pages;
  float* tau_out;         // prefill, entmax (nullable): each head's threshold tau and
  float* z_out;           // normaliser z = sum [y - tau]_+^(1/(alpha-1)), [B, Hq, Tq] each
};

struct AttendArgs {
  const void* q;          // [B, Hq, Tq, D]
  const void* k;          // [B, Hkv, Tk, D]
  const void* v;          // [B, Hkv, Tk, D]
  const void* vt;         // bf16 chunk-transposed V [B, Hkv, nc, D, 64] (MFMA path)
  const uint64_t* mask;   // [B, Hkv, rows, W]
  const float* wbar;      // [B, Hkv, rows, wbar_ld]
  void* out;              // [B, Hq, Tq, D]
  const int32_t* seq_lens;
  int B, Hq, Hkv, D, Tq, Tk, rows, W, wbar_ld, nc;
  float scale_log2;       // sm_scale * log2(e)
  float sigma;            // prior strength: a routed chunk's bias is sigma * log2 w_bar
  int dtype;
  int dense;              // 1: every chunk c < i_t active with prior 1 (comparator)
  const int32_t* block_table;  // decode, paged caches: [B][bt_ld] page of each chunk, or
  int bt_ld;                   // nullptr for contiguous [B, Hkv, Tk, D] caches; pages are
  int num_pages;               // [num_pages][Hkv][64][D] (ids outside [0, num_pages) read as 0)
  int32_t* seg_size;           // decode: the attend kernel's common segment size, for the combine
  const int32_t* list;    // decode: the route kernel's item lists (see RouteArgs)
  int list_ld;
  float* lse;             // prefill (nullable): [B, Hq, Tq] natural-log sum of exp of each
                          // row's biased logits
};

// Backward pass.  Inputs are the forward's tensors, dL/dout, the forward's log-sum-exp and the
// recomputed Stage 0 / Stage 1 state; fp32 accumulators live in the backward workspace.
struct BackwardArgs {
  const void* q;          // [B, Hq, T, D]   dtype
  const void* k;          // [B, Hkv, T, D]  dtype
  const void* v;          // [B, Hkv, T, D]  dtype
  const void* vt;         // bf16 chunk-transposed V [B, Hkv, nc, D, 64] (MFMA path)
  const void* head_cls;   // [Hkv, D]        dtype
  const void* out;        // [B, Hq, T, D]   dtype, the forward's output
  const void* dout;       // [B, Hq, T, D]   dtype, dL/dout
  const float* lse;       // [B, Hq, T] natural-log sum of exp of each row's biased logits
  const float* summ;      // [B, Hkv, nc, D] fp32 summaries
  const bf16* ssplit;     // bf16 hi/lo split summaries (MFMA path; see split_offset)
  const uint64_t* mask;   // [B, Hkv, T, W]
  const float* wbar;      // [B, Hkv, T, nc] (valid at set bits)
  const float* tau;       // [B, Hq, T] each head's entmax threshold
  const float* z;         // [B, Hq, T] and normaliser
  float* dq32;            // [B, Hq, T, D]  Stage 2's part of dq
  float* dk32;            // [B, Hkv, T, D] Stage 2's part of dk
  float* dv32;            // [B, Hkv, T, D]
  float* dwb;             // [B, Hkv, T, nc] dL/dw_bar (valid at set bits)
  float* dsumm;           // [B, Hkv, nc, D] dL/dk_bar
  float* dhc_part;        // [B, Hkv, nc, D] per-chunk parts of dL/dhead_cls
  void* dq;               // [B, Hq, T, D]   dtype (written)
  void* dk;               // [B, Hkv, T, D]  dtype (written)
  void* dv;               // [B, Hkv, T, D]  dtype (written)
  float* dhead_cls;       // [Hkv, D] fp32 (written)
  int B, Hq, Hkv, T, D, nc, W;
  float scale, gamma, alpha, sigma;
  int dtype;
};
// generic kernels (any dtype): Stage 2 and Stage 1 backwards, with fp32 atomics into dk32,
// dv32, dwb and dsumm (which must start at zero); dq written
hipError_t launch_backward_valu(const BackwardArgs& a, hipStream_t s);
// Stage 0 backwards and the head_cls reduction (after either path); dv converted from dv32
// unless dv32 is null
hipError_t launch_backward_stage0(const BackwardArgs& a, hipStream_t s);
// bf16 MFMA kernels for Stage 2 and Stage 1 backwards: dq written, dwb written at set bits,
// dk32, dv32 and dsumm added into (they must start at zero); scratch of
// backward_mfma_scratch() bytes
int backward_mfma_scratch(int B, int Hq, int Hkv, int T, int D, size_t* off_delta, size_t* off_ub,
                          size_t* off_kcm, size_t* off_rho, size_t* off_qsc, size_t* total);
hipError_t launch_backward_mfma(const BackwardArgs& a, void* scratch, hipStream_t s);

// summ_split (nullable, bf16 inputs only): bf16 hi and lo planes of the fp32 summaries
// (hi = bf16(x), lo = bf16(x - hi)) for the MFMA router, tiled for its operand loads: per
// (b, kv head) split_tiles(nc_alloc) tiles of 16 chunks, each [plane][D/32][16 chunks][32]
// (see split_offset), so one wave-wide 16-byte load reads 1 KiB of contiguous memory.
// block_table (nullable): paged K, [num_pages][Hkv][64][D], chunk c of sequence b in page
// block_table[b * bt_ld + c] (chunks whose page id is out of range are skipped).
// ydiag [B, Hq, T] for estimate_diagonal on the MFMA router (bf16 inputs)
hipError_t launch_diag_scores(const void* k, const void* head_cls, const void* q, float* ydiag,
                              int B, int Hq, int Hkv, int T, int D, int nc, float scale,
                              float zscale, hipStream_t s);
hipError_t launch_stage0(const void* k, const void* head_cls, float* summ, void* summ_split,
                         int B, int Hkv, int T_stride, int D, int nc_alloc, int n_full,
                         const int32_t* lo_b, const int32_t* seq_lens, float scale,
                         int dtype, hipStream_t s, const int32_t* block_table = nullptr,
                         int bt_ld = 0, int num_pages = 0);
hipError_t launch_update_nsum(int32_t* n_summarized, const int32_t* seq_lens, int B,
                              int T_stride, hipStream_t s);
hipError_t launch_vtranspose(const void* v, void* vt, int B, int Hkv, int T, int D, int nc,
                             hipStream_t s);
hipError_t launch_route_valu(const RouteArgs& a, hipStream_t s);
hipError_t launch_route_mfma(const RouteArgs& a, const void* summ_split, hipStream_t s);
hipError_t launch_attend_valu(const AttendArgs& a, hipStream_t s);
hipError_t launch_attend_mfma(const AttendArgs& a, hipStream_t s);

// decode (bf16): route one row per (b, kv head); split-K attend over the active chunks
// into per-segment partials pml [B*Hkv][nseg][32] (max, sum) and po [B*Hkv][nseg][16][D],
// then a log-sum-exp combine into a.out.
int decode_nseg_max(int nc);
hipError_t launch_decode_route(const RouteArgs& a, hipStream_t s);
hipError_t launch_decode_attend(const AttendArgs& a, float* pml, float* po, hipStream_t s);

}  // namespace dash
