// Stage 2 on bf16 MFMA (gfx950 v_mfma_f32_16x16x32_bf16): prior-induced sparse softmax
// attention over the active chunks of a bit-packed mask, flash-style online softmax.
//
// Method: gist.science summary of arXiv 2605.18753, "Stufe 2: Prior-induzierte spärliche
// Softmax" (softmax(z + log g), g = 0 where the routing weight is 0, FlashAttention-style
// kernel iterating over the active chunks of a bit-packed mask and adding the routing bias
// to the logits; the query's own chunk is a separate branch); aixai.ru blog,
// "Трёхстадийная архитектура" (the mask is walked in one pass, with no per-query index
// materialisation).  All G query heads of a KV head share the mask and the weights.
//
// Work unit: one workgroup per (b, kv head, R consecutive rows inside one 64-row block),
// i.e. R x G query vectors (256 for G >= 4), 32 per wave.  The workgroup visits the
// diagonal chunk, then the union of its rows' mask words in increasing chunk order (a visit
// list built in LDS); per routed visit, each row gets bias sigma log2(w_bar) where its own bit is
// set and -inf where it is not, so the union walk computes exactly the per-row result.
//
// MFMA mapping (16x16x32, wave64; lane l, k-slot (l/16, i)):
//   S^T = K Q^T  : A = K rows, B = Q^T.  The 16 rows of a key tile are permuted so that
//                  after two tiles ("halves") of a 32-key span, lane l holds the scores of
//                  keys 32p + 8(l/16) + [0, 8) for its query column l%16.
//   O^T += V^T P^T: B = P^T straight from those registers (k-slot i <-> key 8(l/16)+i),
//                  A = V^T rows read as one 16-byte LDS load from a chunk-transposed copy
//                  of V ([chunk][d][64 keys]) that Stage 0's companion kernel writes.
// Softmax runs in base 2: Q is multiplied once by the logit scale times log2 e (rounded to
// bf16, a relative change of at most 2^-9 per element).  The diagonal chunk, visited first,
// sets each query column's reference max m from its own keys; on every routed visit the QK
// accumulator starts at bias - m, so the MFMA returns the base-2 exponent itself, and the
// column sums of the bf16 probabilities come from one more MFMA with an all-ones operand.
// Visits go in rounds of two behind one workgroup barrier: the K/V tiles of a round's two
// chunks are loaded straight into two of four LDS slots (the pair the round before last
// used) during the previous round.
//
// LDS layout: rows are unpadded and the 16-byte chunks of a row are XOR-swizzled by row bits
// (kswz, vswz) so that every quarter wave of an operand read or a tile store touches 16
// distinct 16-byte slots modulo 256 bytes (and every half wave 32 distinct slots modulo 512
// bytes).  The hardware counter of LDS bank-conflict cycles reads about zero for this kernel;
// a layout that is conflict free only per half wave measures as conflicted for about a fifth
// of the kernel's cycles.
#include <type_traits>

#include "dash_internal.h"


namespace dash {

namespace {

constexpr float kNegBig = -1.0e30f;
constexpr int kXcds = 8;            // accelerator complex dies; workgroups are dealt round-robin
// A column's 64 unnormalised probabilities of a chunk may sum to at most 2^11 before its
// reference max is raised; a larger sum, an overflow or a NaN triggers the rescale.
constexpr float kColCap = 2048.0f;
// A operand of all ones: the MFMA then returns each column's sum of the B operand
__device__ const bf16x8 kOnes = {(bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f,
                                 (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f};
// dword 3 of a raw buffer descriptor on gfx9-family parts (32-bit data format, offsets in
// bytes, bounds checked against the record count)
constexpr int kBufferRsrcWord3 = 0x00020000;

__device__ __forceinline__ floatx4 mfma16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max over lanes l, l^16, l^32, l^48 with the gfx950 row-swap moves (no LDS round trip):
// permlane16_swap(v, v) gives each lane the values of rows {2i, 2i+1} of its row pair,
// permlane32_swap(v, v) those of the lower and the upper half-wave
__device__ __forceinline__ float rowgroup_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Swizzle of the 16-byte chunk index inside a K row (D/8 chunks per row).  The 16 keys of a
// quarter wave's operand read differ in bits 0, 1, 3 and 4: with D = 128 (16 chunks, 256-byte
// rows) the four bits give 16 distinct chunks; with D = 64 (128-byte rows) bit 0 picks the
// half of the 256-byte window and bits 1, 3, 4 give 8 distinct chunks.
template <int D>
__device__ __forceinline__ int kswz(int key) {
  if (D == 128) return (key & 3) | (((key >> 3) & 3) << 2);
  return ((key >> 1) & 1) | (((key >> 3) & 3) << 1);
}
// Swizzle of the 16-byte chunk index inside a V^T row (64 keys = 8 chunks = 128 bytes per
// row): a quarter wave reads 16 consecutive rows, bit 0 picks the half of the 256-byte
// window and bits 1, 2, 3 give 8 distinct chunks.
__device__ __forceinline__ int vswz(int d) { return ((d >> 1) & 1) | (((d >> 2) & 3) << 1); }

}  // namespace

template <int D, int NW, int QT, int RMAX, bool DENSE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(QT == 1 ? 4 : 2)))
void k_attend_mfma(AttendArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KS = D / 32;          // k-steps of the QK^T contraction
  constexpr int NDT = D / 16;         // 16-wide d tiles of the output
  constexpr int KP = D * 2;           // K row pitch in LDS (bytes), chunks swizzled
  constexpr int VP = 64 * 2;          // V^T row pitch in LDS (bytes), chunks swizzled
  constexpr int KBYTES = 64 * KP, VBYTES = D * VP;
  constexpr int KSEG = 64 * D / 8, VSEG = D * 8;       // 16-byte segments per tile
  // A chunk's K and V^T tiles go straight into LDS (buffer loads with an LDS destination): one
  // such load of a wave fills 1 KiB, lane i the 16 bytes at offset 16 i, so each lane fetches
  // the global 16 bytes that the swizzled layout puts there; NKI and NVI loads per wave cover
  // the two tiles.
  constexpr int NKI = KBYTES / 1024 / NW, NVI = VBYTES / 1024 / NW;
  static_assert(NKI * NW * 1024 == KBYTES && NVI * NW * 1024 == VBYTES,
                "tile loads must cover every wave evenly");
  constexpr int SLOT = KBYTES + VBYTES;           // K tile, then V^T tile
  constexpr int MAXW = (kMaxRouted + 1 + 63) / 64;

  // four tile slots as separate arrays, so that the compiler can tell the slots being filled
  // from the ones being read and waits for the loads only where a slot is taken up
  __shared__ __attribute__((aligned(16))) uint8_t ls0[SLOT];
  __shared__ __attribute__((aligned(16))) uint8_t ls1[SLOT];
  __shared__ __attribute__((aligned(16))) uint8_t ls2[SLOT];
  __shared__ __attribute__((aligned(16))) uint8_t ls3[SLOT];
  __shared__ uint64_t rowbits[RMAX][MAXW];
  __shared__ uint16_t visit[kMaxRouted + 2];
  __shared__ int woff[MAXW + 1];

  const int G = a.Hq / a.Hkv;
  const int R = NW * 16 * QT / G;            // rows per workgroup (<= 64, divides 64)
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  // Workgroup -> (64-row query block, b, kv head, row tile).  Consecutive workgroups are
  // dealt round-robin to the 8 XCDs; a group of 8 * RPB consecutive workgroups gives each
  // XCD the RPB row tiles of one query block, which share nearly the same mask and so read
  // the same K/V tiles through that XCD's L2.  Blocks go heavy (late rows) first.
  const int BH = a.B * a.Hkv;
  const int RPB = kChunk / R;                // row tiles per 64-row block
  const int nunits = ((a.Tq + kChunk - 1) / kChunk) * BH;
  const int grp = kXcds * RPB;
  const int xcd = (blockIdx.x % grp) % kXcds, sub = (blockIdx.x % grp) / kXcds;
  const int unit = (blockIdx.x / grp) * kXcds + xcd;
  if (unit >= nunits) return;                // padding of the last group (whole workgroup)
  const int uu = nunits - 1 - unit;
  const int bk = uu % BH;
  const int rt = (uu / BH) * RPB + sub;
  const int b = bk / a.Hkv, kvh = bk % a.Hkv;
  const int row0 = rt * R;
  const int it = row0 / kChunk;              // diagonal chunk, shared by all R rows
  const int T = a.Tq;

  // ---- per-row mask words and the union walk
  const int W = a.W;
  const int nw_route = (it + 63) / 64;       // words that can hold routed chunks
  if (!DENSE) {
    for (int idx = tid; idx < R * nw_route; idx += NT) {
      const int r = idx / nw_route, w = idx % nw_route;
      const int t = row0 + r;
      rowbits[r][w] = (t < T) ? a.mask[((size_t)bk * a.rows + t) * W + w] : 0ull;
    }
  }
  __syncthreads();
  if (tid < nw_route) {
    uint64_t u = 0;
    if (DENSE) {
      const int n = min(64, it - 64 * tid);
      u = n >= 64 ? ~0ull : ((1ull << n) - 1ull);
    } else {
      for (int r = 0; r < R; ++r) u |= rowbits[r][tid];
    }
    woff[tid + 1] = __popcll(u);
  }
  __syncthreads();
  if (tid == 0) {
    woff[0] = 0;
    for (int w = 0; w < nw_route; ++w) woff[w + 1] += woff[w];
  }
  __syncthreads();
  if (tid < nw_route) {
    uint64_t u = 0;
    if (DENSE) {
      const int n = min(64, it - 64 * tid);
      u = n >= 64 ? ~0ull : ((1ull << n) - 1ull);
    } else {
      for (int r = 0; r < R; ++r) u |= rowbits[r][tid];
    }
    int o = woff[tid] + 1;
    while (u) {
      visit[o++] = (uint16_t)(64 * tid + __builtin_ctzll(u));
      u &= u - 1;
    }
  }
  if (tid == 0) visit[0] = (uint16_t)it;
  __syncthreads();
  const int nvis = woff[nw_route] + 1;

  // ---- this lane's query columns (one per 16-column query tile of the wave)
  const int l16 = lane & 15, lg = lane >> 4;
  int qrow[QT], qh[QT];
  bool qok[QT];
  bf16x8 qop[QT][KS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int n = 16 * QT * wv + 16 * qt + l16;
    const int r = n / G, g = n % G;
    qrow[qt] = r;
    qh[qt] = kvh * G + g;
    const int t = row0 + r;
    qok[qt] = t < T;
    const bf16* qp = (const bf16*)a.q + ((size_t)(b * a.Hq + qh[qt]) * T + (qok[qt] ? t : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 32 * ks + 8 * lg);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (bf16)((float)v[e] * a.scale_log2);
      if (!qok[qt]) v = bf16x8{};
      qop[qt][ks] = v;
    }
  }

  // ---- global -> LDS prefetch of one chunk's K and V^T tiles through buffer descriptors
  // rebased per chunk (scalar arithmetic only; each lane's byte offsets are fixed).  A K
  // descriptor's range ends at the last key, so rows past the end of the sequence read as
  // zeros; they only occur in the diagonal chunk, where they are masked.
  const bf16* kbase = (const bf16*)a.k + (size_t)bk * a.Tk * D;
  const bf16* vtbase = (const bf16*)a.vt + (size_t)bk * a.nc * D * 64;
  int kdo[NKI], vdo[NVI];
#pragma unroll
  for (int j = 0; j < NKI; ++j) {
    const int byte = (wv * NKI + j) * 1024 + 16 * lane;
    const int row = byte / KP, ch = ((byte % KP) >> 4) ^ kswz<D>(row);
    kdo[j] = row * KP + ch * 16;
  }
#pragma unroll
  for (int j = 0; j < NVI; ++j) {
    const int byte = (wv * NVI + j) * 1024 + 16 * lane;
    const int row = byte / VP, ch = ((byte % VP) >> 4) ^ vswz(row);
    vdo[j] = row * VP + ch * 16;
  }
  typedef __attribute__((address_space(3))) void lds_void;
  auto slot = [&](auto slot_tag) -> uint8_t* {
    constexpr int S = decltype(slot_tag)::value;
    if constexpr (S == 0) return ls0; else if constexpr (S == 1) return ls1;
    else if constexpr (S == 2) return ls2; else return ls3;
  };
  auto prefetch = [&](int c_any, auto slot_tag) {
    const int c = __builtin_amdgcn_readfirstlane(c_any);
    const int keys_left = a.Tk - c * kChunk;            // > 0 for every visited chunk
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + (size_t)c * kChunk * D), (short)0, min(keys_left, kChunk) * D * 2,
        kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vtbase + (size_t)c * D * 64), (short)0, D * 64 * 2, kBufferRsrcWord3);
    uint8_t* base = slot(slot_tag);
#pragma unroll
    for (int j = 0; j < NKI; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(base + (wv * NKI + j) * 1024), 16, (unsigned)kdo[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NVI; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(base + KBYTES + (wv * NVI + j) * 1024), 16, (unsigned)vdo[j], 0, 0, 0);
  };
  // routing weight and mask bit of this lane's rows for routed chunk c, in set S (the first
  // or second visit of a round); the weight is loaded one round ahead and only turned into a
  // bias (log2 w, or -inf where the row's bit is clear) when the round starts, so no wait on
  // it stalls the tile prefetch
  float wnext[2][QT];
  bool onnext[2][QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    wnext[0][qt] = wnext[1][qt] = 1.f;
    onnext[0][qt] = onnext[1][qt] = true;
  }
  auto fetch_weight = [&](int c, auto set_tag) {
    constexpr int S = decltype(set_tag)::value;
    if (DENSE) return;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int r = qrow[qt];
      onnext[S][qt] = (rowbits[r][c >> 6] >> (c & 63)) & 1ull;
      const int t = min(row0 + r, a.rows - 1);
      wnext[S][qt] = a.wbar[((size_t)bk * a.rows + t) * a.wbar_ld + c];
    }
  };

  floatx4 o[QT][NDT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[qt][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  // m: the reference maximum of each query column (base-2 logits), only raised when a
  // chunk's probabilities relative to it grow too large, so most chunks skip the rescale
  // of O and l.
  float m[QT], lsum[QT];
  int tloc[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = kNegBig;
    lsum[qt] = 0.f;
    tloc[qt] = (row0 + qrow[qt]) & 63;
  }

  // the work of one visit on the tile in LDS slot buf; DIAG: the query block's own chunk
  // (always the first visit)
  auto visit_chunk = [&](const uint8_t* sl, const float (&bias)[QT], auto diag_tag) {
    constexpr bool DIAG = decltype(diag_tag)::value;
    asm volatile("" ::: "memory");      // keep each visit's LDS reads inside it
    // a wave none of whose rows has this routed chunk adds exactly nothing (p = 0, no
    // rescale): it only takes part in the tile loads and leaves its SIMD to the other wave
    if (!DIAG && !DENSE) {
      bool any = false;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) any = any || bias[qt] != -INFINITY;
      if (__builtin_amdgcn_ballot_w64(any) == 0ull) return;
    }
    const uint8_t* kl = sl;
    const uint8_t* vl = sl + KBYTES;

    // S^T for 64 keys: tile kt = 2 p + half
    floatx4 sc[QT][4];
    floatx4 seed[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float off = DIAG ? 0.f : bias[qt] - m[qt];
      seed[qt] = floatx4{off, off, off, off};
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int p = kt >> 1, half = kt & 1;
      const int key = 32 * p + 8 * (l16 >> 2) + 4 * half + (l16 & 3);
      const int ksw = kswz<D>(key);        // p and half do not change the swizzle
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 ka =
            *reinterpret_cast<const bf16x8*>(kl + key * KP + ((4 * ks + lg) ^ ksw) * 16);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          sc[qt][kt] = mfma16(ka, qop[qt][ks], ks == 0 ? seed[qt] : sc[qt][kt]);
      }
    }

    // online softmax per query column; build P^T operands.  On routed visits x is already
    // the exponent relative to the column's reference max m; the chunk's max is only taken
    // when a column's probability sum exceeds kColCap (or is not a number).
    float x[QT][16];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1) + j;
          x[qt][4 * kt + j] = (DIAG && key > tloc[qt]) ? -INFINITY : sc[qt][kt][j];
        }
    // bf16 probabilities 2^(x - sh) as the PV operand (half 0: keys 32p + 8 lg + j, half 1:
    // + 4), and their column sums from the matrix cores (all-ones A operand)
    bf16x8 pop[QT][2];
    floatx4 csum[QT];
    auto probs = [&](int qt, float sh) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        bf16x8 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] = (bf16)fast_exp2(x[qt][8 * p + j] - sh);
          v[4 + j] = (bf16)fast_exp2(x[qt][8 * p + 4 + j] - sh);
        }
        pop[qt][p] = v;
      }
      csum[qt] = mfma16(kOnes, pop[qt][0], floatx4{0.f, 0.f, 0.f, 0.f});
      csum[qt] = mfma16(kOnes, pop[qt][1], csum[qt]);
    };
    auto colmax = [&](int qt) {
      float mr = fmaxf(fmaxf(x[qt][0], x[qt][1]), x[qt][2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) mr = fmaxf(fmaxf(mr, x[qt][i]), x[qt][i + 1]);
      return rowgroup_max(fmaxf(mr, x[qt][15]));
    };
    if (DIAG) {
      // first visit: the reference max is this chunk's max logit (the query's own key is
      // always present), so every later offset bias - m is of moderate size
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        m[qt] = colmax(qt);
        probs(qt, m[qt]);
      }
    } else {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) probs(qt, 0.f);
      bool over = false;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) over = over || !(csum[qt][0] <= kColCap);
      if (__builtin_amdgcn_ballot_w64(over) != 0ull) {
        // raise the reference max by this chunk's largest offset logit, rescale O and l
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const float mr = fmaxf(colmax(qt), 0.f);
          const float corr = fast_exp2(-mr);
          m[qt] += mr;
          lsum[qt] *= corr;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[qt][dt] *= corr;
          probs(qt, mr);
        }
      }
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) lsum[qt] += csum[qt][0];

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(
            vl + (16 * dt + l16) * VP + ((4 * p + lg) ^ vswz(l16)) * 16);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) o[qt][dt] = mfma16(va, pop[qt][p], o[qt][dt]);
      }
    }
  };

  // rounds of two visits behind one barrier: visits 2r and 2r + 1 use the LDS slots of pair
  // r & 1 (slots 0, 1 or 2, 3), whose loads went out during round r - 1 into the pair that
  // round r - 2 used; every wave finished that round before the barrier of round r - 1.
  // Visit 0 is the diagonal chunk.  The rounds are unrolled by pair so that each one's slots
  // are known at compile time.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  prefetch(visit[0], S0{});
  if (1 < nvis) {
    prefetch(visit[1], S1{});
    fetch_weight(visit[1], S1{});
  }
  auto round = [&](int r, auto first_tag, auto pair_tag) {
    constexpr bool FIRST = decltype(first_tag)::value;   // round 0: visit 0 is the diagonal
    constexpr int P = decltype(pair_tag)::value;
    using A0 = std::integral_constant<int, 2 * P>;
    using A1 = std::integral_constant<int, 2 * P + 1>;
    using N0 = std::integral_constant<int, 2 - 2 * P>;
    using N1 = std::integral_constant<int, 3 - 2 * P>;
    const int v0 = 2 * r, v1 = 2 * r + 1;
    const bool has1 = v1 < nvis;
    float bias[2][QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      bias[0][qt] = (FIRST || DENSE) ? 0.f : (onnext[0][qt] ? a.sigma * fast_log2(wnext[0][qt]) : -INFINITY);
      bias[1][qt] = DENSE ? 0.f : (onnext[1][qt] ? a.sigma * fast_log2(wnext[1][qt]) : -INFINITY);
    }
    // this round's tiles and weights are the only loads in flight: wait for them (vmcnt(0),
    // gfx9 encoding), then meet, so every wave's share of the tiles is in LDS
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    __syncthreads();
    if (v0 + 2 < nvis) {
      prefetch(visit[v0 + 2], N0{});
      fetch_weight(visit[v0 + 2], S0{});
    }
    if (v1 + 2 < nvis) {
      prefetch(visit[v1 + 2], N1{});
      fetch_weight(visit[v1 + 2], S1{});
    }
    if (FIRST) visit_chunk(slot(A0{}), bias[0], std::true_type{});
    else visit_chunk(slot(A0{}), bias[0], std::false_type{});
    if (has1) visit_chunk(slot(A1{}), bias[1], std::false_type{});
  };
  round(0, std::true_type{}, std::integral_constant<int, 0>{});
  for (int r = 1; 2 * r < nvis; r += 2) {
    round(r, std::false_type{}, std::integral_constant<int, 1>{});
    if (2 * (r + 1) < nvis) round(r + 1, std::false_type{}, std::integral_constant<int, 0>{});
  }

  // ---- normalise and write
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float l = lsum[qt];               // full column sum (every lane of the column)
    const float rl = 1.0f / l;
    if (!qok[qt]) continue;
    if (a.lse != nullptr && lg == 0)
      a.lse[(size_t)(b * a.Hq + qh[qt]) * T + row0 + qrow[qt]] =
          (m[qt] + fast_log2(l)) * 0.69314718055994531f;
    bf16* op = (bf16*)a.out + ((size_t)(b * a.Hq + qh[qt]) * T + row0 + qrow[qt]) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (bf16)(o[qt][dt][j] * rl);
      *reinterpret_cast<bf16x4*>(op + 16 * dt + 4 * lg) = v;
    }
  }
}

// Shape: two 16-column query tiles per wave and up to eight waves (two per SIMD, one
// workgroup per CU), keeping a workgroup inside one 64-row block.  The two tiles share
// every K and V^T operand read from LDS.  (One tile per wave at four waves per SIMD, the
// same 256 query vectors per workgroup, was measured slower on the 128K workload: twice
// the LDS operand traffic per MFMA outweighs the higher occupancy.)
template <int D, bool DENSE>
static hipError_t launch_attend_mfma_t(const AttendArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int NW = G >= 4 ? 8 : 2 * G;
  const int R = NW * 32 / G;
  const int nunits = ((a.Tq + kChunk - 1) / kChunk) * a.B * a.Hkv;
  dim3 grid(((nunits + kXcds - 1) / kXcds) * kXcds * (kChunk / R));
  switch (NW) {
    case 8: k_attend_mfma<D, 8, 2, 64, DENSE><<<grid, 512, 0, s>>>(a); break;
    case 4: k_attend_mfma<D, 4, 2, 64, DENSE><<<grid, 256, 0, s>>>(a); break;
    default: k_attend_mfma<D, 2, 2, 64, DENSE><<<grid, 128, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t launch_attend_mfma(const AttendArgs& a, hipStream_t s) {
  if (a.dense)
    return a.D == 128 ? launch_attend_mfma_t<128, true>(a, s) : launch_attend_mfma_t<64, true>(a, s);
  return a.D == 128 ? launch_attend_mfma_t<128, false>(a, s) : launch_attend_mfma_t<64, false>(a, s);
}

}  // namespace dash
