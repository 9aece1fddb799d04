// Incremental decoding: one new query row per sequence against the K/V cache and the
// chunk-summary cache (arXiv 2605.18753 as summarised on gist.science: "Stufe 0" -- a
// complete chunk's summary is frozen and cached; the kernels support incremental decoding
// with a chunk-representation cache, "Hauptbeiträge").  Decode row t equals prefill row t.
//
// Four kernels per step, all on the caller's stream:
//   k_decode_scores  the G heads' scores against every routed summary on MFMA (fp32
//                    summaries split into bf16 hi + lo in registers), one 16-chunk tile per
//                    wave over many workgroups, so the summary reads are spread over the
//                    whole GPU rather than one CU per (b, kv head).
//   k_decode_route   one 16-wave workgroup per (b, kv head): wave g solves head g's entmax
//                    threshold with wave-only reductions (or, for the top-k comparison
//                    router, wave 0 selects on the heads' summed scores); then a fixed-order sum over the
//                    heads, a ballot per 64 chunks for the mask word, w_bar at set bits and
//                    the attend kernel's work list.
//   k_decode_attend  split-K: the active chunks of (b, kv head) plus the partial diagonal
//                    chunk form a list; all lists are cut into segments of one common
//                    size, as many as keep every workgroup slot of the GPU busy in one
//                    round, so that long and short lists are balanced; the work unit is
//                    a 32-key half item, so a segment splits over the workgroup's 4 waves
//                    to within half an item (waves 2i and 2i + 1 take the two halves of
//                    every second item, starting at item i).  S^T = K Q^T with K rows
//                    loaded straight from global as MFMA operands, V staged through
//                    wave-private LDS in [d][key] order for the V^T P^T product; the waves'
//                    (max, sum, O) partials are merged in LDS and written once per
//                    workgroup.
//   k_decode_combine log-sum-exp merge of the segment partials, one workgroup per (b, kv
//                    head).
// Decoding is HBM-bound: the active K/V chunks (32 KiB each at D = 128) dominate the bytes.
#include <atomic>
#include <type_traits>

#include "route_common.h"

namespace dash {

namespace {

__device__ __forceinline__ floatx4 mfma16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// reductions over lanes l, l^16, l^32, l^48 (the four 16-lane rows) with the row-swap moves
template <typename Op>
__device__ __forceinline__ float xg_reduce(float v, Op op) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xg_max(float v) {
  return xg_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ float xg_sum(float v) {
  return xg_reduce(v, [](float x, float y) { return x + y; });
}

constexpr int kSeg = 16;        // the fewest list items an attend segment (workgroup) takes
// dword 3 of a raw buffer descriptor on gfx9-family parts (32-bit data format, offsets in
// bytes, bounds checked against the record count)
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kAttWaves = 4;
constexpr float kNegBig = -1.0e30f;
// A lane's 16 unnormalised probabilities of an item may sum to at most 2^8 before the
// reference max is raised; a larger sum, an overflow or a NaN triggers the rescale.
constexpr float kSumCap = 256.0f;

}  // namespace

// ------------------------------------------------------------------------------ route
// Scores of one row per (b, kv head) against every routed summary, spread over many
// workgroups (one 16-chunk tile per wave): S^T tile = 16 chunks x 16 head columns on MFMA,
// the fp32 summaries split into bf16 hi + lo in registers.  Written scaled, as
// sco[b, kv head][g][c], for the solver kernel.
template <int D>
__global__ __launch_bounds__(256) void k_decode_scores(RouteArgs a) {
  constexpr int KS = D / 32;
  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int bk = blockIdx.y, b = bk / a.Hkv, kvh = bk % a.Hkv;
  const int ct = blockIdx.x * 4 + wv;              // this wave's tile of 16 chunks
  // the sequence length, the queries and the tile's summary rows are loaded together: no
  // address depends on the length (rows are clamped to the cache), only which results count
  const int slen = a.seq_lens[b];
  bf16x8 qop[KS];
  const bool qok = l16 < G;
  {
    const bf16* qp = (const bf16*)a.q + ((size_t)b * a.Hq + kvh * G + (qok ? l16 : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks + 8 * lg);
  }
  const int crow = 16 * ct + l16;
  const float* srow = a.summ + ((size_t)bk * a.nc_alloc + min(crow, a.nc_alloc - 1)) * D;
  float4 xr[2 * KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    xr[2 * ks] = *reinterpret_cast<const float4*>(srow + 32 * ks + 8 * lg);
    xr[2 * ks + 1] = *reinterpret_cast<const float4*>(srow + 32 * ks + 8 * lg + 4);
  }
  const int t = slen - 1;
  const bool valid = t >= 0 && t < a.tcap;
  const int it = valid ? t / kChunk : 0;
  if (16 * ct >= it) return;                       // (whole wave)
  const bool cok = crow < it;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    if (!qok) qop[ks] = bf16x8{};
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const float4 x0 = xr[2 * ks], x1 = xr[2 * ks + 1];
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    bf16x8 hi, lo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16 h = (bf16)xs[i];
      hi[i] = h;
      lo[i] = (bf16)(xs[i] - (float)h);
    }
    if (!cok) { hi = bf16x8{}; lo = bf16x8{}; }
    acc = mfma16(hi, qop[ks], acc);
    acc = mfma16(lo, qop[ks], acc);
  }
  // C[4 lg + j][l16]: chunk 16 ct + 4 lg + j, head column l16
  if (l16 < G) {
    float* dst = a.sco + ((size_t)bk * G + l16) * a.sco_ld + 16 * ct + 4 * lg;
    *reinterpret_cast<float4*>(dst) =
        make_float4(a.zscale * acc[0], a.zscale * acc[1], a.zscale * acc[2], a.zscale * acc[3]);
  }
}

// Threshold, weights, GQA average, mask, work list: one 16-wave workgroup per (b, kv head).
template <int D, int MODE>
__global__ __launch_bounds__(1024) void k_decode_route(RouteArgs a) {
  constexpr int NW = 16, NR = kMaxRoutedRegs;
  constexpr int ld = kMaxRouted + 16;
  __shared__ __attribute__((aligned(16))) float sc[16 * ld];  // [head][chunk] weights
  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bk = blockIdx.x;
  const int t = a.seq_lens[bk / a.Hkv] - 1;
  const bool valid = t >= 0 && t < a.tcap;
  const int it = valid ? t / kChunk : 0;
  const float* srow = a.sco + ((size_t)bk * G + (wv < G ? wv : 0)) * a.sco_ld;

  // estimate_diagonal: the own chunk's summary over its keys i_t C .. t (Stage 0's formula);
  // every head then scores it as routed entry i_t, which joins the threshold but never the
  // mask, the weights or the work list.  Wave w scores keys 4w .. 4w + 3 against head_cls
  // (its lanes spanning the columns, so each key row is one coalesced read); then thread
  // (key group, column) sums its keys' softmax-weighted columns and the groups are added.
  constexpr int NGD = 1024 / D, KPG = kChunk / NGD;   // key groups, keys per group
  __shared__ float kdg[D];
  __shared__ float dlg[kChunk];
  __shared__ float dpart[NGD][D];
  const bool diag = a.kdiag != nullptr && MODE != kTopK && it > 0 && it < kMaxRouted;
  float ydiag = -INFINITY;
  if (diag) {
    const int b = bk / a.Hkv, kvh = bk % a.Hkv;
    // paged caches: the own chunk's page; an id outside the pool reads as zero keys
    int pg = 0;
    if (a.kdiag_bt) pg = a.kdiag_bt[(size_t)b * a.kdiag_bt_ld + it];
    const bool pok = a.kdiag_bt == nullptr || (pg >= 0 && pg < a.kdiag_pages);
    const bf16* kb = a.kdiag_bt
        ? (const bf16*)a.kdiag + ((size_t)(pok ? pg : 0) * a.Hkv + kvh) * kChunk * D
        : (const bf16*)a.kdiag + ((size_t)bk * a.kdiag_ld + (size_t)it * kChunk) * D;
    const bf16* hc = (const bf16*)a.head_cls + (size_t)kvh * D;
    const int nk = pok ? t - it * kChunk + 1 : 0;
    constexpr int E = D / 64;
    float hv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) hv[e] = (float)hc[lane * E + e];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * wv + i;
      float part = 0.f;
      if (j < nk) {
#pragma unroll
        for (int e = 0; e < E; ++e) part = fmaf(hv[e], (float)kb[(size_t)j * D + lane * E + e], part);
      }
      part = wave_sum(part);
      if (lane == 0) dlg[j] = j < nk ? part * a.s0_scale_log2 : -INFINITY;
    }
    __syncthreads();
    float m = -INFINITY;
    for (int j = 0; j < nk; ++j) m = fmaxf(m, dlg[j]);
    float se = 0.f;
    for (int j = 0; j < nk; ++j) se += fast_exp2(dlg[j] - m);
    const int dc = tid % D, kg = tid / D;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < KPG; ++i) {
      const int j = kg * KPG + i;
      if (j < nk) acc = fmaf(fast_exp2(dlg[j] - m), (float)kb[(size_t)j * D + dc], acc);
    }
    dpart[kg][dc] = se > 0.f ? acc / se : 0.f;
    __syncthreads();
    if (tid < D) {
      float sum = 0.f;
#pragma unroll
      for (int g2 = 0; g2 < NGD; ++g2) sum += dpart[g2][tid];
      kdg[tid] = sum;
    }
    __syncthreads();
    if (wv < G) {
      const bf16* qh = (const bf16*)a.q + (size_t)(b * a.Hq + kvh * G + wv) * D;
      float acc = 0.f;
      for (int d = lane; d < D; d += 64) acc = fmaf((float)qh[d], kdg[d], acc);
      ydiag = a.zscale * wave_sum(acc);
    }
  }
  const int nent = diag ? it + 1 : it;   // entries of the normalisation

  // per-head threshold: wave g owns head g, lane l holds chunks l, l + 64, ...; the
  // register count follows the routed length (in steps of 128 chunks past 1024)
  auto solve = [&](auto nr_tag) {
    constexpr int NRU = decltype(nr_tag)::value;
    float y[NRU];
    if constexpr (MODE == kTopK) {
      // top-k comparison router (wave 0): group score = the G heads' scores summed in head
      // order; the chunks at or above the k-th largest get weight 1 for every head (so their
      // mean is 1).  The k-th largest is the largest order-preserving key u with
      // count(key >= u) >= k, built from the top bit down; it stops once that count is k.
      constexpr uint32_t kKeyFinite = 0x00800000u;   // every finite score's key is above it
#pragma unroll
      for (int r = 0; r < NRU; ++r) y[r] = 0.f;
      for (int g = 0; g < G; ++g) {
        const float* sg = a.sco + ((size_t)bk * G + g) * a.sco_ld;
#pragma unroll
        for (int r = 0; r < NRU; ++r) {
          const int c = lane + 64 * r;
          if (c < it) y[r] += sg[c];
        }
      }
      uint32_t key[NRU];
#pragma unroll
      for (int r = 0; r < NRU; ++r) {
        const uint32_t u = __float_as_uint(y[r]);
        key[r] = lane + 64 * r < it ? ((u & 0x80000000u) ? ~u : (u | 0x80000000u)) : 0u;
      }
      uint32_t thr = 0u;
      float have = (float)it;
      if (it > a.topk) {
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t cand = max(thr | (1u << bit), kKeyFinite);
          float cnt = 0.f;
#pragma unroll
          for (int r = 0; r < NRU; ++r) cnt += key[r] >= cand ? 1.f : 0.f;
          cnt = wave_sum(cnt);
          if (cnt >= (float)a.topk) {
            thr |= 1u << bit;
            have = cnt;
          }
          if (have == (float)a.topk) break;
        }
      }
      const uint32_t lim = max(thr, kKeyFinite);
#pragma unroll
      for (int r = 0; r < NRU; ++r) {
        const int c = lane + 64 * r;
        if (c < it) {
          const float v = key[r] >= lim ? 1.f : 0.f;
          for (int g = 0; g < G; ++g) sc[g * ld + c] = v;
        }
      }
      return;
    } else {
#pragma unroll
    for (int r = 0; r < NRU; ++r) {
      const int c = lane + 64 * r;
      y[r] = c < it ? srow[c] : (c == it ? ydiag : -INFINITY);
    }
    float z;
    const float tau = entmax_threshold<MODE, NRU>(y, nent, a.alpha, WaveReduce(), &z);
    const float rz = 1.0f / z, inv = 1.0f / (a.alpha - 1.0f);
    // every slot is stored (LDS columns up to 64 NRU <= kMaxRouted exist); the GQA sum reads
    // only chunks below i_t, so the own chunk's estimate_diagonal entry is never used
#pragma unroll
    for (int r = 0; r < NRU; ++r) {
      const int c = lane + 64 * r;
      float wgt;
      if constexpr (MODE == kAlpha15) {
        const float d = fmaxf(y[r] - tau, 0.f);
        wgt = (d * d) * rz;
      } else if constexpr (MODE == kAlpha2) {
        wgt = fmaxf(y[r] - tau, 0.f) * rz;
      } else {
        wgt = entmax_weight<MODE>(y[r], tau, inv, rz);
      }
      sc[wv * ld + c] = wgt;
    }
    }
  };
  if ((MODE == kTopK ? wv == 0 : wv < G) && it > 0) {
    if (nent <= 256) solve(std::integral_constant<int, 4>{});
    else if (nent <= 512) solve(std::integral_constant<int, 8>{});
    else if (nent <= 768) solve(std::integral_constant<int, 12>{});
    else if (nent <= 1024) solve(std::integral_constant<int, 16>{});
    else if (nent <= 1152) solve(std::integral_constant<int, 18>{});
    else if (nent <= 1280) solve(std::integral_constant<int, 20>{});
    else if (nent <= 1408) solve(std::integral_constant<int, 22>{});
    else if (nent <= 1536) solve(std::integral_constant<int, 24>{});
    else if (nent <= 1664) solve(std::integral_constant<int, 26>{});
    else if (nent <= 1792) solve(std::integral_constant<int, 28>{});
    else if (nent <= 1920) solve(std::integral_constant<int, 30>{});
    else solve(std::integral_constant<int, NR>{});
  }
  __syncthreads();

  // GQA average in head order, mask words by ballot, w_bar at set bits
  __shared__ uint64_t wbits[kMaxRoutedWords];
  __shared__ int wpre[kMaxRoutedWords + 1];
  const float rG = 1.0f / (float)G;
  for (int w = wv; w < a.W; w += NW) {
    const int c = 64 * w + lane;
    float s = 0.f;
    if (c < it)
      for (int g = 0; g < G; ++g) s += sc[g * ld + c];
    const float wb = s * rG;
    const bool on = c < it && wb > 0.f;
    const uint64_t bits = __ballot(on);
    if (on) a.wbar[(size_t)bk * a.wbar_ld + c] = wb;
    if (lane == 0) {
      a.mask[(size_t)bk * a.W + w] = bits;
      if (w < kMaxRoutedWords) wbits[w] = bits;
    }
  }
  // the attend kernels' work list: count, the set chunks in increasing order, then the
  // diagonal chunk
  const int nwr = (it + 63) / 64;                 // words that can hold routed chunks
  __syncthreads();
  if (wv == 0) {
    int v = lane < nwr ? __popcll(wbits[lane]) : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(v, o, 64);
      if (lane >= o) v += u;
    }
    if (lane < nwr) wpre[lane + 1] = v;
    if (lane == 0) wpre[0] = 0;
  }
  __syncthreads();
  int32_t* lst = a.list + (size_t)bk * a.list_ld;
  for (int w = wv; w < nwr; w += NW) {
    const uint64_t bits = wbits[w];
    if ((bits >> lane) & 1ull) {
      const uint64_t below = lane ? (bits & ((1ull << lane) - 1ull)) : 0ull;
      lst[1 + wpre[w] + __popcll(below)] = 64 * w + lane;
    }
  }
  if (tid == 0) {
    lst[0] = wpre[nwr] + 1;
    lst[1 + wpre[nwr]] = it;
  }
}

// ------------------------------------------------------------------------------ attend
// Global segmentation of the work lists (one wave): all B * Hkv lists are cut into segments
// of one common size per = max(kSeg, ceil(N / (S - B Hkv))), N the total number of items
// and S the number of attend workgroups, so that a (b, kv head) with n items gets
// ceil(n / per) <= n / per + 1 segments and all of them fit in S.  Returns per.
__device__ __forceinline__ int wave_isum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int segment_size(const AttendArgs& a, int S, int lane) {
  const int BH = a.B * a.Hkv;
  int n = 0;
  for (int i = lane; i < BH; i += 64) n += a.list[(size_t)i * a.list_ld];
  n = wave_isum(n);
  const int room = max(1, S - BH);
  return max(kSeg, (n + room - 1) / room);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// V^T operand of the 16x16x32 MFMA for d rows d0 + (l % 16) and keys k0 + [0, 8), read from
// a row-major [key][d] LDS tile with two transposing loads (ds_read_b64_tr_b16): within a
// 16-lane group, source lane r = 4k + q points at V[k0 + k][d0 + 4q] and output lane i
// receives V[k0 + k][d0 + i] for k = 0..3.
__device__ __forceinline__ bf16x8 vt_operand(const bf16* tile, int pitch, int k0, int d0, int l16) {
  const int k = l16 >> 2, q = l16 & 3;
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const bf16* p0 = tile + (k0 + k) * pitch + d0 + 4 * q;
  const bf16* p1 = p0 + 4 * pitch;
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p1));
  // concatenate as whole vectors: element-wise bf16 re-packing of these results was
  // miscompiled (halves duplicated) by this toolchain
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 r = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, r);
}

template <int D>
__global__ __launch_bounds__(kAttWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void k_decode_attend(AttendArgs a, float* __restrict__ pml, float* __restrict__ po, int nseg_max,
                     int seg_total) {
  constexpr int NT = kAttWaves * 64;
  constexpr int KS = D / 32, NDT = D / 16;
  constexpr int VP = D + 16;                      // V row pitch in LDS (bf16 elements)
  constexpr int SEGR = D / 8;                     // 16-byte segments per V row
  constexpr int VL = 32 * SEGR / 64;              // segments per lane per half tile
  __shared__ __attribute__((aligned(16))) bf16 vts[kAttWaves][32 * VP];
  __shared__ float mrg_ml[kAttWaves][2][16];

  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  // ---- this workgroup's (b, kv head) and segment: wave 0 finds the (b, kv head) whose run
  // of segments holds this workgroup's index, by a prefix over the lists' segment counts
  __shared__ int smap[4];
  if (wv == 0) {
    const int BH = a.B * a.Hkv;
    const int per = segment_size(a, seg_total, lane);
    const int wg = blockIdx.x;
    int base = 0, fbk = -1, fseg = 0, fnt = 0;
    for (int i0 = 0; i0 < BH; i0 += 64) {
      const int i = i0 + lane;
      const int nt = i < BH ? a.list[(size_t)i * a.list_ld] : 0;
      const int ns = (nt + per - 1) / per;
      int incl = ns;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int x = __shfl_up(incl, o, 64);
        if (lane >= o) incl += x;
      }
      const int excl = base + incl - ns;
      const uint64_t hit = __ballot(i < BH && wg >= excl && wg < excl + ns);
      if (hit) {
        const int src = __builtin_ctzll(hit);
        fbk = i0 + src;
        fseg = wg - __shfl(excl, src, 64);
        fnt = __shfl(nt, src, 64);
        break;
      }
      base += __shfl(incl, 63, 64);
    }
    if (lane == 0) {
      smap[0] = fbk;
      smap[1] = fseg;
      smap[2] = fnt;
      smap[3] = per;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid == 0) *a.seg_size = smap[3];     // for the combine kernel
  const int bk = smap[0];
  if (bk < 0) return;                             // past the last segment (whole workgroup)
  const int seg = smap[1];
  const int b = bk / a.Hkv, kvh = bk % a.Hkv;
  const int t = a.seq_lens[b] - 1;
  if (t < 0 || t >= a.Tk) {                       // no valid query row: NaN outputs
    if (seg == 0)
      for (int i = tid; i < G * D; i += NT)
        ((bf16*)a.out)[((size_t)b * a.Hq + kvh * G) * D + i] = (bf16)__builtin_nanf("");
    return;
  }
  const int it = t / kChunk;

  // ---- this workgroup's segment of the route kernel's list (active chunks + the diagonal
  // chunk)
  const int32_t* lst = a.list + (size_t)bk * a.list_ld;
  const int ntot = smap[2];
  const int per = smap[3];
  const int lo = seg * per;
  const int nitems = min(per, ntot - lo);
  // The work unit is a 32-key half of an item, so that the segment's work splits over the
  // waves to within half an item: wave wv takes half hp = wv & 1 (keys 32 hp .. 32 hp + 31)
  // of the items lo + wv / 2 + 2 j; lane j of myc holds the chunk of its item j.
  static_assert(kAttWaves == 4, "two waves per half-item column");
  const int hp = wv & 1;
  const int nmy = max(0, (nitems - (wv >> 1) + 1) / 2);
  const int32_t* myl = lst + 1 + lo + (wv >> 1);
  const int myc = lane < nmy ? myl[2 * lane] : it;
  auto chunk_of = [&](int j) {
    return j < 64 ? __builtin_amdgcn_readlane(myc, j) : myl[2 * j];
  };
  // paged caches: the page of each of those chunks (-1 past the list)
  const int32_t* btab = a.block_table ? a.block_table + (size_t)b * a.bt_ld : nullptr;
  const int mypg = btab ? (lane < nmy ? btab[myc] : -1) : 0;
  auto page_of = [&](int j, int c) {
    return j < 64 ? __builtin_amdgcn_readlane(mypg, j) : btab[c];
  };

  // ---- query columns: the G heads of this kv head (columns >= G are zero)
  bf16x8 qop[KS];
  {
    const bool qok = l16 < G;
    const bf16* qp = (const bf16*)a.q + ((size_t)b * a.Hq + kvh * G + (qok ? l16 : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 32 * ks + 8 * lg);
      qop[ks] = qok ? v : bf16x8{};
    }
  }
  const bf16* kb = (const bf16*)a.k + (size_t)bk * a.Tk * D;
  const bf16* vb = (const bf16*)a.v + (size_t)bk * a.Tk * D;
  bf16* vl = vts[wv];
  const float sl2 = a.scale_log2;
  float m = kNegBig, lsum = 0.f;
  floatx4 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // registers for one half-item: K operands (A of S^T, key tiles 2 hp and 2 hp + 1) and
  // this lane's V segments of the half, fetched through buffer descriptors whose range ends
  // at the item's last valid key (t on the diagonal), so keys past it read as zeros without
  // branches
  bf16x8 kop[2][KS];
  uint4 vseg[VL];
  int koff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int key = 32 * hp + 8 * (l16 >> 2) + 4 * h + (l16 & 3);
    koff[h] = (key * D + 8 * lg) * 2;
  }
  const int voff0 = 32 * hp * SEGR * 16;          // byte offset of the half's first V row
  // a chunk's K and V rows: contiguous caches index by chunk, paged ones by page; a page id
  // outside the pool gives an empty range, so its keys and values read as zeros
  auto load_item = [&](int j) {
    const int c = __builtin_amdgcn_readfirstlane(chunk_of(j));
    int nkeys = min(kChunk, t - c * kChunk + 1);                // 64 except on the diagonal
    const bf16* kp = kb + (size_t)c * kChunk * D;
    const bf16* vp = vb + (size_t)c * kChunk * D;
    if (btab) {
      const int pg = __builtin_amdgcn_readfirstlane(page_of(j, c));
      const bool okp = pg >= 0 && pg < a.num_pages;
      const size_t off = ((size_t)(okp ? pg : 0) * a.Hkv + kvh) * kChunk * D;
      kp = (const bf16*)a.k + off;
      vp = (const bf16*)a.v + off;
      if (!okp) nkeys = 0;
    }
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)kp, (short)0, nkeys * D * 2, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)vp, (short)0, nkeys * D * 2, kBufferRsrcWord3);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kop[h][ks] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(kr, koff[h] + 64 * ks, 0, 0));
    // V is read once per step and staged through LDS: the loads carry the non-temporal hint
    // (cache policy bit 1, nt), so the streamed values do not displace what the step's other
    // reads find in the caches (64K decode step 112.1 -> 99.9 us; the same hint on the K
    // loads, which feed the matrix cores from registers, was slower)
#pragma unroll
    for (int i = 0; i < VL; ++i)
      vseg[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, voff0 + (i * 64 + lane) * 16, 0, 2));
  };

  if (nmy > 0) load_item(0);
  // routing bias of each item (sigma log2 w_bar; 0 for the diagonal chunk), lane j for item j,
  // loaded while the first tiles are in flight
  const float mybias =
      (lane < nmy && myc != it) ? a.sigma * fast_log2(a.wbar[(size_t)bk * a.wbar_ld + myc]) : 0.f;
  for (int j = 0; j < nmy; ++j) {
    const int c = chunk_of(j);
    const bool diag = c == it;
    const int kmax = diag ? t : c * kChunk + 63;
    // the half's V rows -> LDS (row-major, padded)
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int sg = i * 64 + lane;
      const int key = sg / SEGR, db = (sg % SEGR) * 8;
      *reinterpret_cast<uint4*>(vl + key * VP + db) = vseg[i];
    }
    // wait for these stores before the transposing LDS reads below: unlike ordinary LDS
    // reads they are not ordered behind the wave's outstanding LDS writes
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // S^T = K Q^T over the half's 32 keys
    floatx4 s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s[h] = mfma16(kop[h][ks], qop[ks], s[h]);
    }
    const float bias = j < 64 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mybias), j))
                              : (diag ? 0.f : a.sigma * fast_log2(a.wbar[(size_t)bk * a.wbar_ld + c]));
    // next item's loads overlap the softmax and the PV product
    if (j + 1 < nmy) load_item(j + 1);
    // online softmax against the reference max m, which is only raised (with the rescale
    // of O and l) when a lane's partial probability sum exceeds kSumCap; keys past the
    // query are masked on the diagonal item only
    float x[8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) x[4 * h + jj] = s[h][jj];
    if (diag) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int key = 32 * hp + 8 * lg + 4 * h + jj;
          if (c * kChunk + key > kmax) x[4 * h + jj] = -INFINITY;
        }
    }
    float off = bias - m;
    float ps = 0.f;
    float pr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr[i] = fast_exp2(fmaf(x[i], sl2, off));
      ps += pr[i];
    }
    if (__builtin_amdgcn_ballot_w64(!(ps <= kSumCap)) != 0ull) {
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
      mx = xg_max(mx);
      const float mn = fmaxf(m, fmaf(mx, sl2, bias));
      const float corr = fast_exp2(m - mn);
      m = mn;
      lsum *= corr;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= corr;
      off = bias - mn;
      ps = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pr[i] = fast_exp2(fmaf(x[i], sl2, off));
        ps += pr[i];
      }
    }
    lsum += ps;
    // P^T operand of the half (k-slot i <-> key 32 hp + 8 lg + i)
    bf16x8 pop;
#pragma unroll
    for (int i = 0; i < 8; ++i) pop[i] = (bf16)pr[i];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      o[dt] = mfma16(vt_operand(vl, VP, 8 * lg, 16 * dt, l16), pop, o[dt]);
    asm volatile("" ::: "memory");  // the next item's stores stay after these reads
  }
  // merge the waves' partials: (m, l) per query column, then O rescaled and summed in LDS
  lsum = xg_sum(lsum);
  if (lg == 0) {
    mrg_ml[wv][0][l16] = m;
    mrg_ml[wv][1][l16] = lsum;
  }
  __syncthreads();
  float mt = kNegBig;
#pragma unroll
  for (int w = 0; w < kAttWaves; ++w) mt = fmaxf(mt, mrg_ml[w][0][l16]);
  const float f = fast_exp2(m - mt);
  float* ob = reinterpret_cast<float*>(&vts[0][0]);          // reuse: [D][16] floats
  for (int w = 0; w < kAttWaves; ++w) {
    if (wv == w) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d = 16 * dt + 4 * lg + jj;
          const float v = o[dt][jj] * f;
          ob[d * 16 + l16] = (w == 0) ? v : ob[d * 16 + l16] + v;
        }
    }
    __syncthreads();
  }
  const size_t pbase = (size_t)bk * nseg_max;
  const size_t pidx = pbase + seg;
  if (tid < 16) {
    float lt = 0.f;
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) lt += mrg_ml[w][1][tid] * fast_exp2(mrg_ml[w][0][tid] - mt);
    pml[pidx * 32 + tid] = mt;
    pml[pidx * 32 + 16 + tid] = lt;
  }
  for (int i = tid; i < 16 * D; i += NT) {
    const int q = i / D, d = i % D;
    po[(pidx * 16 + q) * D + d] = ob[d * 16 + q];
  }

}

// ------------------------------------------------------------------------------ combine
// Log-sum-exp merge of a (b, kv head)'s segment partials into the G heads' outputs: one
// workgroup per (b, kv head), thread -> (query column, 8 consecutive d).
template <int D>
__global__ __launch_bounds__(256) void k_decode_combine(AttendArgs a, const float* __restrict__ pml,
                                                        const float* __restrict__ po, int nseg_max,
                                                        int seg_total) {
  constexpr int NT = 256, NSMAX = (kMaxRouted + 1 + kSeg) / kSeg + 1;
  constexpr int kPre = 16;                        // segments whose partials are loaded at once
  static_assert(2 * D <= NT, "one thread per (query column, 8 d)");
  __shared__ float fsm[NSMAX * 16], fsl[NSMAX * 16], colm[16], coll[16];
  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x;
  const int bk = blockIdx.x, b = bk / a.Hkv, kvh = bk % a.Hkv;
  const size_t pbase = (size_t)bk * nseg_max;
  // one round of loads: the sequence length, the list length, the segment size, and
  // the partials and (max, sum) pairs of up to kPre segments before their count is known
  // (all inside the partial buffers; those of segments past the count are never used)
  const int t = a.seq_lens[b] - 1;
  const int q = tid / (D / 8), d0 = (tid % (D / 8)) * 8;
  const bool act = tid < 2 * D && q < G;
  const float* src = po + (pbase * 16 + (act ? q : 0)) * D + d0;
  const int npre = min(nseg_max, kPre);
  float4 u[kPre][2];
#pragma unroll
  for (int s2 = 0; s2 < kPre; ++s2)
    if (s2 < npre) {
      u[s2][0] = *reinterpret_cast<const float4*>(src + (size_t)s2 * 16 * D);
      u[s2][1] = *reinterpret_cast<const float4*>(src + (size_t)s2 * 16 * D + 4);
    }
  for (int i = tid; i < npre * 16; i += NT) {
    const size_t pi = pbase + i / 16;
    fsm[i] = pml[pi * 32 + (i & 15)];
    fsl[i] = pml[pi * 32 + 16 + (i & 15)];
  }
  const int nt = a.list[(size_t)bk * a.list_ld];
  const int per = *a.seg_size;                    // written by the attend kernel
  __syncthreads();
  if (t < 0 || t >= a.Tk) return;                 // the attend kernel wrote NaN
  const int nsegb = (nt + per - 1) / per;
  if (nsegb > npre) {                             // more segments than the first round held
    for (int i = npre * 16 + tid; i < nsegb * 16; i += NT) {
      const size_t pi = pbase + i / 16;
      fsm[i] = pml[pi * 32 + (i & 15)];
      fsl[i] = pml[pi * 32 + 16 + (i & 15)];
    }
    __syncthreads();
  }
  if (tid < 16) {
    float mx = kNegBig;
    for (int s2 = 0; s2 < nsegb; ++s2) mx = fmaxf(mx, fsm[s2 * 16 + tid]);
    float l = 0.f;
    for (int s2 = 0; s2 < nsegb; ++s2) l += fsl[s2 * 16 + tid] * fast_exp2(fsm[s2 * 16 + tid] - mx);
    colm[tid] = mx;
    coll[tid] = 1.0f / l;
  }
  __syncthreads();
  if (!act) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const float4& u0, const float4& u1, float fct) {
    acc[0] = fmaf(u0.x, fct, acc[0]);
    acc[1] = fmaf(u0.y, fct, acc[1]);
    acc[2] = fmaf(u0.z, fct, acc[2]);
    acc[3] = fmaf(u0.w, fct, acc[3]);
    acc[4] = fmaf(u1.x, fct, acc[4]);
    acc[5] = fmaf(u1.y, fct, acc[5]);
    acc[6] = fmaf(u1.z, fct, acc[6]);
    acc[7] = fmaf(u1.w, fct, acc[7]);
  };
  const float cm = colm[q], cl = coll[q];
#pragma unroll
  for (int s2 = 0; s2 < kPre; ++s2)
    if (s2 < nsegb) add(u[s2][0], u[s2][1], fast_exp2(fsm[s2 * 16 + q] - cm) * cl);
  for (int s2 = kPre; s2 < nsegb; ++s2)
    add(*reinterpret_cast<const float4*>(src + (size_t)s2 * 16 * D),
        *reinterpret_cast<const float4*>(src + (size_t)s2 * 16 * D + 4),
        fast_exp2(fsm[s2 * 16 + q] - cm) * cl);
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)acc[e];
  *reinterpret_cast<bf16x8*>((bf16*)a.out + ((size_t)b * a.Hq + kvh * G + q) * D + d0) = v;
}

// ------------------------------------------------------------------------------ launchers
int decode_nseg_max(int nc) { return (nc + 1 + kSeg - 1) / kSeg; }

hipError_t launch_decode_route(const RouteArgs& a, hipStream_t s) {
  dim3 gs((a.nc_alloc + 63) / 64, a.B * a.Hkv);
  if (a.D == 128) k_decode_scores<128><<<gs, 256, 0, s>>>(a);
  else k_decode_scores<64><<<gs, 256, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(a.B * a.Hkv);
  if (a.D == 128) {
    if (a.topk > 0) k_decode_route<128, kTopK><<<grid, 1024, 0, s>>>(a);
    else if (a.alpha == 1.5f) k_decode_route<128, kAlpha15><<<grid, 1024, 0, s>>>(a);
    else if (a.alpha == 2.0f) k_decode_route<128, kAlpha2><<<grid, 1024, 0, s>>>(a);
    else k_decode_route<128, kAlphaGeneral><<<grid, 1024, 0, s>>>(a);
  } else {
    if (a.topk > 0) k_decode_route<64, kTopK><<<grid, 1024, 0, s>>>(a);
    else if (a.alpha == 1.5f) k_decode_route<64, kAlpha15><<<grid, 1024, 0, s>>>(a);
    else if (a.alpha == 2.0f) k_decode_route<64, kAlpha2><<<grid, 1024, 0, s>>>(a);
    else k_decode_route<64, kAlphaGeneral><<<grid, 1024, 0, s>>>(a);
  }
  return hipGetLastError();
}

// Workgroup slots of the device (two attend workgroups per CU), looked up once per device
// (callers on several host threads may race to fill the entry; they store the same value).
static int attend_slots() {
  static std::atomic<int> slots[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
  int n = slots[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    n = 2 * cus;
    slots[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_decode_attend(const AttendArgs& a, float* pml, float* po, hipStream_t s) {
  if (a.seg_size == nullptr || a.list == nullptr || pml == nullptr || po == nullptr)
    return hipErrorInvalidValue;                  // workspace pieces the kernels write
  const int nseg = decode_nseg_max(a.nc);
  const int bh = a.B * a.Hkv;
  // one workgroup per segment: as many as fill every slot once (at least one per (b, kv
  // head)); the common segment size keeps every (b, kv head) within the partial buffers
  // (each segment has at least kSeg items)
  const int total = max(attend_slots(), bh);
  if (a.D == 128) k_decode_attend<128><<<total, kAttWaves * 64, 0, s>>>(a, pml, po, nseg, total);
  else k_decode_attend<64><<<total, kAttWaves * 64, 0, s>>>(a, pml, po, nseg, total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.D == 128) k_decode_combine<128><<<bh, 256, 0, s>>>(a, pml, po, nseg, total);
  else k_decode_combine<64><<<bh, 256, 0, s>>>(a, pml, po, nseg, total);
  return hipGetLastError();
}

}  // namespace dash
