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
//                    threshold with wave-only reductions; then a fixed-order sum over the
//                    heads, a ballot per 64 chunks for the mask word, w_bar at set bits and
//                    the attend kernels' work list.
//   k_decode_attend  split-K: the active chunks of (b, kv head) plus the partial diagonal
//                    chunk form a list; each workgroup takes 16 consecutive items, each of
//                    its 4 waves a quarter of them.  S^T = K Q^T with K rows loaded straight
//                    from global as MFMA operands, V staged through wave-private LDS in
//                    [d][key] order for the V^T P^T product; the waves' (max, sum, O)
//                    partials are merged in LDS and written once per workgroup.
//   k_decode_combine log-sum-exp merge of the segment partials, one workgroup per (b, head).
// Decoding is HBM-bound: the active K/V chunks (32 KiB each at D = 128) dominate the bytes.
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

constexpr int kSeg = 16;        // list items per attend workgroup
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
  const int t = a.seq_lens[b] - 1;
  const bool valid = t >= 0 && t < a.tcap;
  const int it = valid ? t / kChunk : 0;
  const int ct = blockIdx.x * 4 + wv;              // this wave's tile of 16 chunks
  if (16 * ct >= it) return;                       // (whole wave)
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
  const int crow = 16 * ct + l16;
  const bool cok = crow < it;
  const float* srow = a.summ + ((size_t)bk * a.nc_alloc + (cok ? crow : 0)) * D;
  float4 xr[2 * KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    xr[2 * ks] = *reinterpret_cast<const float4*>(srow + 32 * ks + 8 * lg);
    xr[2 * ks + 1] = *reinterpret_cast<const float4*>(srow + 32 * ks + 8 * lg + 4);
  }
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

  // per-head threshold: wave g owns head g, lane l holds chunks l, l + 64, ...; the
  // register count follows the routed length
  auto solve = [&](auto nr_tag) {
    constexpr int NRU = decltype(nr_tag)::value;
    float y[NRU];
#pragma unroll
    for (int r = 0; r < NRU; ++r) {
      const int c = lane + 64 * r;
      y[r] = c < it ? srow[c] : -INFINITY;
    }
    float z;
    const float tau = entmax_threshold<MODE, NRU>(y, it, a.alpha, WaveReduce(), &z);
    const float rz = 1.0f / z, inv = 1.0f / (a.alpha - 1.0f);
#pragma unroll
    for (int r = 0; r < NRU; ++r) {
      const int c = lane + 64 * r;
      if (c < it) sc[wv * ld + c] = entmax_weight<MODE>(y[r], tau, inv, rz);
    }
  };
  if (wv < G && it > 0) {
    if (it <= 256) solve(std::integral_constant<int, 4>{});
    else if (it <= 512) solve(std::integral_constant<int, 8>{});
    else if (it <= 1024) solve(std::integral_constant<int, 16>{});
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
void k_decode_attend(AttendArgs a, float* __restrict__ pml,
                                                                  float* __restrict__ po, int nseg_max) {
  constexpr int KS = D / 32, NDT = D / 16;
  constexpr int VP = D + 16;                      // V row pitch in LDS (bf16 elements)
  constexpr int SEGR = D / 8;                     // 16-byte segments per V row
  constexpr int VL = 64 * SEGR / 64;              // segments per lane per tile
  __shared__ __attribute__((aligned(16))) bf16 vts[kAttWaves][64 * VP];
  __shared__ float mrg_ml[kAttWaves][2][16];

  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int seg = blockIdx.x, bk = blockIdx.y;
  const int b = bk / a.Hkv, kvh = bk % a.Hkv;
  const int t = a.seq_lens[b] - 1;
  if (t < 0 || t >= a.Tk) return;                 // the combine kernel writes NaN
  const int it = t / kChunk;

  // ---- this workgroup's items from the route kernel's list, with their routing bias
  // (log2 w_bar; 0 for the diagonal chunk), staged in LDS once so that the loop below never
  // waits on a global load other than its own tiles
  __shared__ int citem[kSeg];
  __shared__ float cbias[kSeg];
  const int32_t* lst = a.list + (size_t)bk * a.list_ld;
  const int ntot = lst[0];                        // active chunks + the diagonal chunk
  const int lo = seg * kSeg;
  const int nitems = min(kSeg, ntot - lo);
  if (nitems <= 0) return;
  if (tid < nitems) {
    const int c = lst[1 + lo + tid];
    citem[tid] = c;
    cbias[tid] = c == it ? 0.f : fast_log2(a.wbar[(size_t)bk * a.wbar_ld + c]);
  }
  __syncthreads();

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

  // registers for one item: K operands (A of S^T) and this lane's V segments, fetched
  // through buffer descriptors whose range ends at the item's last valid key (t on the
  // diagonal), so keys past it read as zeros without branches
  bf16x8 kop[4][KS];
  uint4 vseg[VL];
  int koff[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int key = 32 * (kt >> 1) + 8 * (l16 >> 2) + 4 * (kt & 1) + (l16 & 3);
    koff[kt] = (key * D + 8 * lg) * 2;
  }
  auto load_item = [&](int c_any) {
    const int c = __builtin_amdgcn_readfirstlane(c_any);
    const int nkeys = min(kChunk, t - c * kChunk + 1);          // 64 except on the diagonal
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kb + (size_t)c * kChunk * D), (short)0, nkeys * D * 2, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vb + (size_t)c * kChunk * D), (short)0, nkeys * D * 2, kBufferRsrcWord3);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kop[kt][ks] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(kr, koff[kt] + 64 * ks, 0, 0));
#pragma unroll
    for (int i = 0; i < VL; ++i)
      vseg[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, (i * 64 + lane) * 16, 0, 0));
  };

  if (wv < nitems) load_item(citem[wv]);
  for (int ii = wv; ii < nitems; ii += kAttWaves) {
    const int c = citem[ii];
    const bool diag = c == it;
    const int kmax = diag ? t : c * kChunk + 63;
    // V rows -> LDS (row-major, padded)
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int sg = i * 64 + lane;
      const int key = sg / SEGR, db = (sg % SEGR) * 8;
      *reinterpret_cast<uint4*>(vl + key * VP + db) = vseg[i];
    }
    // wait for these stores before the transposing LDS reads below: unlike ordinary LDS
    // reads they are not ordered behind the wave's outstanding LDS writes
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // S^T = K Q^T
    floatx4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s[kt] = mfma16(kop[kt][ks], qop[ks], s[kt]);
    }
    const float bias = cbias[ii];
    // next item's loads overlap the softmax and the PV product
    if (ii + kAttWaves < nitems) load_item(citem[ii + kAttWaves]);
    // online softmax against the reference max m, which is only raised (with the rescale
    // of O and l) when a lane's partial probability sum exceeds kSumCap; keys past the
    // query are masked on the diagonal item only
    float x[16];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * kt + j] = s[kt][j];
    if (diag) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1) + j;
          if (c * kChunk + key > kmax) x[4 * kt + j] = -INFINITY;
        }
    }
    float off = bias - m;
    float ps = 0.f;
    float pr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      pr[i] = fast_exp2(fmaf(x[i], sl2, off));
      ps += pr[i];
    }
    if (__builtin_amdgcn_ballot_w64(!(ps <= kSumCap)) != 0ull) {
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, x[i]);
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
      for (int i = 0; i < 16; ++i) {
        pr[i] = fast_exp2(fmaf(x[i], sl2, off));
        ps += pr[i];
      }
    }
    lsum += ps;
    bf16x8 pop[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pop[p][j] = (bf16)pr[8 * p + j];
        pop[p][4 + j] = (bf16)pr[8 * p + 4 + j];
      }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int p = 0; p < 2; ++p)
        o[dt] = mfma16(vt_operand(vl, VP, 32 * p + 8 * lg, 16 * dt, l16), pop[p], o[dt]);
    }
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
        for (int j = 0; j < 4; ++j) {
          const int d = 16 * dt + 4 * lg + j;
          const float v = o[dt][j] * f;
          ob[d * 16 + l16] = (w == 0) ? v : ob[d * 16 + l16] + v;
        }
    }
    __syncthreads();
  }
  const size_t pidx = (size_t)bk * nseg_max + seg;
  if (tid < 16) {
    float lt = 0.f;
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) lt += mrg_ml[w][1][tid] * fast_exp2(mrg_ml[w][0][tid] - mt);
    pml[pidx * 32 + tid] = mt;
    pml[pidx * 32 + 16 + tid] = lt;
  }
  for (int i = tid; i < 16 * D; i += kAttWaves * 64) {
    const int q = i / D, d = i % D;
    po[(pidx * 16 + q) * D + d] = ob[d * 16 + q];
  }
}

// ------------------------------------------------------------------------------ combine
// one workgroup of D threads per (b, head); the segment maxima and sums are reduced in
// parallel, then each thread merges its column of the partial outputs.
template <typename TOut, int D>
__global__ __launch_bounds__(D) void k_decode_combine(AttendArgs a, const float* __restrict__ pml,
                                                      const float* __restrict__ po, int nseg_max) {
  __shared__ float fs[256];
  __shared__ float red[D / 64 > 0 ? D / 64 : 1];
  const int bh = blockIdx.x, b = bh / a.Hq, h = bh % a.Hq;
  const int G = a.Hq / a.Hkv, kvh = h / G, q = h % G;
  const int bk = b * a.Hkv + kvh;
  const int d = threadIdx.x, lane = d & 63, wv = d >> 6;
  TOut* op = (TOut*)a.out + (size_t)bh * D;
  const int t = a.seq_lens[b] - 1;
  if (t < 0 || t >= a.Tk) {
    op[d] = from_f32<TOut>(__builtin_nanf(""));
    return;
  }
  const int nseg = (a.list[(size_t)bk * a.list_ld] + kSeg - 1) / kSeg;   // <= 129
  // max over segments
  float mloc = kNegBig;
  for (int s = d; s < nseg; s += D) mloc = fmaxf(mloc, pml[((size_t)bk * nseg_max + s) * 32 + q]);
  mloc = wave_max(mloc);
  if (lane == 0) red[wv] = mloc;
  __syncthreads();
  float mt = red[0];
  for (int w = 1; w < D / 64; ++w) mt = fmaxf(mt, red[w]);
  __syncthreads();
  // per-segment factors and the total sum
  float lloc = 0.f;
  for (int s = d; s < nseg; s += D) {
    const size_t pi = (size_t)bk * nseg_max + s;
    const float f = fast_exp2(pml[pi * 32 + q] - mt);
    fs[s] = f;
    lloc += pml[pi * 32 + 16 + q] * f;
  }
  lloc = wave_sum(lloc);
  if (lane == 0) red[wv] = lloc;
  __syncthreads();
  float l = 0.f;
  for (int w = 0; w < D / 64; ++w) l += red[w];
  float acc = 0.f;
  for (int s = 0; s < nseg; ++s) acc += po[(((size_t)bk * nseg_max + s) * 16 + q) * D + d] * fs[s];
  op[d] = from_f32<TOut>(acc / l);
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
    if (a.alpha == 1.5f) k_decode_route<128, kAlpha15><<<grid, 1024, 0, s>>>(a);
    else if (a.alpha == 2.0f) k_decode_route<128, kAlpha2><<<grid, 1024, 0, s>>>(a);
    else k_decode_route<128, kAlphaGeneral><<<grid, 1024, 0, s>>>(a);
  } else {
    if (a.alpha == 1.5f) k_decode_route<64, kAlpha15><<<grid, 1024, 0, s>>>(a);
    else if (a.alpha == 2.0f) k_decode_route<64, kAlpha2><<<grid, 1024, 0, s>>>(a);
    else k_decode_route<64, kAlphaGeneral><<<grid, 1024, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_attend(const AttendArgs& a, float* pml, float* po, hipStream_t s) {
  const int nseg = decode_nseg_max(a.nc);
  dim3 grid(nseg, a.B * a.Hkv);
  if (a.D == 128) k_decode_attend<128><<<grid, kAttWaves * 64, 0, s>>>(a, pml, po, nseg);
  else k_decode_attend<64><<<grid, kAttWaves * 64, 0, s>>>(a, pml, po, nseg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(a.B * a.Hq);
  if (a.D == 128) k_decode_combine<bf16, 128><<<g2, 128, 0, s>>>(a, pml, po, nseg);
  else k_decode_combine<bf16, 64><<<g2, 64, 0, s>>>(a, pml, po, nseg);
  return hipGetLastError();
}

}  // namespace dash
