// Backward pass on bf16 MFMA (gfx950 v_mfma_f32_16x16x32_bf16) for bf16 inputs.
//
// Method: the gradient of the three-stage forward taken in reverse (gist.science summary of
// arXiv 2605.18753, "Stufe 1: Entmax-Chunk-Routing", remark on differentiability, and
// "Hauptbeiträge"); the alpha-entmax Jacobian is that of Peters, Niculae and Martins (2019):
// s = p^(2 - alpha) on the support, dx = s (dp - rho), rho = (s . dp) / sum s.
//
// Kernels (launch order):
//   k_bwd_delta     Delta = <dO, O> per (b, head, row).
//   k_bwd_union     per (b, kv head, 64-row block) the OR of its rows' mask words.
//   k_bwd_ksplit    the summaries split into bf16 hi and lo rows, chunk-major (Stage 1's
//                   operands, gathered by chunk).
//   k_bwd_dq_mfma   query-outer, the forward's work unit and union walk: per visit
//                   S^T = K Q^T seeded with bias - lse (so the MFMA returns log2 P),
//                   dP^T = V dO^T, dS = P (dP - Delta), dQ^T += K^T dS^T (K^T read from the
//                   row-major K tile by transposing LDS reads); the routed chunk's
//                   dL/dw_bar = sigma / w_bar * (sum of dS over its keys and the row's heads)
//                   is written by one lane per row.
//   k_bwd_dkdv_mfma chunk-outer: one workgroup per (b, kv head, range of 64 query blocks,
//                   chunk) with 8 waves, two per 16 keys; it walks the range's 64-row query
//                   blocks whose rows route to the chunk (and its own block, causally) in
//                   spans of 64 query vectors staged in LDS, each wave taking 32 of them: S = Q K^T and dP = dO V^T with the
//                   span's rows permuted so that P and dS land in the lanes as the A operands of
//                   dV += P^T dO and dK += dS^T Q, added into fp32 accumulators by atomics.
//                   A span's loads are raw, branch-free buffer loads issued two spans ahead.
//                   Workgroups are dispatched range by range, so the ones in flight share one
//                   range's queries and output gradients through the caches.
//   k_bwd_route_dq  Stage 1, row-outer (the forward router's work unit, 16 query vectors on
//                   8 waves), over the chunks routed to its rows only (listed in LDS): pass 1
//                   recomputes the scores (hi + lo rows) and each head's weights from its saved
//                   tau, z, and reduces sum s and sum s dp into rho; pass 2 recomputes them,
//                   forms dx and adds dq += gamma scale dx K_bar on MFMA (dx straight from the
//                   score registers, K_bar's operand the hi rows transposed through LDS);
//                   writes the final dq and rho.  A tile's operand and dL/dw_bar loads are
//                   issued one tile ahead.
//   k_bwd_route_dk  Stage 1, chunk-outer: one workgroup per (b, kv head, 16 chunks, slice of
//                   8192 query vectors of the later rows); its waves take spans of 32 vectors,
//                   recompute the span's scores as S = Q K_bar^T (rows permuted as in
//                   k_bwd_dkdv_mfma), form dx with the saved rho and add dK_bar += dX^T Q;
//                   waves are summed in LDS and added into dK_bar by atomics.  Each wave
//                   loads its next span while the current one computes.
// Stage 0 backwards and the head_cls reduction use the generic kernels (backward_valu.hip).
#include <algorithm>
#include <type_traits>

#include "route_common.h"

namespace dash {

namespace {

constexpr int kXcdsB = 8;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer descriptor dword 3 (bounds-checked)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kBwdRange = 64;            // query blocks per dK/dV workgroup range
constexpr int kBwdSlice = 8192;          // query vectors per Stage 1 dK_bar workgroup
constexpr int kRouteDqWaves = 8;         // waves per Stage 1 dq workgroup

__device__ __forceinline__ floatx4 mma(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// sum over lanes l, l^16, l^32, l^48 (the four 16-lane rows)
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// sum over the G adjacent lanes of a 16-lane row that hold one row's heads (G a power of 2)
__device__ __forceinline__ float heads_sum(float v, int G) {
  if (G >= 2) v += dppf<0xB1>(v);     // quad_perm [1,0,3,2]
  if (G >= 4) v += dppf<0x4E>(v);     // quad_perm [2,3,0,1]
  if (G >= 8) v += dppf<0x141>(v);    // row_half_mirror
  if (G >= 16) v += dppf<0x140>(v);   // row_mirror
  return v;
}

// XOR swizzle of the 16-byte chunk index inside a row of a [row][D] bf16 LDS tile.  With
// D = 128 (16 chunks per row) row bits 4, 0, 1 and 3 go to chunk bits 0, 1, 2 and 3: the
// 16 rows of a quarter wave's 16-byte operand read differ in row bits 0, 1, 3 and 4, so they
// hit 16 distinct slots, and the 32 lanes of a half wave's transposing 8-byte read
// (ds_read_b64_tr_b16: rows r + 8 lg + k, chunk bit 0 from the column) hit 32 distinct
// 8-byte slots, the column bit landing on chunk bit 0 and the rows on bits 1 to 3.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if (D == 128) return ((row >> 4) & 1) | ((row & 3) << 1) | (((row >> 3) & 1) << 3);
  return ((row >> 1) & 1) | (((row >> 3) & 3) << 1);
}
template <int D>
__device__ __forceinline__ int tile_off(int row, int d) {       // byte offset of (row, d)
  return row * (2 * D) + ((((d >> 3) ^ swz<D>(row))) << 4) + (d & 7) * 2;
}
// 16-byte operand read: row `row`, elements d0 .. d0 + 7 (d0 a multiple of 8)
template <int D>
__device__ __forceinline__ bf16x8 tile_row8(const uint8_t* tile, int row, int d0) {
  return *reinterpret_cast<const bf16x8*>(tile + tile_off<D>(row, d0));
}

typedef short v4i16b __attribute__((ext_vector_type(4)));
typedef short v8i16b __attribute__((ext_vector_type(8)));
// Transposed operand from a row-major [row][D] swizzled tile: lane (l16, lg) receives
// tile[r0 + 8 lg + i][d0 + l16] for i = 0..7, i.e. the 16x16x32 MFMA operand whose 16
// rows/columns are tile columns d0 .. d0 + 15 and whose k-slots are tile rows.  Two
// ds_read_b64_tr_b16: within a 16-lane group source lane 4k + q points at
// tile[r + k][d0 + 4q .. + 3] and output lane i receives tile[r + 0..3][d0 + i].
template <int D>
__device__ __forceinline__ bf16x8 tile_tr8(const uint8_t* tile, int r0, int d0, int lane) {
  const int l16 = lane & 15, lg = lane >> 4;
  const int k = l16 >> 2, q = l16 & 3;
  const int ra = r0 + 8 * lg + k;
  typedef __attribute__((address_space(3))) v4i16b lds_v4;
  const v4i16b x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(tile + tile_off<D>(ra, d0 + 4 * q)));
  const v4i16b y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(tile + tile_off<D>(ra + 4, d0 + 4 * q)));
  const v8i16b r = __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ bf16x8 scale_bf16x8(bf16x8 v, float s) {
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)((float)v[e] * s);
  return v;
}

}  // namespace

// ------------------------------------------------------------------------------ prep
// Delta[b, h, t] = <dO, O>: 16 lanes per row, D / 16 elements each.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_delta(BackwardArgs a, float* __restrict__ delta) {
  constexpr int E = D / 16;
  const size_t rows = (size_t)a.B * a.Hq * a.T;
  const size_t row = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
    const bf16* dp = (const bf16*)a.dout + row * D + l * E;
    const bf16* op = (const bf16*)a.out + row * D + l * E;
#pragma unroll
    for (int e = 0; e < E; ++e) acc = fmaf((float)dp[e], (float)op[e], acc);
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 8);
  if (row < rows && l == 0) delta[row] = acc;
}

// ub[bk][blk][w] = OR over the block's rows t < T of mask[bk][t][w]
__global__ void k_bwd_union(BackwardArgs a, uint64_t* __restrict__ ub, int nblk) {
  const int blk = blockIdx.x, bk = blockIdx.y;
  for (int w = threadIdx.x; w < a.W; w += blockDim.x) {
    uint64_t u = 0;
    const int r1 = min(kChunk, a.T - blk * kChunk);
    for (int r = 0; r < r1; ++r) u |= a.mask[((size_t)bk * a.T + blk * kChunk + r) * a.W + w];
    ub[((size_t)bk * nblk + blk) * a.W + w] = u;
  }
}

// kcm[bk][c][p][d]: the summaries of the complete chunks split as Stage 0 splits them
// (p = 0: bf16(k_bar), p = 1: bf16(k_bar - that)), chunk-major, so that a gathered chunk's
// hi and lo rows are whole cache lines
__global__ void k_bwd_ksplit(BackwardArgs a, bf16* __restrict__ kcm) {
  const int bk = blockIdx.y;
  const int n = (a.T / kChunk) * a.D;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const int c = i / a.D, d = i % a.D;
    const float v = a.summ[((size_t)bk * a.nc + c) * a.D + d];
    const bf16 h = (bf16)v;
    bf16* o = kcm + ((size_t)bk * a.nc + c) * 2 * a.D;
    o[d] = h;
    o[a.D + d] = (bf16)(v - (float)h);
  }
}

// ------------------------------------------------------------------------------ dQ, dw_bar
template <int D, int NW, int RMAX>
__global__ __launch_bounds__(NW * 64) void k_bwd_dq_mfma(BackwardArgs a, const float* __restrict__ delta) {
  constexpr int NT = NW * 64;
  constexpr int KS = D / 32, NDT = D / 16;
  constexpr int TB = 64 * 2 * D;                  // bytes of one 64-row tile
  constexpr int SEGR = D / 8, SEG = 64 * SEGR, PT = SEG / NT;
  static_assert(SEG % NT == 0, "tile segments must divide over the threads");
  constexpr int MAXW = (kMaxRouted + 1 + 63) / 64;
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[2][TB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[2][TB];
  __shared__ uint64_t rowbits[RMAX][MAXW];
  __shared__ uint16_t visit[kMaxRouted + 2];
  __shared__ int woff[MAXW + 1];

  const int G = a.Hq / a.Hkv;
  constexpr int R = RMAX;                          // rows per workgroup = NW * 16 / G
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int T = a.T;
  const int BH = a.B * a.Hkv;
  constexpr int RPB = kChunk / R;
  const int nunits = ((T + kChunk - 1) / kChunk) * BH;
  const int grp = kXcdsB * RPB;
  const int xcd = (blockIdx.x % grp) % kXcdsB, sub = (blockIdx.x % grp) / kXcdsB;
  const int unit = (blockIdx.x / grp) * kXcdsB + xcd;
  if (unit >= nunits) return;
  const int uu = nunits - 1 - unit;
  const int bk = uu % BH;
  const int rt = (uu / BH) * RPB + sub;
  const int b = bk / a.Hkv, kvh = bk % a.Hkv;
  const int row0 = rt * R;
  const int it = row0 / kChunk;
  const int W = a.W;

  // ---- the union walk of the forward
  const int nw_route = (it + 63) / 64;
  for (int idx = tid; idx < R * nw_route; idx += NT) {
    const int r = idx / nw_route, w = idx % nw_route;
    const int t = row0 + r;
    rowbits[r][w] = (t < T) ? a.mask[((size_t)bk * T + t) * W + w] : 0ull;
  }
  __syncthreads();
  if (tid < nw_route) {
    uint64_t u = 0;
    for (int r = 0; r < R; ++r) u |= rowbits[r][tid];
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
    for (int r = 0; r < R; ++r) u |= rowbits[r][tid];
    int o = woff[tid] + 1;
    while (u) {
      visit[o++] = (uint16_t)(64 * tid + __builtin_ctzll(u));
      u &= u - 1;
    }
  }
  if (tid == 0) visit[0] = (uint16_t)it;
  __syncthreads();
  const int nvis = woff[nw_route] + 1;

  // ---- this lane's query column: one 16-column tile per wave
  const int n = 16 * wv + l16, r = n / G, g = n % G;
  const int t = row0 + r;
  const bool qok = t < T;
  const size_t qi = (size_t)(b * a.Hq + kvh * G + g) * T + (qok ? t : 0);
  const float sl2 = a.scale * kLog2e;
  bf16x8 qop[KS], dop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 qv = *reinterpret_cast<const bf16x8*>((const bf16*)a.q + qi * D + 32 * ks + 8 * lg);
    const bf16x8 dv = *reinterpret_cast<const bf16x8*>((const bf16*)a.dout + qi * D + 32 * ks + 8 * lg);
    qop[ks] = qok ? scale_bf16x8(qv, sl2) : bf16x8{};
    dop[ks] = qok ? dv : bf16x8{};
  }
  const float dlt = qok ? delta[qi] : 0.f;
  const float lse2 = qok ? a.lse[qi] * kLog2e : 0.f;
  const int tloc = t & 63;

  // ---- K and V tiles: global -> registers -> LDS (both row-major, swizzled)
  const bf16* kbase = (const bf16*)a.k + (size_t)bk * T * D;
  const bf16* vbase = (const bf16*)a.v + (size_t)bk * T * D;
  int goff[PT], loff[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int seg = tid + i * NT;
    const int row = seg / SEGR, ch = seg % SEGR;
    goff[i] = (row * D + ch * 8) * 2;
    loff[i] = tile_off<D>(row, ch * 8);
  }
  // three register sets: the K/V tiles and the routing weight of visits v + 1 and v + 2 are
  // in flight while visit v computes; every load is unconditional (a visit past the last
  // reads the first visit's chunk with offsets past the range, as zeros), so the compiler's
  // waits are exact
  constexpr int kOob = 0x7ffffff0;
  uint4 kreg[3][PT], vreg[3][PT];
  float wnext[3];
  bool onnext[3];
  auto prefetch = [&](int v_any, auto set_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(set_tag)::value;
    const bool live = v_any < nvis;
    const int c = __builtin_amdgcn_readfirstlane((int)visit[live ? v_any : 0]);
    const int nbytes = min(T - c * kChunk, kChunk) * D * 2;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + (size_t)c * kChunk * D), (short)0, nbytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vbase + (size_t)c * kChunk * D), (short)0, nbytes, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int off = live ? goff[i] : kOob;
      kreg[S][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0));
      vreg[S][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0));
    }
    onnext[S] = (rowbits[r][c >> 6] >> (c & 63)) & 1ull;
    wnext[S] = a.wbar[((size_t)bk * T + (qok ? t : T - 1)) * a.nc + c];
  };
  auto stash = [&](int buf, auto set_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(set_tag)::value;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      *reinterpret_cast<uint4*>(&lds_k[buf][loff[i]]) = kreg[S][i];
      *reinterpret_cast<uint4*>(&lds_v[buf][loff[i]]) = vreg[S][i];
    }
  };
  // a barrier without the fence of __syncthreads, whose release would wait for every load in
  // flight: this wave's LDS writes are waited for explicitly, and the compiler may not move
  // memory operations across it
  auto tile_barrier = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  floatx4 dq[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dq[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto visit_chunk = [&](int buf, int c, float bias2, float wb, auto diag_tag) __attribute__((always_inline)) {
    constexpr bool DIAG = decltype(diag_tag)::value;
    asm volatile("" ::: "memory");
    if (!DIAG && __builtin_amdgcn_ballot_w64(bias2 != -INFINITY) == 0ull) return;
    const uint8_t* kl = lds_k[buf];
    const uint8_t* vl = lds_v[buf];
    const float sd = (DIAG ? 0.f : bias2) - lse2;
    floatx4 sc[4], dpv[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int key = 32 * (kt >> 1) + 8 * (l16 >> 2) + 4 * (kt & 1) + (l16 & 3);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 ka = tile_row8<D>(kl, key, 32 * ks + 8 * lg);
        const bf16x8 va = tile_row8<D>(vl, key, 32 * ks + 8 * lg);
        sc[kt] = mma(ka, qop[ks], ks == 0 ? floatx4{sd, sd, sd, sd} : sc[kt]);
        dpv[kt] = mma(va, dop[ks], ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : dpv[kt]);
      }
    }
    // lane: column q = l16, keys 32 p + 8 lg + 4 half + j for kt = 2 p + half
    float ds[16];
    float dsum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1) + j;
        float x = sc[kt][j];
        if (DIAG && key > tloc) x = -INFINITY;
        const float p = fast_exp2(x);
        const float v = qok ? p * (dpv[kt][j] - dlt) : 0.f;
        ds[4 * kt + j] = v;
        dsum += v;
      }
    bf16x8 dso[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dso[p][j] = (bf16)ds[8 * p + j];
        dso[p][4 + j] = (bf16)ds[8 * p + 4 + j];
      }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int p = 0; p < 2; ++p) dq[dt] = mma(tile_tr8<D>(kl, 32 * p, 16 * dt, lane), dso[p], dq[dt]);
    if (!DIAG) {
      // dL/dw_bar of this row and chunk: dS summed over the chunk's keys and the row's heads
      const float s = heads_sum(rows_sum(dsum), G);
      if (g == 0 && lg == 0 && qok && bias2 != -INFINITY)
        a.dwb[((size_t)bk * T + t) * a.nc + c] = a.sigma * s / wb;
    }
  };

  // visit v: its tiles, loaded into register set v % 3, go to LDS slot v & 1 (which visit
  // v - 2 read before every wave passed visit v - 1's barrier); then the set is refilled with
  // visit v + 3.  Visit 0, the diagonal, is peeled; the later ones go three per round.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  prefetch(0, S0{});
  prefetch(1, S1{});
  prefetch(2, S2{});
  stash(0, S0{});
  tile_barrier();
  prefetch(3, S0{});
  visit_chunk(0, it, 0.f, 0.f, std::true_type{});
  auto step = [&](int v, auto set_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(set_tag)::value;
    const int buf = v & 1;
    stash(buf, set_tag);
    const int c = visit[v < nvis ? v : 0];
    const float wb = wnext[S];
    const float bias2 = onnext[S] ? a.sigma * fast_log2(wnext[S]) : -INFINITY;
    tile_barrier();
    prefetch(v + 3, set_tag);
    if (v < nvis) visit_chunk(buf, c, bias2, wb, std::false_type{});
  };
  for (int v = 1; v < nvis; v += 3) {
    step(v, S1{});
    step(v + 1, S2{});
    step(v + 2, S0{});
  }
  __builtin_amdgcn_s_waitcnt(0);                  // the prefetches past the last visit
  if (qok) {
    float* dst = a.dq32 + qi * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      *reinterpret_cast<float4*>(dst + 16 * dt + 4 * lg) =
          make_float4(a.scale * dq[dt][0], a.scale * dq[dt][1], a.scale * dq[dt][2], a.scale * dq[dt][3]);
  }
}

// Q scaled by sm_scale * log2 e and rounded to bf16, exactly as the forward's Stage 2 uses it,
// for the dK/dV kernel's direct-to-LDS span loads (which cannot scale on the way).
template <int D>
__global__ __launch_bounds__(256) void k_bwd_qscale(BackwardArgs a, bf16* __restrict__ qsc) {
  const float sl2 = a.scale * kLog2e;
  const size_t n8 = (size_t)a.B * a.Hq * a.T * D / 8;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n8;
       i += (size_t)gridDim.x * blockDim.x) {
    const bf16x8 v = reinterpret_cast<const bf16x8*>(a.q)[i];
    reinterpret_cast<bf16x8*>(qsc)[i] = scale_bf16x8(v, sl2);
  }
}

// ------------------------------------------------------------------------------ dK, dV
// One workgroup per (b, kv head, block range, chunk c) with 8 waves: wave w owns keys
// c*64 + 16 (w % 4) + [0, 16) and takes half w / 4 (32 vectors) of every 64-vector span.
template <int D>
__global__ __launch_bounds__(512) void k_bwd_dkdv_mfma(BackwardArgs a, const float* __restrict__ delta,
                                                       const uint64_t* __restrict__ ub, int nblk,
                                                       const bf16* __restrict__ qsc) {
  constexpr int NT = 512, SPAN = 64, NBUF = 4;
  constexpr int KS = D / 32, NDT = D / 16;
  constexpr int SB = SPAN * 2 * D;                // bytes of a span tile
  constexpr int NBLK = SB / 1024 / 8;             // 1 KiB LDS blocks per wave and tile
  static_assert(NBLK >= 1 && SB % (1024 * 8) == 0, "a span tile must split into 1 KiB blocks per wave");
  // the ring's slots are separate arrays, so that the compiler can tell the slot a load is
  // filling from the slot being read and does not wait for the former before the latter
  // (each slot holds the Q tile, then the dO tile)
  __shared__ __attribute__((aligned(16))) uint8_t rs0[2 * SB], rs1[2 * SB], rs2[2 * SB], rs3[2 * SB];
  __shared__ float qinfo[NBUF][4][SPAN];          // lse2, delta, bias2, t (as float)
  __shared__ uint16_t blist[kBwdRange];          // candidate blocks (own first)
  __shared__ uint32_t spanbits[kBwdRange];        // per candidate block: its live spans
  __shared__ uint16_t slist[kBwdRange * 16];      // live spans: block << 4 | span
  __shared__ int nbl_s, nspan_s;

  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int kg = wv & 3, half_q = wv >> 2;        // key group, half of the span
  const int T = a.T;
  const int c = blockIdx.x, rg = blockIdx.y, bk = blockIdx.z;
  const int blo = kBwdRange * rg, bhi = min(nblk, blo + kBwdRange);   // this range's blocks
  if (c >= bhi) return;                           // (whole workgroup)
  const int b = bk / a.Hkv, kvh = bk % a.Hkv;
  const float sl2 = a.scale * kLog2e;

  // ---- query blocks of the range whose rows route to chunk c: its own block first (when
  // in the range), then every later block whose union mask has bit c
  if (wv == 0) {
    const bool own_in = c >= blo;
    int cnt = own_in ? 1 : 0;
    if (lane == 0 && own_in) blist[0] = (uint16_t)c;
    for (int b0 = max(c + 1, blo); b0 < bhi; b0 += 64) {
      const int blk = b0 + lane;
      const bool on = blk < bhi &&
                      ((ub[((size_t)bk * nblk + blk) * a.W + (c >> 6)] >> (c & 63)) & 1ull);
      const uint64_t m = __ballot(on);
      if (on) blist[cnt + __popcll(m & ((1ull << lane) - 1ull))] = (uint16_t)blk;
      cnt += __popcll(m);
    }
    if (lane == 0) nbl_s = cnt;
  }
  __syncthreads();
  const int nbl = nbl_s;
  if (nbl == 0) return;                           // (whole workgroup)
  // ---- live spans: a span is 64 / G rows of a block (times its G heads); it is walked only
  // if one of its rows routes to chunk c (every span of the own block is, causally).  Lane l
  // of a wave reads row l's mask word of a candidate block; waves take the blocks in turn.
  const int rps = kChunk / G;                     // rows per span
  for (int i = wv; i < nbl; i += NT / 64) {
    const int blk = blist[i], tt = blk * kChunk + lane;
    bool on = tt < T;
    if (on && blk != c) on = (a.mask[((size_t)bk * T + tt) * a.W + (c >> 6)] >> (c & 63)) & 1ull;
    const uint64_t rows = __ballot(on);
    uint32_t sb = 0u;
    for (int sp = 0; sp < G; ++sp)
      if ((rows >> (sp * rps)) & (rps == 64 ? ~0ull : ((1ull << rps) - 1ull))) sb |= 1u << sp;
    if (lane == 0) spanbits[i] = sb;
  }
  __syncthreads();
  if (wv == 0) {
    const uint32_t sb = lane < nbl ? spanbits[lane] : 0u;
    const int nmine = __popc(sb);
    int incl = nmine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int x = __shfl_up(incl, o, 64);
      if (lane >= o) incl += x;
    }
    int at = incl - nmine;
    if (lane < nbl) {
      const uint16_t hb = (uint16_t)(blist[lane] << 4);
      for (uint32_t m = sb; m; m &= m - 1) slist[at++] = (uint16_t)(hb | __builtin_ctz(m));
    }
    if (lane == 63) nspan_s = incl;
  }
  __syncthreads();
  const int nspan = nspan_s;                      // live 64-vector spans
  if (nspan == 0) return;                         // (whole workgroup, before any load)

  // ---- this wave's keys as B operands (columns = keys)
  const int kloc = 16 * kg + l16;                 // key within the chunk
  const int key = c * kChunk + kloc;
  const bool kok = key < T;
  bf16x8 kb[KS], vb[KS];
  {
    const bf16* kp = (const bf16*)a.k + ((size_t)bk * T + (kok ? key : 0)) * D;
    const bf16* vp = (const bf16*)a.v + ((size_t)bk * T + (kok ? key : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(kp + 32 * ks + 8 * lg);
      const bf16x8 y = *reinterpret_cast<const bf16x8*>(vp + 32 * ks + 8 * lg);
      kb[ks] = kok ? x : bf16x8{};
      vb[ks] = kok ? y : bf16x8{};
    }
  }

  // ---- span tiles: row m < 64 of span s of block blk is query vector n = 64 s' + m of the
  // block (n = row * G + head).  The Q and dO tiles go from memory straight into a ring of
  // NBUF LDS slots (buffer loads with an LDS destination: lane i of a load fills the 16
  // bytes at the slot's 1 KiB block base + 16 i, so each lane fetches the global 16 bytes
  // that the swizzled layout puts there); Q comes pre-scaled by sm_scale * log2 e and rounded
  // to bf16 as in the forward (k_bwd_qscale).  Spans s + 1 .. s + NBUF - 2 are in flight
  // while span s computes.  The per-row values (lse, delta, the prior bias and the row) go
  // through registers, raw, one set per slot, and are turned into qinfo when the slot is
  // stashed.  Every load is unconditional: a row past T or a span past the end gets an
  // offset past its descriptor's range and reads as zero.
  constexpr int kOob = 0x7ffffff0;
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(qsc + (size_t)(b * a.Hq + kvh * G) * T * D), (short)0, G * T * D * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const bf16*)a.dout + (size_t)(b * a.Hq + kvh * G) * T * D), (short)0, G * T * D * 2,
      kRsrcWord3);
  const int kindw = __builtin_amdgcn_readfirstlane(wv);
  const float* ibase = kindw == 0 ? a.lse + (size_t)(b * a.Hq + kvh * G) * T
                     : kindw == 1 ? delta + (size_t)(b * a.Hq + kvh * G) * T
                                  : a.wbar + (size_t)bk * T * a.nc;
  const int irange = kindw == 2 ? T * a.nc * 4 : (kindw < 2 ? G * T * 4 : 0);
  const __amdgpu_buffer_rsrc_t irs = __builtin_amdgcn_make_buffer_rsrc((void*)ibase, (short)0, irange, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.mask + (size_t)bk * T * a.W), (short)0, kindw == 2 ? T * a.W * 8 : 0, kRsrcWord3);
  // this lane's tile position in each of the wave's NBLK blocks: row and first element
  int drow[NBLK], dcol[NBLK];
#pragma unroll
  for (int j = 0; j < NBLK; ++j) {
    const int byte = (wv * NBLK + j) * 1024 + 16 * lane;
    drow[j] = byte / (2 * D);
    dcol[j] = 8 * (((byte % (2 * D)) >> 4) ^ swz<D>(drow[j]));
  }
  typedef __attribute__((address_space(3))) void lds_void;
  auto qslot = [&](auto set_tag) -> uint8_t* {
    constexpr int S = decltype(set_tag)::value;
    if constexpr (S == 0) return rs0; else if constexpr (S == 1) return rs1;
    else if constexpr (S == 2) return rs2; else return rs3;
  };
  auto oslot = [&](auto set_tag) -> uint8_t* { return qslot(set_tag) + SB; };
  float inf_raw[NBUF];                            // lse / delta / w_bar of this thread's row
  uint32_t inf_bits[NBUF];                        // the mask half-word (kind 2)
  int inf_row[NBUF];                              // the row index t
  bool inf_own[NBUF];                             // the span's block is chunk c's own
  const int lgG = __builtin_ctz(G);               // G is a power of two
  auto prefetch = [&](int s_any, auto set_tag) {
    constexpr int S = decltype(set_tag)::value;
    const bool live = s_any < nspan;
    const int ent = slist[live ? s_any : 0];
    const int blk = ent >> 4, sp = ent & 15;
#pragma unroll
    for (int j = 0; j < NBLK; ++j) {
      const int nn = SPAN * sp + drow[j], tr = blk * kChunk + (nn >> lgG), gg = nn & (G - 1);
      const int off = live && tr < T ? (((gg * T + tr) * D + dcol[j]) * 2) : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lds_void*)(qslot(set_tag) + (wv * NBLK + j) * 1024), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ors, (lds_void*)(oslot(set_tag) + (wv * NBLK + j) * 1024), 16, off, 0, 0, 0);
    }
    asm volatile("" ::: "memory");                // the row values are issued after the tiles
    const int m = tid % SPAN;
    const int nn = SPAN * sp + m, tr = blk * kChunk + (nn >> lgG), gg = nn & (G - 1);
    const bool ok = live && tr < T && tid < 3 * SPAN;
    const int ioff = !ok ? kOob : (kindw == 2 ? (tr * a.nc + c) * 4 : (gg * T + tr) * 4);
    const int moff = !ok ? kOob : (tr * a.W + (c >> 6)) * 8 + ((c & 63) >= 32 ? 4 : 0);
    inf_raw[S] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(irs, ioff, 0, 0));
    inf_bits[S] = __builtin_amdgcn_raw_buffer_load_b32(mrs, moff, 0, 0);
    inf_row[S] = tr;
    inf_own[S] = blk == c;
  };
  // every span issues 2 NBLK tile loads and 2 row-value loads per wave, in that order; before
  // slot S is used, every wave waits until at most the NBUF - 2 younger spans' loads are in
  // flight, i.e. this span's tiles have landed in LDS, and the workgroup meets at a barrier
  constexpr int kLoadsPerSpan = 2 * NBLK + 2;
  constexpr int kWaitN = (NBUF - 2) * kLoadsPerSpan;
  static_assert(kWaitN < 64, "vmcnt holds 6 bits");
  auto stash = [&](auto set_tag) {
    constexpr int S = decltype(set_tag)::value;
    // s_waitcnt vmcnt(kWaitN) with expcnt and lgkmcnt left free (gfx9 encoding)
    __builtin_amdgcn_s_waitcnt((kWaitN & 15) | ((kWaitN >> 4) << 14) | (7 << 4) | (15 << 8));
    if (tid < 4 * SPAN) {
      const int kind = tid / SPAN;
      const int tr = inf_row[S];
      float v;
      if (kind == 0) v = inf_raw[S] * kLog2e;
      else if (kind == 1) v = inf_raw[S];
      else if (kind == 2) {
        if (tr >= T) v = -INFINITY;
        else if (inf_own[S]) v = 0.f;             // the block's own chunk: no prior
        else v = ((inf_bits[S] >> (c & 31)) & 1u) ? a.sigma * fast_log2(inf_raw[S]) : -INFINITY;
      } else v = (float)tr;
      qinfo[S][kind][tid % SPAN] = v;
    }
  };
  // a barrier without the fence of __syncthreads (whose release would wait for every load in
  // flight, the ring's included): LDS writes are waited for explicitly, and the compiler may
  // not move memory operations across it
  auto ring_barrier = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  floatx4 dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    dk[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    dv[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // the ring starts as zeros, so every value a masked row ever reads is finite
  for (int i = tid; i < 2 * SB / 16; i += NT) {
    const uint4 z = make_uint4(0, 0, 0, 0);
    reinterpret_cast<uint4*>(rs0)[i] = z;
    reinterpret_cast<uint4*>(rs1)[i] = z;
    reinterpret_cast<uint4*>(rs2)[i] = z;
    reinterpret_cast<uint4*>(rs3)[i] = z;
  }
  __syncthreads();

  const int r0 = 32 * half_q;                     // this wave's 32 rows of the span tile
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  prefetch(0, S0{});
  prefetch(1, S1{});
  prefetch(2, S2{});
  // span s: slot s % NBUF, whose loads went out NBUF - 1 spans earlier; then the slot that
  // span s - 1 used (every wave finished it before this barrier) is refilled with s + 3
  auto span_step = [&](int s, auto set_tag, auto next_tag) {
    constexpr int SS = decltype(set_tag)::value;
    const int buf = SS;
    stash(set_tag);
    const bool own = (slist[s < nspan ? s : 0] >> 4) == c;
    ring_barrier();
    prefetch(s + NBUF - 1, next_tag);
    if (s >= nspan) return;                       // past the last span (whole workgroup)
    // a wave none of whose 32 rows of the span routes to chunk c has P = dS = 0 there and
    // adds exactly nothing: it skips the span (the block's own chunk is never skipped)
    if (__builtin_amdgcn_ballot_w64(qinfo[buf][2][r0 + (lane & 31)] != -INFINITY) == 0ull) return;
    const uint8_t* ql = qslot(set_tag);
    const uint8_t* ol = oslot(set_tag);
    // S = Q K^T, dP = dO V^T over two halves; half h, A row l16 <- tile row
    // r0 + 8 (l16 / 4) + 4 h + l16 % 4, so lane (l16, lg) holds rows r0 + 8 lg + 4 h + i
    floatx4 sv[2], dpv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = r0 + 8 * (l16 >> 2) + 4 * h + (l16 & 3);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sv[h] = mma(tile_row8<D>(ql, m, 32 * ks + 8 * lg), kb[ks], ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : sv[h]);
        dpv[h] = mma(tile_row8<D>(ol, m, 32 * ks + 8 * lg), vb[ks], ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : dpv[h]);
      }
    }
    bf16x8 pa, dsa;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = r0 + 8 * lg + 4 * h + i;
        float x = sv[h][i] + qinfo[buf][2][m] - qinfo[buf][0][m];
        if (own && kloc > (int)qinfo[buf][3][m] - c * kChunk) x = -INFINITY;
        if (!kok) x = -INFINITY;
        const float p = fast_exp2(x);
        pa[4 * h + i] = (bf16)p;
        dsa[4 * h + i] = (bf16)(p * (dpv[h][i] - qinfo[buf][1][m]));
      }
    // dV += P^T dO, dK += dS^T Q (B operands: the span tiles read transposed)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      dv[dt] = mma(pa, tile_tr8<D>(ol, r0, 16 * dt, lane), dv[dt]);
      dk[dt] = mma(dsa, tile_tr8<D>(ql, r0, 16 * dt, lane), dk[dt]);
    }
  };
  // all four steps run every round (a span past the end only stashes and prefetches), so the
  // loads in flight are the same on every path
  for (int s = 0; s < nspan; s += NBUF) {
    span_step(s, S0{}, S3{});
    span_step(s + 1, S1{}, S0{});
    span_step(s + 2, S2{}, S1{});
    span_step(s + 3, S3{}, S2{});
  }
  // lane holds rows (keys) 16 kg + 4 lg + i, column d = 16 dt + l16.  dK = s sum dS q
  // = ln 2 * sum dS (q sm_scale log2 e).  The second half's waves hand their sums to the
  // first half's through LDS (the span tiles, free once the ring's last loads, past the
  // end, have landed), which add them into the fp32 accumulators.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // [4 key groups][64 lanes][NDT / 2 * 4] floats per tile: d tiles dt < NDT / 2 in slot 0,
  // the others in slot 1 (dK in the Q tiles, dV in the dO tiles)
  constexpr int HD = NDT / 2;
  static_assert(4 * 64 * HD * 4 * 4 <= SB, "hand-over fits two slots");
  auto xk = [&](int dt, int i) -> float& {
    float* base = reinterpret_cast<float*>(dt < HD ? rs0 : rs1);
    return base[(kg * 64 + lane) * HD * 4 + (dt % HD) * 4 + i];
  };
  auto xv = [&](int dt, int i) -> float& {
    float* base = reinterpret_cast<float*>(dt < HD ? rs0 + SB : rs1 + SB);
    return base[(kg * 64 + lane) * HD * 4 + (dt % HD) * 4 + i];
  };
  if (half_q == 1) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xk(dt, i) = dk[dt][i];
        xv(dt, i) = dv[dt][i];
      }
  }
  __syncthreads();
  if (half_q == 1) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kk = c * kChunk + 16 * kg + 4 * lg + i;
    if (kk >= T) continue;
    const size_t ro = ((size_t)bk * T + kk) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const float ok = xk(dt, i);
      const float ov = xv(dt, i);
      atomicAdd(a.dk32 + ro + 16 * dt + l16, kLn2 * (dk[dt][i] + ok));
      atomicAdd(a.dv32 + ro + 16 * dt + l16, dv[dt][i] + ov);
    }
  }
}

// ------------------------------------------------------------------------------ Stage 1
template <int MODE>
__device__ __forceinline__ float jac_s(float p, float alpha) {   // p^(2 - alpha), p > 0
  if (MODE == kAlpha15) return sqrtf(p);
  if (MODE == kAlpha2) return 1.f;
  return pow_pos(p, 2.0f - alpha);
}

// Row-outer: 16 query vectors (R = 16 / G rows of one block) on 8 waves.  Both passes run
// over the chunks routed to any of the R rows only, listed in LDS from the union of their mask
// words: a head's entmax support lies inside its row's routed set, so s and dx vanish outside
// it.  Wave w takes the 16-entry list tiles w, w + 8, ...
template <int D, int MODE, int NW>
__global__ __launch_bounds__(NW * 64) void k_bwd_route_dq(BackwardArgs a, const bf16* __restrict__ kcm,
                                                         float* __restrict__ rho_out) {
  constexpr int NT = NW * 64, KS = D / 32, NDT = D / 16;
  constexpr int MAXW = kMaxRouted / 64;           // mask words of the chunks before a row
  constexpr int XT = 32 * 2 * D;                  // bytes of a wave's 32-row transpose tile
  constexpr int DQS = NW * 16 * (D + 4) * 4;      // bytes of the waves' partial dq
  constexpr int UB = DQS > NW * XT ? DQS : NW * XT;
  __shared__ float part[2][NW][16];
  __shared__ uint64_t rowbits[16][MAXW];
  __shared__ int woff[MAXW + 1];
  __shared__ __attribute__((aligned(16))) uint16_t clist[kMaxRouted + 16];
  __shared__ __attribute__((aligned(16))) uint8_t ubuf[UB];   // transpose tiles, then dq parts
  const int G = a.Hq / a.Hkv;
  const int R = 16 / G;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int T = a.T;
  const int BH = a.B * a.Hkv;
  const int w_id = gridDim.x - 1 - blockIdx.x;    // late (heavy) rows first
  const int rt = w_id / BH, bk = w_id % BH;
  const int b = bk / a.Hkv, kvh = bk % a.Hkv;
  const int row0 = rt * R;
  const int it = row0 / kChunk;                   // the same for all R rows (R divides 64)

  // ---- the list of chunks routed to any of the rows (ascending)
  const int nwr = (it + 63) / 64;
  for (int idx = tid; idx < R * nwr; idx += NT) {
    const int rr = idx / nwr, w = idx % nwr;
    const int tt = row0 + rr;
    uint64_t m = tt < T ? a.mask[((size_t)bk * T + tt) * a.W + w] : 0ull;
    if (w == nwr - 1 && (it & 63) != 0) m &= (1ull << (it & 63)) - 1;
    rowbits[rr][w] = m;
  }
  __syncthreads();
  uint64_t un = 0;
  if (tid < nwr) {
    for (int rr = 0; rr < R; ++rr) un |= rowbits[rr][tid];
    woff[tid + 1] = __popcll(un);
  }
  __syncthreads();
  if (tid == 0) {
    woff[0] = 0;
    for (int w = 0; w < nwr; ++w) woff[w + 1] += woff[w];
  }
  __syncthreads();
  const int ncl = woff[nwr];
  if (tid < nwr) {
    int o = woff[tid];
    while (un) {
      clist[o++] = (uint16_t)(64 * tid + __builtin_ctzll(un));
      un &= un - 1;
    }
  }
  if (tid < 16) clist[ncl + tid] = 0;             // the last tile's tail: chunk 0, weight 0
  __syncthreads();

  const int n = l16, r = n / G, g = n % G;
  const int t = row0 + r;
  const bool qok = t < T;
  const size_t qi = (size_t)(b * a.Hq + kvh * G + g) * T + (qok ? t : 0);
  bf16x8 qop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 qv = *reinterpret_cast<const bf16x8*>((const bf16*)a.q + qi * D + 32 * ks + 8 * lg);
    qop[ks] = qok ? qv : bf16x8{};
  }
  const float gs = a.gamma * a.scale;
  const float zscale = (a.alpha - 1.0f) * gs;
  const float inv = 1.0f / (a.alpha - 1.0f), rG = 1.0f / (float)G;
  const bool act = qok && it > 0;
  const float tau = act ? a.tau[qi] : 0.f;
  const float rz = act ? 1.0f / a.z[qi] : 0.f;
  const int ntile = (ncl + 15) / 16;
  const int nj = ntile > wv ? (ntile - wv + NW - 1) / NW : 0;

  // A tile's loads (this wave's tiles wv, wv + NW, ...): the hi and lo summary rows of its 16
  // listed chunks from the chunk-major split copy, and the lane's four dL/dw_bar values, all as
  // buffer loads issued together and without branches (a tile past the wave's last one reads
  // as zero), so the loads of the next tile are in flight while this one is evaluated.
  constexpr int kOob = 0x7ffffff0;
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kcm + (size_t)bk * a.nc * 2 * D), (short)0, a.nc * 2 * D * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.dwb + (size_t)bk * T * a.nc), (short)0, T * a.nc * 4, kRsrcWord3);
  const int trow = qok ? t : 0;
  struct TileLoads {
    bf16x8 hi[KS], lo[KS];
    uint32_t cc[2];                               // the lane's four chunk ids, 16 bits each
    float dw[4];
  };
  auto chunk_of = [](const TileLoads& L, int i) { return (int)((L.cc[i >> 1] >> (16 * (i & 1))) & 0xffffu); };
  auto load_tile = [&](int j, TileLoads& L) __attribute__((always_inline)) {
    const int ct = wv + NW * j;
    const bool live = j < nj;
    const int crow = clist[live ? 16 * ct + l16 : 0];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      L.hi[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                     crs, live ? (2 * crow * D + 32 * ks + 8 * lg) * 2 : kOob, 0, 0));
      L.lo[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                     crs, live ? ((2 * crow + 1) * D + 32 * ks + 8 * lg) * 2 : kOob, 0, 0));
    }
    const int p0 = 16 * ct + 4 * lg;              // the lane's list entries p0 .. p0 + 3
    const uint2 cc = *reinterpret_cast<const uint2*>(&clist[live ? p0 : 0]);
    L.cc[0] = cc.x;
    L.cc[1] = cc.y;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      L.dw[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                    wrs, live && act && p0 + i < ncl ? (trow * a.nc + chunk_of(L, i)) * 4 : kOob, 0, 0));
  };
  // s and dp of the lane's 4 list entries of a loaded tile
  auto eval_tile = [&](int j, const TileLoads& L, float (&s4)[4], float (&dp4)[4]) __attribute__((always_inline)) {
    const int ct = wv + NW * j;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      acc = mma(L.hi[ks], qop[ks], acc);
      acc = mma(L.lo[ks], qop[ks], acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s4[i] = 0.f;
      dp4[i] = 0.f;
      if (act && j < nj && 16 * ct + 4 * lg + i < ncl) {
        const float p = entmax_weight<MODE>(zscale * acc[i], tau, inv, rz);
        if (p > 0.f) {
          const int c = chunk_of(L, i);
          s4[i] = jac_s<MODE>(p, a.alpha);
          dp4[i] = ((rowbits[r][c >> 6] >> (c & 63)) & 1ull) ? L.dw[i] * rG : 0.f;
        }
      }
    }
  };
  // ---- pass 1: sum s and sum s dp per query vector
  float ss = 0.f, sd = 0.f;
  {
    TileLoads A, B;
    load_tile(0, A);
    for (int j = 0; j < nj; j += 2) {
      float s4[4], dp4[4];
      load_tile(j + 1, B);
      eval_tile(j, A, s4, dp4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ss += s4[i];
        sd = fmaf(s4[i], dp4[i], sd);
      }
      load_tile(j + 2, A);
      eval_tile(j + 1, B, s4, dp4);               // zeros past the last tile
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ss += s4[i];
        sd = fmaf(s4[i], dp4[i], sd);
      }
    }
  }
  ss = rows_sum(ss);
  sd = rows_sum(sd);
  if (lg == 0) {
    part[0][wv][l16] = ss;
    part[1][wv][l16] = sd;
  }
  __syncthreads();
  float sst = 0.f, sdt = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    sst += part[0][w][l16];
    sdt += part[1][w][l16];
  }
  const float rho = sst > 0.f ? sdt / sst : 0.f;
  if (wv == 0 && lg == 0 && qok) rho_out[qi] = rho;
  // ---- pass 2: dx, and dq += gs * dX K_bar over pairs of tiles (k-slots i < 4: tile j, list
  // entries 16 ta + 4 lg + i; i >= 4: tile j + 1, entries 16 tb + 4 lg + i - 4).  K_bar's operand
  // is the pair's hi rows, already in registers for the scores, written into this wave's LDS
  // tile in that k-slot order (entry p of tile j at row 8 (p >> 2) + (p & 3), of tile j + 1 four
  // rows further) and read back transposed.
  floatx4 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  uint8_t* xt = ubuf + wv * XT;
  const int xrow = 8 * (l16 >> 2) + (l16 & 3);
  {
    TileLoads A, B;
    load_tile(0, A);
    for (int j = 0; j < nj; j += 2) {
      bf16x8 xa;
      float s4[4], dp4[4];
      load_tile(j + 1, B);
      eval_tile(j, A, s4, dp4);
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = (bf16)(gs * s4[i] * (dp4[i] - rho));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        *reinterpret_cast<bf16x8*>(xt + tile_off<D>(xrow, 32 * ks + 8 * lg)) = A.hi[ks];
      load_tile(j + 2, A);
      eval_tile(j + 1, B, s4, dp4);               // zeros past the last tile
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[4 + i] = (bf16)(gs * s4[i] * (dp4[i] - rho));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        *reinterpret_cast<bf16x8*>(xt + tile_off<D>(xrow + 4, 32 * ks + 8 * lg)) = B.hi[ks];
      // the transposing reads are not ordered behind the wave's outstanding LDS writes
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] = mma(xa, tile_tr8<D>(xt, 0, 16 * dt, lane), acc[dt]);
    }
  }
  __syncthreads();                                // every wave is done with its transpose tile
  // lane: C[4 lg + i][l16] = (query vector 4 lg + i, d = 16 dt + l16); sum the waves in LDS
  float (*dqs)[16][D + 4] = reinterpret_cast<float (*)[16][D + 4]>(ubuf);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) dqs[wv][4 * lg + i][16 * dt + l16] = acc[dt][i];
  __syncthreads();
  for (int idx = tid; idx < 16 * D; idx += NT) {
    const int nn = idx / D, d = idx % D;
    const int rr = nn / G, gg = nn % G, tt = row0 + rr;
    if (tt >= T) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += dqs[w][nn][d];
    const size_t o = ((size_t)(b * a.Hq + kvh * G + gg) * T + tt) * D + d;
    ((bf16*)a.dq)[o] = (bf16)(a.dq32[o] + v);
  }
}

// Chunk-outer: one workgroup per (b, kv head, 16-chunk tile ct, slice of kBwdSlice query
// vectors n = (t - t0) G + head of the rows t >= t0 = 64 (16 ct + 1)); 8 waves take spans of
// 32 vectors.  dK_bar (16 chunks x D) of each wave is summed in LDS and added by atomics.
template <int D, int MODE>
__global__ __launch_bounds__(512) void k_bwd_route_dk(BackwardArgs a, const float* __restrict__ rho) {
  constexpr int NW = 8, KS = D / 32, NDT = D / 16;
  constexpr int SB = 32 * 2 * D;
  __shared__ __attribute__((aligned(16))) uint8_t lq[NW][SB];
  __shared__ float info[NW][32][4];               // tau, z, rho, mask half-word per span row
  __shared__ float red[16][D + 4];
  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int T = a.T;
  const int ct = blockIdx.x, sl = blockIdx.y, bk = blockIdx.z;
  const int b = bk / a.Hkv, kvh = bk % a.Hkv;
  const float gs = a.gamma * a.scale;
  const float zscale = (a.alpha - 1.0f) * gs;
  const float inv = 1.0f / (a.alpha - 1.0f), rG = 1.0f / (float)G;
  const int c = 16 * ct + l16;                    // this lane's chunk (B column)
  // rows that may route to this tile: t >= 64 (16 ct + 1), as query vectors
  // n = (t - t0) G + head; this workgroup takes n in [sl * kBwdSlice, + kBwdSlice)
  const int t0 = kChunk * (16 * ct + 1);
  const long long nq_all = t0 < a.T ? (long long)(a.T - t0) * G : 0;
  const long long nlo = (long long)sl * kBwdSlice;
  if (nlo >= nq_all) return;                      // (whole workgroup)
  const bool cok = c < a.nc;
  // B operands: K_bar^T columns = chunks (hi and lo planes of the split summaries)
  const bf16* sp = a.ssplit + (size_t)bk * split_bk_stride(a.nc, D);
  bf16x8 khi[KS], klo[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    khi[ks] = *reinterpret_cast<const bf16x8*>(sp + split_offset(c, 0, 32 * ks + 8 * lg, D));
    klo[ks] = *reinterpret_cast<const bf16x8*>(sp + split_offset(c, 1, 32 * ks + 8 * lg, D));
    if (!cok) { khi[ks] = bf16x8{}; klo[ks] = bf16x8{}; }
  }
  const long long nq = nq_all;
  const int nspan = (int)((min(nq_all - nlo, (long long)kBwdSlice) + 31) / 32);
  floatx4 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  uint8_t* myq = lq[wv];
  float* myinfo = &info[wv][0][0];

  // Per-wave software pipeline over the wave's spans s = wv, wv + NW, ...: the next span's
  // query rows, per-row thresholds, normalisers, rho, mask half-word and this lane's dL/dw_bar
  // values are loaded (raw bits, through buffer descriptors; anything past the end or past the
  // rows reads as zero) while the current span computes.  Query vector n of the slice is row
  // t0 + n / G, head n % G (G a power of two).
  constexpr int kOob = 0x7ffffff0;
  constexpr int QPL = 32 * (D / 8) / 64;          // 16-byte query segments per lane per span
  const int lgG = __builtin_ctz(G);
  const size_t hbase = (size_t)(b * a.Hq + kvh * G) * T;   // first row of this kv head's heads
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const bf16*)a.q + hbase * D), (short)0, G * T * D * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.tau + hbase), (short)0, G * T * 4, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.z + hbase), (short)0, G * T * 4, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc((void*)(rho + hbase), (short)0, G * T * 4, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.mask + (size_t)bk * T * a.W), (short)0, T * a.W * 8, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.dwb + (size_t)bk * T * a.nc), (short)0, T * a.nc * 4, kRsrcWord3);
  const int cb = 16 * ct;                         // the tile's chunks share one mask half-word
  const int mhalf = (cb & 63) >= 32 ? 4 : 0;
  uint4 qn[QPL];
  float inf_n[3];
  uint32_t mw_n;
  float dw_n[8];
  auto load_span = [&](int s) {
    const bool live = s < nspan;
    const long long n0 = nlo + (long long)s * 32;
#pragma unroll
    for (int j = 0; j < QPL; ++j) {
      const int i = lane + 64 * j, m = i / (D / 8), d0 = (i % (D / 8)) * 8;
      const long long nn = n0 + m;
      const bool ok = live && nn < nq;
      const int tt = t0 + (int)(nn >> lgG), gg = (int)(nn & (G - 1));
      qn[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            qrs, ok ? ((gg * T + tt) * D + d0) * 2 : kOob, 0, 0));
    }
    {
      const int m = lane & 31;
      const long long nn = n0 + m;
      const bool ok = live && nn < nq && lane < 32;
      const int tt = t0 + (int)(nn >> lgG), gg = (int)(nn & (G - 1));
      const int ro = ok ? (gg * T + tt) * 4 : kOob;
      inf_n[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(trs, ro, 0, 0));
      inf_n[1] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(zrs, ro, 0, 0));
      inf_n[2] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rrs, ro, 0, 0));
      mw_n = __builtin_amdgcn_raw_buffer_load_b32(mrs, ok ? (tt * a.W + (cb >> 6)) * 8 + mhalf : kOob, 0, 0);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long long nn = n0 + 8 * lg + 4 * h + i;
        const bool ok = live && nn < nq && cok;
        const int tt = t0 + (int)(nn >> lgG);
        dw_n[4 * h + i] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(wrs, ok ? (tt * a.nc + c) * 4 : kOob, 0, 0));
      }
  };

  load_span(wv);
  for (int s = wv; s < nspan; s += NW) {
    // stash: the span's query rows in this wave's LDS tile (row m <- vector n0 + m) and its
    // per-row values; this lane's dL/dw_bar values stay in registers
#pragma unroll
    for (int j = 0; j < QPL; ++j) {
      const int i = lane + 64 * j, m = i / (D / 8), d0 = (i % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(myq + tile_off<D>(m, d0)) = qn[j];
    }
    if (lane < 32) {
      myinfo[lane * 4 + 0] = inf_n[0];
      myinfo[lane * 4 + 1] = inf_n[1];
      myinfo[lane * 4 + 2] = inf_n[2];
      myinfo[lane * 4 + 3] = __builtin_bit_cast(float, mw_n);
    }
    float dw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) dw[e] = dw_n[e];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    load_span(s + NW);                            // the wave's next span (or nothing)
    const long long n0 = nlo + (long long)s * 32;
    // S = Q K_bar^T with span rows permuted (lane holds rows 8 lg + 4 h + i of column c)
    floatx4 sv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = 8 * (l16 >> 2) + 4 * h + (l16 & 3);
      sv[h] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 qa = tile_row8<D>(myq, m, 32 * ks + 8 * lg);
        sv[h] = mma(qa, khi[ks], sv[h]);
        sv[h] = mma(qa, klo[ks], sv[h]);
      }
    }
    bf16x8 xa;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 8 * lg + 4 * h + i;
        const long long nn = n0 + m;
        float dx = 0.f;
        if (nn < nq && cok) {
          const int tt = t0 + (int)(nn >> lgG);
          if (c < tt / kChunk) {
            const float tau = myinfo[m * 4 + 0], zz = myinfo[m * 4 + 1], rh = myinfo[m * 4 + 2];
            const uint32_t mw = __builtin_bit_cast(uint32_t, myinfo[m * 4 + 3]);
            const float p = entmax_weight<MODE>(zscale * sv[h][i], tau, inv, 1.0f / zz);
            if (p > 0.f) {
              const bool on = (mw >> (c & 31)) & 1u;
              const float dp = on ? dw[4 * h + i] * rG : 0.f;
              dx = gs * jac_s<MODE>(p, a.alpha) * (dp - rh);
            }
          }
        }
        xa[4 * h + i] = (bf16)dx;
      }
    // dK_bar (chunks x d) += dX^T Q: A = dX^T (row = chunk l16, k-slots = span rows),
    // B = Q read transposed from the span tile
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = mma(xa, tile_tr8<D>(myq, 0, 16 * dt, lane), acc[dt]);
    __builtin_amdgcn_wave_barrier();
  }
  // sum the waves: C[4 lg + i][l16] = (chunk 16 ct + 4 lg + i, d = 16 dt + l16)
  for (int w = 0; w < NW; ++w) {
    if (wv == w) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float& dst = red[4 * lg + i][16 * dt + l16];
          dst = (w == 0) ? acc[dt][i] : dst + acc[dt][i];
        }
    }
    __syncthreads();
  }
  for (int idx = tid; idx < 16 * D; idx += 512) {
    const int cc = 16 * ct + idx / D, d = idx % D;
    if (cc < a.nc) atomicAdd(a.dsumm + ((size_t)bk * a.nc + cc) * D + d, red[idx / D][d]);
  }
}

// ------------------------------------------------------------------------------ launcher
int backward_mfma_scratch(int B, int Hq, int Hkv, int T, int D, size_t* off_delta, size_t* off_ub,
                          size_t* off_kcm, size_t* off_rho, size_t* off_qsc, size_t* total) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const int nc = (T + kChunk - 1) / kChunk, W = (nc + 63) / 64;
  size_t o = 0;
  *off_delta = o;
  o += al((size_t)B * Hq * T * 4);
  *off_ub = o;
  o += al((size_t)B * Hkv * nc * W * 8);
  *off_kcm = o;                                   // chunk-major split summaries
  o += al((size_t)B * Hkv * nc * 2 * D * 2);
  *off_rho = o;
  o += al((size_t)B * Hq * T * 4);
  *off_qsc = o;                                   // Q pre-scaled for the dK/dV span loads
  o += al((size_t)B * Hq * T * D * 2);
  *total = o;
  return 0;
}

template <int D>
static hipError_t launch_backward_mfma_t(const BackwardArgs& a, char* scratch, hipStream_t s) {
  size_t od, ou, ok, orho, oqs, tot;
  backward_mfma_scratch(a.B, a.Hq, a.Hkv, a.T, a.D, &od, &ou, &ok, &orho, &oqs, &tot);
  bf16* qsc = reinterpret_cast<bf16*>(scratch + oqs);
  float* delta = reinterpret_cast<float*>(scratch + od);
  uint64_t* ub = reinterpret_cast<uint64_t*>(scratch + ou);
  bf16* kcm = reinterpret_cast<bf16*>(scratch + ok);
  float* rho = reinterpret_cast<float*>(scratch + orho);
  const int G = a.Hq / a.Hkv;
  const int BH = a.B * a.Hkv;
  const int nblk = a.nc;                          // 64-row query blocks = chunks
  const size_t rows = (size_t)a.B * a.Hq * a.T;
  k_bwd_delta<D><<<(unsigned)((rows + 15) / 16), 256, 0, s>>>(a, delta);
  k_bwd_union<<<dim3(nblk, BH), 64, 0, s>>>(a, ub, nblk);
  k_bwd_ksplit<<<dim3(64, BH), 256, 0, s>>>(a, kcm);
  // dQ (Stage 2's part) and dw_bar
  {
    const int NW = G >= 2 ? 8 : 4;
    const int R = NW * 16 / G;
    const int nunits = nblk * BH;
    dim3 grid(((nunits + kXcdsB - 1) / kXcdsB) * kXcdsB * (kChunk / R));
    switch (G) {
      case 16: k_bwd_dq_mfma<D, 8, 8><<<grid, 512, 0, s>>>(a, delta); break;
      case 8: k_bwd_dq_mfma<D, 8, 16><<<grid, 512, 0, s>>>(a, delta); break;
      case 4: k_bwd_dq_mfma<D, 8, 32><<<grid, 512, 0, s>>>(a, delta); break;
      case 2: k_bwd_dq_mfma<D, 8, 64><<<grid, 512, 0, s>>>(a, delta); break;
      default: k_bwd_dq_mfma<D, 4, 64><<<grid, 256, 0, s>>>(a, delta); break;
    }
  }
  // dK (Stage 2's part) and dV, from Q pre-scaled as the forward used it
  {
    const size_t n8 = rows * D / 8;
    const unsigned gq = (unsigned)std::min<size_t>((n8 + 255) / 256, 8192);
    k_bwd_qscale<D><<<gq, 256, 0, s>>>(a, qsc);
  }
  k_bwd_dkdv_mfma<D><<<dim3(a.nc, (nblk + kBwdRange - 1) / kBwdRange, BH), 512, 0, s>>>(a, delta, ub, nblk, qsc);
  // Stage 1: dq (final) and rho, then dK_bar
  {
    const int R = 16 / G;
    dim3 grid((unsigned)(((a.T + R - 1) / R) * BH));
    const int ntc = (a.nc + 15) / 16;
    const int nsl = (int)(((long long)a.T * G + kBwdSlice - 1) / kBwdSlice);
    if (a.alpha == 1.5f) {
      k_bwd_route_dq<D, kAlpha15, kRouteDqWaves><<<grid, kRouteDqWaves * 64, 0, s>>>(a, kcm, rho);
      k_bwd_route_dk<D, kAlpha15><<<dim3(ntc, nsl, BH), 512, 0, s>>>(a, rho);
    } else if (a.alpha == 2.0f) {
      k_bwd_route_dq<D, kAlpha2, kRouteDqWaves><<<grid, kRouteDqWaves * 64, 0, s>>>(a, kcm, rho);
      k_bwd_route_dk<D, kAlpha2><<<dim3(ntc, nsl, BH), 512, 0, s>>>(a, rho);
    } else {
      k_bwd_route_dq<D, kAlphaGeneral, kRouteDqWaves><<<grid, kRouteDqWaves * 64, 0, s>>>(a, kcm, rho);
      k_bwd_route_dk<D, kAlphaGeneral><<<dim3(ntc, nsl, BH), 512, 0, s>>>(a, rho);
    }
  }
  return hipGetLastError();
}

hipError_t launch_backward_mfma(const BackwardArgs& a, void* scratch, hipStream_t s) {
  return a.D == 128 ? launch_backward_mfma_t<128>(a, (char*)scratch, s)
                    : launch_backward_mfma_t<64>(a, (char*)scratch, s);
}

}  // namespace dash
