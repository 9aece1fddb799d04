// C ABI of libdash: argument validation, workspace planning and kernel dispatch.
//
// Validation is plain host C++ and runs before any HIP call, so every error path can be
// exercised without a GPU.  The library owns no device memory: callers pass workspaces
// sized by the *_workspace_size() queries.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/dash.h"
#include "dash_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return DASH_OK;
}

constexpr int kMaxT = dash::kChunk * (dash::kMaxRouted + 1);

struct Dims {
  int B, Hq, Hkv, T, D, G, nc, nfull, W;
  float scale, alpha, gamma, sigma;
  int dtype;
  size_t es;
};

int check_params(const dash_params* p, Dims* d, bool need_bf16 = false) {
  if (!p) return fail(DASH_ERR_INVALID_ARG, "params is NULL");
  if (p->dtype != DASH_BF16 && p->dtype != DASH_FP32)
    return fail(DASH_ERR_DTYPE, "unknown dtype %d", p->dtype);
  if (p->B <= 0 || p->Hq <= 0 || p->Hkv <= 0)
    return fail(DASH_ERR_INVALID_ARG, "B, Hq, Hkv must be positive (got %d, %d, %d)", p->B,
                p->Hq, p->Hkv);
  if (p->T <= 0) return fail(DASH_ERR_INVALID_ARG, "T must be positive (got %d)", p->T);
  if (p->Hq % p->Hkv != 0)
    return fail(DASH_ERR_SHAPE, "Hq (%d) is not a multiple of Hkv (%d)", p->Hq, p->Hkv);
  if (!p->enable_gqa && p->Hq != p->Hkv)
    return fail(DASH_ERR_SHAPE, "Hq != Hkv needs enable_gqa");
  const int G = p->Hq / p->Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(DASH_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4, 8 or 16 (got %d)", G);
  if (p->D != 64 && p->D != 128)
    return fail(DASH_ERR_UNSUPPORTED, "head dim must be 64 or 128 (got %d)", p->D);
  if (p->chunk_size != dash::kChunk)
    return fail(DASH_ERR_UNSUPPORTED, "chunk_size must be 64 (got %d)", p->chunk_size);
  if (!(p->alpha > 1.0f) || !std::isfinite(p->alpha))
    return fail(DASH_ERR_INVALID_ARG, "alpha must be finite and > 1");
  if (!(p->gamma > 0.0f) || !std::isfinite(p->gamma))
    return fail(DASH_ERR_INVALID_ARG, "gamma must be finite and > 0");
  if (p->topk < 0) return fail(DASH_ERR_INVALID_ARG, "topk must be >= 0 (got %d)", p->topk);
  if (!(p->sigma >= 0.0f) || !std::isfinite(p->sigma))
    return fail(DASH_ERR_INVALID_ARG, "sigma (prior strength) must be finite and >= 0");
  if (!std::isfinite(p->sm_scale)) return fail(DASH_ERR_INVALID_ARG, "sm_scale is not finite");
  if (p->T > kMaxT)
    return fail(DASH_ERR_UNSUPPORTED, "T=%d exceeds %d (at most %d routed chunks per row)", p->T,
                kMaxT, dash::kMaxRouted);
  if (need_bf16 && p->dtype != DASH_BF16) return fail(DASH_ERR_DTYPE, "this entry point is bf16 only");
  d->B = p->B;
  d->Hq = p->Hq;
  d->Hkv = p->Hkv;
  d->T = p->T;
  d->D = p->D;
  d->G = G;
  d->nc = (p->T + dash::kChunk - 1) / dash::kChunk;
  d->nfull = p->T / dash::kChunk;
  d->W = (d->nc + 63) / 64;
  d->scale = p->sm_scale > 0.f ? p->sm_scale : 1.0f / std::sqrt((float)p->D);
  d->alpha = p->alpha;
  d->gamma = p->gamma;
  d->sigma = p->sigma;
  d->dtype = p->dtype;
  d->es = p->dtype == DASH_BF16 ? 2 : 4;
  return DASH_OK;
}

int check_ptr(const void* ptr, const char* name, bool required = true) {
  if (!ptr) return required ? fail(DASH_ERR_INVALID_ARG, "%s is NULL", name) : DASH_OK;
  if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
    return fail(DASH_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return DASH_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------- prefill workspace
struct PrefillLayout {
  size_t summ, ssplit, vt, mask, wbar, ydiag, total;
};

PrefillLayout prefill_layout(const Dims& d) {
  PrefillLayout L;
  size_t off = 0;
  L.summ = off;
  off += align256((size_t)d.B * d.Hkv * d.nc * d.D * 4);
  L.ssplit = off;
  off += d.dtype == DASH_BF16 ? align256((size_t)d.B * d.Hkv * dash::split_bk_stride(d.nc, d.D) * 2) : 0;
  L.vt = off;
  off += d.dtype == DASH_BF16 ? align256((size_t)d.B * d.Hkv * d.nc * d.D * 64 * 2) : 0;
  L.mask = off;
  off += align256((size_t)d.B * d.Hkv * d.T * d.W * 8);
  L.wbar = off;
  off += align256((size_t)d.B * d.Hkv * d.T * d.nc * 4);
  L.ydiag = off;   // estimate_diagonal: the own chunk's Stage 1 score per (b, head, row)
  off += d.dtype == DASH_BF16 ? align256((size_t)d.B * d.Hq * d.T * 4) : 0;
  L.total = off;
  return L;
}

struct DecodeLayout {
  size_t mask, wbar, list, sco, pml, po, segsz, total;
};

DecodeLayout decode_layout(const Dims& d) {
  DecodeLayout L;
  size_t off = 0;
  L.mask = off;
  off += align256((size_t)d.B * d.Hkv * d.W * 8);
  L.wbar = off;
  off += align256((size_t)d.B * d.Hkv * d.nc * 4);
  L.list = off;
  off += align256((size_t)d.B * d.Hkv * (d.nc + 2) * 4);
  L.sco = off;
  off += d.dtype == DASH_BF16 ? align256((size_t)d.B * d.Hq * (16 * ((d.nc + 15) / 16)) * 4) : 0;
  const size_t nseg = (size_t)dash::decode_nseg_max(d.nc);
  L.pml = off;
  off += d.dtype == DASH_BF16 ? align256((size_t)d.B * d.Hkv * nseg * 32 * 4) : 0;
  L.po = off;
  off += d.dtype == DASH_BF16 ? align256((size_t)d.B * d.Hkv * nseg * 16 * d.D * 4) : 0;
  L.segsz = off;
  off += d.dtype == DASH_BF16 ? 256 : 0;
  L.total = off;
  return L;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return DASH_OK;
  if (!ws) return fail(DASH_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(DASH_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if (have < need)
    return fail(DASH_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", have, need);
  return DASH_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DASH_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

__global__ void k_fill_f32(float* p, size_t n, float v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t fill_f32(float* p, size_t n, float v, hipStream_t s) {
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) return hipSuccess;
  k_fill_f32<<<(unsigned)blocks, 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

// Fixed device scratch for dash_decode_noalloc: one copy per GPU, alive until the process
// ends.  Host code never passes this name to a kernel (on the host it is only a stand-in for
// the symbol); it uses the device address that hipGetSymbolAddress returns for the current
// device, looked up once per device.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (nullptr and a message on failure).
void* scratch_address(int* status) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *status = fail(DASH_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = fail(DASH_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
    return nullptr;
  }
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *status = fail(DASH_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);   // same value from any thread
  }
  *status = DASH_OK;
  return ptr;
}

}  // namespace

extern "C" {

int dash_abi_version(void) { return 105; }

const char* dash_last_error(void) { return g_err.c_str(); }

int dash_prefill_workspace_size(const dash_params* p, size_t* bytes) {
  Dims d;
  if (int rc = check_params(p, &d)) return rc;
  if (!bytes) return fail(DASH_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = prefill_layout(d).total;
  return ok();
}

static int prefill_impl(const dash_params* p, int stages, const void* q, const void* k,
                        const void* v, const void* head_cls, void* out,
                        uint64_t* active_blocks, float* block_weights, float* summary_out,
                        void* workspace, size_t workspace_bytes, void* stream,
                        float* lse = nullptr) {
  Dims d;
  if (int rc = check_params(p, &d)) return rc;
  if (p->topk > 0 && d.dtype != DASH_BF16)
    return fail(DASH_ERR_UNSUPPORTED, "the top-k comparison router is built for bf16 only");
  if (p->estimate_diagonal != 0) {
    if (p->topk > 0)
      return fail(DASH_ERR_UNSUPPORTED, "estimate_diagonal=1 applies to the entmax router only");
    if (d.T > dash::kChunk * dash::kMaxRouted)
      return fail(DASH_ERR_UNSUPPORTED, "estimate_diagonal=1: T=%d exceeds %d", d.T,
                  dash::kChunk * dash::kMaxRouted);
  }
  if (int rc = check_ptr(q, "q")) return rc;
  if (int rc = check_ptr(k, "k")) return rc;
  if (int rc = check_ptr(v, "v")) return rc;
  if (int rc = check_ptr(head_cls, "head_cls")) return rc;
  if (int rc = check_ptr(out, "out")) return rc;
  if (int rc = check_ptr(active_blocks, "active_blocks", false)) return rc;
  if (int rc = check_ptr(block_weights, "block_weights", false)) return rc;
  if (int rc = check_ptr(summary_out, "summary_out", false)) return rc;
  const PrefillLayout L = prefill_layout(d);
  if (int rc = check_ws(workspace, workspace_bytes, L.total)) return rc;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* summ = summary_out ? summary_out : reinterpret_cast<float*>(ws + L.summ);
  uint64_t* mask = active_blocks ? active_blocks : reinterpret_cast<uint64_t*>(ws + L.mask);
  float* wbar = block_weights ? block_weights : reinterpret_cast<float*>(ws + L.wbar);
  hipError_t e;

  if (stages & 1) {
    void* ss = d.dtype == DASH_BF16 ? (void*)(ws + L.ssplit) : nullptr;
    if ((e = dash::launch_stage0(k, head_cls, summ, ss, d.B, d.Hkv, d.T, d.D, d.nc, d.nfull,
                                 nullptr, nullptr, d.scale, d.dtype, s)) != hipSuccess)
      return hip_fail(e, "stage 0 launch");
  }
  if ((stages & 8) && d.dtype == DASH_BF16) {
    if ((e = dash::launch_vtranspose(v, ws + L.vt, d.B, d.Hkv, d.T, d.D, d.nc, s)) != hipSuccess)
      return hip_fail(e, "V transpose launch");
  }
  if ((stages & 2) && block_weights) {
    if ((e = fill_f32(block_weights, (size_t)d.B * d.Hkv * d.T * d.nc, 0.f, s)) != hipSuccess)
      return hip_fail(e, "clearing block_weights");
  }

  dash::RouteArgs ra{};
  ra.q = q;
  ra.summ = summ;
  ra.mask = mask;
  ra.wbar = wbar;
  ra.seq_lens = nullptr;
  ra.B = d.B;
  ra.Hq = d.Hq;
  ra.Hkv = d.Hkv;
  ra.D = d.D;
  ra.Tq = d.T;
  ra.rows = d.T;
  ra.nc_alloc = d.nc;
  ra.W = d.W;
  ra.wbar_ld = d.nc;
  ra.tcap = d.T;
  ra.alpha = d.alpha;
  ra.zscale = (d.alpha - 1.0f) * d.gamma * d.scale;
  ra.topk = p->topk;
  ra.dtype = d.dtype;
  if (p->estimate_diagonal != 0) {
    ra.kdiag = k;
    ra.head_cls = head_cls;
    ra.kdiag_ld = d.T;
    ra.s0_scale_log2 = d.scale * 1.4426950408889634f;
  }
  if (stages & 2) {
    if (d.dtype == DASH_BF16) {
      if (p->estimate_diagonal != 0) {
        float* yd = reinterpret_cast<float*>(ws + L.ydiag);
        if ((e = dash::launch_diag_scores(k, head_cls, q, yd, d.B, d.Hq, d.Hkv, d.T, d.D, d.nc,
                                          d.scale, ra.zscale, s)) != hipSuccess)
          return hip_fail(e, "diagonal score launch");
        ra.ydiag = yd;
      }
      e = dash::launch_route_mfma(ra, ws + L.ssplit, s);
    } else {
      e = dash::launch_route_valu(ra, s);
    }
    if (e != hipSuccess) return hip_fail(e, "stage 1 launch");
  }
  if (!(stages & 4)) return ok();

  dash::AttendArgs aa{};
  aa.q = q;
  aa.k = k;
  aa.v = v;
  aa.vt = nullptr;
  aa.mask = mask;
  aa.wbar = wbar;
  aa.out = out;
  aa.seq_lens = nullptr;
  aa.B = d.B;
  aa.Hq = d.Hq;
  aa.Hkv = d.Hkv;
  aa.D = d.D;
  aa.Tq = d.T;
  aa.Tk = d.T;
  aa.rows = d.T;
  aa.W = d.W;
  aa.wbar_ld = d.nc;
  aa.nc = d.nc;
  aa.scale_log2 = d.scale * 1.4426950408889634f;
  aa.sigma = d.sigma;
  aa.dtype = d.dtype;
  aa.dense = 0;
  aa.lse = lse;
  if (d.dtype == DASH_BF16) {
    aa.vt = ws + L.vt;
    if ((e = dash::launch_attend_mfma(aa, s)) != hipSuccess)
      return hip_fail(e, "stage 2 launch");
  } else {
    if ((e = dash::launch_attend_valu(aa, s)) != hipSuccess) return hip_fail(e, "stage 2 launch");
  }
  return ok();
}

int dash_prefill(const dash_params* p, const void* q, const void* k, const void* v,
                 const void* head_cls, void* out, uint64_t* active_blocks,
                 float* block_weights, float* summary_out, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return prefill_impl(p, 15, q, k, v, head_cls, out, active_blocks, block_weights, summary_out,
                      workspace, workspace_bytes, stream);
}

int dash_prefill_train(const dash_params* p, const void* q, const void* k, const void* v,
                       const void* head_cls, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (int rc = check_ptr(lse, "lse")) return rc;
  return prefill_impl(p, 15, q, k, v, head_cls, out, nullptr, nullptr, nullptr, workspace,
                      workspace_bytes, stream, lse);
}

namespace {

struct BackwardLayout {
  PrefillLayout fwd;
  size_t tau, z, dq32, dk32, dv32, dwb, dsumm, dhcp, mscratch, total;
};

BackwardLayout backward_layout(const Dims& d) {
  BackwardLayout L;
  L.fwd = prefill_layout(d);
  size_t off = L.fwd.total;
  const size_t rows_q = (size_t)d.B * d.Hq * d.T, rows_kv = (size_t)d.B * d.Hkv * d.T;
  L.tau = off;
  off += align256(rows_q * 4);
  L.z = off;
  off += align256(rows_q * 4);
  L.dq32 = off;
  off += align256(rows_q * d.D * 4);
  L.dk32 = off;
  off += align256(rows_kv * d.D * 4);
  L.dv32 = off;
  off += align256(rows_kv * d.D * 4);
  L.dwb = off;
  off += align256(rows_kv * d.nc * 4);
  L.dsumm = off;
  off += align256((size_t)d.B * d.Hkv * d.nc * d.D * 4);
  L.dhcp = off;
  off += align256((size_t)d.B * d.Hkv * d.nc * d.D * 4);
  L.mscratch = off;          // bf16: the MFMA kernels' delta, block unions, split K_bar, rho, scaled Q
  if (d.dtype == DASH_BF16) {
    size_t o1, o2, o3, o4, o5, tot;
    dash::backward_mfma_scratch(d.B, d.Hq, d.Hkv, d.T, d.D, &o1, &o2, &o3, &o4, &o5, &tot);
    off += align256(tot);
  }
  L.total = off;
  return L;
}

int check_backward_params(const dash_params* p, Dims* d) {
  if (int rc = check_params(p, d)) return rc;
  if (p->topk > 0)
    return fail(DASH_ERR_UNSUPPORTED, "the backward pass is built for alpha-entmax routing only (topk = %d)", p->topk);
  if (p->estimate_diagonal != 0)
    return fail(DASH_ERR_UNSUPPORTED, "the backward pass is built with estimate_diagonal = 0 only");
  return DASH_OK;
}

}  // namespace

int dash_prefill_backward_workspace_size(const dash_params* p, size_t* bytes) {
  Dims d;
  if (int rc = check_backward_params(p, &d)) return rc;
  if (!bytes) return fail(DASH_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = backward_layout(d).total;
  return ok();
}

int dash_prefill_backward(const dash_params* p, const void* q, const void* k, const void* v,
                          const void* head_cls, const void* out, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv, float* dhead_cls,
                          void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  if (int rc = check_backward_params(p, &d)) return rc;
  if (int rc = check_ptr(q, "q")) return rc;
  if (int rc = check_ptr(k, "k")) return rc;
  if (int rc = check_ptr(v, "v")) return rc;
  if (int rc = check_ptr(head_cls, "head_cls")) return rc;
  if (int rc = check_ptr(out, "out")) return rc;
  if (int rc = check_ptr(dout, "dout")) return rc;
  if (int rc = check_ptr(lse, "lse")) return rc;
  if (int rc = check_ptr(dq, "dq")) return rc;
  if (int rc = check_ptr(dk, "dk")) return rc;
  if (int rc = check_ptr(dv, "dv")) return rc;
  if (int rc = check_ptr(dhead_cls, "dhead_cls")) return rc;
  const BackwardLayout L = backward_layout(d);
  if (int rc = check_ws(workspace, workspace_bytes, L.total)) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  hipError_t e;
  float* summ = reinterpret_cast<float*>(ws + L.fwd.summ);
  uint64_t* mask = reinterpret_cast<uint64_t*>(ws + L.fwd.mask);
  float* wbar = reinterpret_cast<float*>(ws + L.fwd.wbar);
  float* tau = reinterpret_cast<float*>(ws + L.tau);
  float* zn = reinterpret_cast<float*>(ws + L.z);
  // Stages 0 and 1 again, as the forward ran them, keeping each head's threshold
  void* ss = d.dtype == DASH_BF16 ? (void*)(ws + L.fwd.ssplit) : nullptr;
  if ((e = dash::launch_stage0(k, head_cls, summ, ss, d.B, d.Hkv, d.T, d.D, d.nc, d.nfull,
                               nullptr, nullptr, d.scale, d.dtype, s)) != hipSuccess)
    return hip_fail(e, "stage 0 launch");
  if (d.dtype == DASH_BF16) {
    if ((e = dash::launch_vtranspose(v, ws + L.fwd.vt, d.B, d.Hkv, d.T, d.D, d.nc, s)) != hipSuccess)
      return hip_fail(e, "V transpose launch");
  }
  dash::RouteArgs ra{};
  ra.q = q;
  ra.summ = summ;
  ra.mask = mask;
  ra.wbar = wbar;
  ra.B = d.B;
  ra.Hq = d.Hq;
  ra.Hkv = d.Hkv;
  ra.D = d.D;
  ra.Tq = d.T;
  ra.rows = d.T;
  ra.nc_alloc = d.nc;
  ra.W = d.W;
  ra.wbar_ld = d.nc;
  ra.tcap = d.T;
  ra.alpha = d.alpha;
  ra.zscale = (d.alpha - 1.0f) * d.gamma * d.scale;
  ra.dtype = d.dtype;
  ra.tau_out = tau;
  ra.z_out = zn;
  e = d.dtype == DASH_BF16 ? dash::launch_route_mfma(ra, ss, s) : dash::launch_route_valu(ra, s);
  if (e != hipSuccess) return hip_fail(e, "stage 1 launch");
  // accumulators that the kernels add into (the generic kernels also add into dw_bar)
  if ((e = fill_f32(reinterpret_cast<float*>(ws + L.dk32), (size_t)d.B * d.Hkv * d.T * d.D, 0.f, s)) != hipSuccess ||
      (e = fill_f32(reinterpret_cast<float*>(ws + L.dv32), (size_t)d.B * d.Hkv * d.T * d.D, 0.f, s)) != hipSuccess ||
      (e = fill_f32(reinterpret_cast<float*>(ws + L.dsumm), (size_t)d.B * d.Hkv * d.nc * d.D, 0.f, s)) != hipSuccess)
    return hip_fail(e, "clearing the gradient accumulators");
  if (d.dtype != DASH_BF16) {
    if ((e = fill_f32(reinterpret_cast<float*>(ws + L.dwb), (size_t)d.B * d.Hkv * d.T * d.nc, 0.f, s)) != hipSuccess)
      return hip_fail(e, "clearing the gradient accumulators");
  }
  dash::BackwardArgs ba{};
  ba.q = q;
  ba.k = k;
  ba.v = v;
  ba.vt = d.dtype == DASH_BF16 ? ws + L.fwd.vt : nullptr;
  ba.head_cls = head_cls;
  ba.out = out;
  ba.dout = dout;
  ba.lse = lse;
  ba.summ = summ;
  ba.ssplit = reinterpret_cast<const dash::bf16*>(ss);
  ba.mask = mask;
  ba.wbar = wbar;
  ba.tau = tau;
  ba.z = zn;
  ba.dq32 = reinterpret_cast<float*>(ws + L.dq32);
  ba.dk32 = reinterpret_cast<float*>(ws + L.dk32);
  ba.dv32 = reinterpret_cast<float*>(ws + L.dv32);
  ba.dwb = reinterpret_cast<float*>(ws + L.dwb);
  ba.dsumm = reinterpret_cast<float*>(ws + L.dsumm);
  ba.dhc_part = reinterpret_cast<float*>(ws + L.dhcp);
  ba.dq = dq;
  ba.dk = dk;
  ba.dv = dv;
  ba.dhead_cls = dhead_cls;
  ba.B = d.B;
  ba.Hq = d.Hq;
  ba.Hkv = d.Hkv;
  ba.T = d.T;
  ba.D = d.D;
  ba.nc = d.nc;
  ba.W = d.W;
  ba.scale = d.scale;
  ba.gamma = d.gamma;
  ba.alpha = d.alpha;
  ba.sigma = d.sigma;
  ba.dtype = d.dtype;
  if (d.dtype == DASH_BF16) {
    if ((e = dash::launch_backward_mfma(ba, ws + L.mscratch, s)) != hipSuccess)
      return hip_fail(e, "backward launch");
  } else {
    if ((e = dash::launch_backward_valu(ba, s)) != hipSuccess) return hip_fail(e, "backward launch");
  }
  if ((e = dash::launch_backward_stage0(ba, s)) != hipSuccess) return hip_fail(e, "Stage 0 backward launch");
  return ok();
}

int dash_prefill_stage(const dash_params* p, int stage, const void* q, const void* k,
                       const void* v, const void* head_cls, void* out,
                       uint64_t* active_blocks, float* block_weights, float* summary_out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (stage < 0 || stage > 3) return fail(DASH_ERR_INVALID_ARG, "stage must be 0, 1, 2 or 3");
  return prefill_impl(p, 1 << stage, q, k, v, head_cls, out, active_blocks, block_weights,
                      summary_out, workspace, workspace_bytes, stream);
}

int dash_decode_workspace_size(const dash_params* p, size_t* bytes) {
  Dims d;
  if (int rc = check_params(p, &d)) return rc;
  if (!bytes) return fail(DASH_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = decode_layout(d).total;
  return ok();
}

namespace {

// block_table == nullptr: contiguous [B, Hkv, T_max, D] caches; otherwise page pools
// [num_pages, Hkv, C, D] (bf16 only) with chunk c of sequence b in page block_table[b][c].
int decode_impl(const dash_params* p, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_table, int32_t num_pages, const int32_t* seq_lens,
                const float* summary_cache, void* out, uint64_t* active_blocks, void* workspace,
                size_t workspace_bytes, void* stream, const void* head_cls = nullptr) {
  Dims d;
  if (int rc = check_params(p, &d)) return rc;
  if (p->topk > 0 && d.dtype != DASH_BF16)
    return fail(DASH_ERR_UNSUPPORTED, "the top-k comparison router is built for bf16 only");
  if (p->estimate_diagonal != 0) {
    if (p->topk > 0)
      return fail(DASH_ERR_UNSUPPORTED, "estimate_diagonal=1 applies to the entmax router only");
    if (d.T > dash::kChunk * dash::kMaxRouted)
      return fail(DASH_ERR_UNSUPPORTED, "estimate_diagonal=1: T=%d exceeds %d", d.T,
                  dash::kChunk * dash::kMaxRouted);
    if (!head_cls)
      return fail(DASH_ERR_INVALID_ARG, "estimate_diagonal=1 needs head_cls (dash_decode_diag, dash_decode_paged_diag)");
    if (int rc = check_ptr(head_cls, "head_cls")) return rc;
  }
  if (block_table) {
    if (d.dtype != DASH_BF16) return fail(DASH_ERR_UNSUPPORTED, "paged caches are bf16 only");
    if (num_pages <= 0) return fail(DASH_ERR_INVALID_ARG, "num_pages must be positive");
  }
  if (int rc = check_ptr(q, "q")) return rc;
  if (int rc = check_ptr(k_cache, "k_cache")) return rc;
  if (int rc = check_ptr(v_cache, "v_cache")) return rc;
  if (!seq_lens) return fail(DASH_ERR_INVALID_ARG, "seq_lens is NULL");
  if (int rc = check_ptr(summary_cache, "summary_cache")) return rc;
  if (int rc = check_ptr(out, "out")) return rc;
  if (int rc = check_ptr(active_blocks, "active_blocks", false)) return rc;
  const DecodeLayout L = decode_layout(d);
  if (int rc = check_ws(workspace, workspace_bytes, L.total)) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  uint64_t* mask = active_blocks ? active_blocks : reinterpret_cast<uint64_t*>(ws + L.mask);
  float* wbar = reinterpret_cast<float*>(ws + L.wbar);
  hipError_t e;

  dash::RouteArgs ra{};
  ra.q = q;
  ra.summ = summary_cache;
  ra.mask = mask;
  ra.wbar = wbar;
  ra.seq_lens = seq_lens;
  ra.B = d.B;
  ra.Hq = d.Hq;
  ra.Hkv = d.Hkv;
  ra.D = d.D;
  ra.Tq = 1;
  ra.rows = 1;
  ra.nc_alloc = d.nc;
  ra.W = d.W;
  ra.wbar_ld = d.nc;
  ra.tcap = d.T;
  ra.alpha = d.alpha;
  ra.zscale = (d.alpha - 1.0f) * d.gamma * d.scale;
  ra.topk = p->topk;
  ra.dtype = d.dtype;
  ra.list = reinterpret_cast<int32_t*>(ws + L.list);
  ra.list_ld = d.nc + 2;
  ra.sco = reinterpret_cast<float*>(ws + L.sco);
  ra.sco_ld = 16 * ((d.nc + 15) / 16);
  if (p->estimate_diagonal != 0) {
    ra.kdiag = k_cache;
    ra.head_cls = head_cls;
    ra.kdiag_ld = d.T;
    ra.s0_scale_log2 = d.scale * 1.4426950408889634f;
    ra.kdiag_bt = block_table;
    ra.kdiag_bt_ld = d.nc;
    ra.kdiag_pages = num_pages;
  }
  e = d.dtype == DASH_BF16 ? dash::launch_decode_route(ra, s) : dash::launch_route_valu(ra, s);
  if (e != hipSuccess) return hip_fail(e, "decode route launch");

  dash::AttendArgs aa{};
  aa.q = q;
  aa.k = k_cache;
  aa.v = v_cache;
  aa.mask = mask;
  aa.wbar = wbar;
  aa.out = out;
  aa.seq_lens = seq_lens;
  aa.B = d.B;
  aa.Hq = d.Hq;
  aa.Hkv = d.Hkv;
  aa.D = d.D;
  aa.Tq = 1;
  aa.Tk = d.T;
  aa.rows = 1;
  aa.W = d.W;
  aa.wbar_ld = d.nc;
  aa.nc = d.nc;
  aa.scale_log2 = d.scale * 1.4426950408889634f;
  aa.sigma = d.sigma;
  aa.dtype = d.dtype;
  aa.dense = 0;
  aa.list = reinterpret_cast<const int32_t*>(ws + L.list);
  aa.list_ld = d.nc + 2;
  aa.seg_size = reinterpret_cast<int32_t*>(ws + L.segsz);
  aa.block_table = block_table;
  aa.bt_ld = d.nc;
  aa.num_pages = num_pages;
  if (d.dtype == DASH_BF16)
    e = dash::launch_decode_attend(aa, reinterpret_cast<float*>(ws + L.pml),
                                   reinterpret_cast<float*>(ws + L.po), s);
  else
    e = dash::launch_attend_valu(aa, s);
  if (e != hipSuccess) return hip_fail(e, "decode attend launch");
  return ok();
}

int append_impl(const dash_params* p, const void* k_cache, const int32_t* block_table,
                int32_t num_pages, const void* head_cls, const int32_t* seq_lens,
                float* summary_cache, int32_t* n_summarized, void* stream) {
  Dims d;
  if (int rc = check_params(p, &d)) return rc;
  if (int rc = check_ptr(k_cache, "k_cache")) return rc;
  if (int rc = check_ptr(head_cls, "head_cls")) return rc;
  if (!seq_lens) return fail(DASH_ERR_INVALID_ARG, "seq_lens is NULL");
  if (int rc = check_ptr(summary_cache, "summary_cache")) return rc;
  if (!n_summarized) return fail(DASH_ERR_INVALID_ARG, "n_summarized is NULL");
  if (block_table) {
    if (d.dtype != DASH_BF16) return fail(DASH_ERR_UNSUPPORTED, "paged caches are bf16 only");
    if (num_pages <= 0) return fail(DASH_ERR_INVALID_ARG, "num_pages must be positive");
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if ((e = dash::launch_stage0(k_cache, head_cls, summary_cache, nullptr, d.B, d.Hkv, d.T, d.D, d.nc,
                               d.nfull, n_summarized, seq_lens, d.scale, d.dtype, s, block_table,
                               d.nc, num_pages)) != hipSuccess)
    return hip_fail(e, "append launch");
  if ((e = dash::launch_update_nsum(n_summarized, seq_lens, d.B, d.T, s)) != hipSuccess)
    return hip_fail(e, "append bookkeeping launch");
  return ok();
}

}  // namespace

int dash_decode(const dash_params* p, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* seq_lens, const float* summary_cache, void* out,
                uint64_t* active_blocks, void* workspace, size_t workspace_bytes,
                void* stream) {
  return decode_impl(p, q, k_cache, v_cache, nullptr, 0, seq_lens, summary_cache, out,
                     active_blocks, workspace, workspace_bytes, stream);
}

int dash_decode_diag(const dash_params* p, const void* q, const void* k_cache,
                     const void* v_cache, const void* head_cls, const int32_t* seq_lens,
                     const float* summary_cache, void* out, uint64_t* active_blocks,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(p, q, k_cache, v_cache, nullptr, 0, seq_lens, summary_cache, out,
                     active_blocks, workspace, workspace_bytes, stream, head_cls);
}

int dash_decode_paged_diag(const dash_params* p, const void* q, const void* k_pages,
                           const void* v_pages, int32_t num_pages, const int32_t* block_table,
                           const void* head_cls, const int32_t* seq_lens,
                           const float* summary_cache, void* out, uint64_t* active_blocks,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(p, q, k_pages, v_pages, block_table, num_pages, seq_lens, summary_cache,
                     out, active_blocks, workspace, workspace_bytes, stream, head_cls);
}

int dash_decode_paged(const dash_params* p, const void* q, const void* k_pages,
                      const void* v_pages, int32_t num_pages, const int32_t* block_table,
                      const int32_t* seq_lens, const float* summary_cache, void* out,
                      uint64_t* active_blocks, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (!block_table) return fail(DASH_ERR_INVALID_ARG, "block_table is NULL");
  return decode_impl(p, q, k_pages, v_pages, block_table, num_pages, seq_lens, summary_cache,
                     out, active_blocks, workspace, workspace_bytes, stream);
}

int dash_decode_noalloc(const dash_params* p, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* seq_lens,
                        const float* summary_cache, void* out, uint64_t* active_blocks,
                        void* stream) {
  Dims d;
  if (int rc = check_params(p, &d)) return rc;
  const size_t need = decode_layout(d).total;
  if (need > kNoAllocScratchBytes)
    return fail(DASH_ERR_WORKSPACE,
                "dash_decode_noalloc: this shape needs %zu bytes of scratch, above the fixed "
                "%zu (use dash_decode with a workspace)", need, kNoAllocScratchBytes);
  int st = DASH_OK;
  void* ws = scratch_address(&st);
  if (!ws) return st;
  return decode_impl(p, q, k_cache, v_cache, nullptr, 0, seq_lens, summary_cache, out,
                     active_blocks, ws, kNoAllocScratchBytes, stream);
}

int dash_append_chunk(const dash_params* p, const void* k_cache, const void* head_cls,
                      const int32_t* seq_lens, float* summary_cache, int32_t* n_summarized,
                      void* stream) {
  return append_impl(p, k_cache, nullptr, 0, head_cls, seq_lens, summary_cache, n_summarized,
                     stream);
}

int dash_append_chunk_paged(const dash_params* p, const void* k_pages, int32_t num_pages,
                            const int32_t* block_table, const void* head_cls,
                            const int32_t* seq_lens, float* summary_cache,
                            int32_t* n_summarized, void* stream) {
  if (!block_table) return fail(DASH_ERR_INVALID_ARG, "block_table is NULL");
  return append_impl(p, k_pages, block_table, num_pages, head_cls, seq_lens, summary_cache,
                     n_summarized, stream);
}

int dash_dense_causal_workspace_size(const dash_params* p, size_t* bytes) {
  Dims d;
  if (int rc = check_params(p, &d, true)) return rc;
  if (!bytes) return fail(DASH_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = align256((size_t)d.B * d.Hkv * d.nc * d.D * 64 * 2) + 256;
  return ok();
}

int dash_dense_causal(const dash_params* p, const void* q, const void* k, const void* v,
                      void* out, void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  if (int rc = check_params(p, &d, true)) return rc;
  if (int rc = check_ptr(q, "q")) return rc;
  if (int rc = check_ptr(k, "k")) return rc;
  if (int rc = check_ptr(v, "v")) return rc;
  if (int rc = check_ptr(out, "out")) return rc;
  size_t need = 0;
  dash_dense_causal_workspace_size(p, &need);
  if (int rc = check_ws(workspace, workspace_bytes, need)) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  dash::AttendArgs aa{};
  aa.q = q;
  aa.k = k;
  aa.v = v;
  aa.out = out;
  aa.B = d.B;
  aa.Hq = d.Hq;
  aa.Hkv = d.Hkv;
  aa.D = d.D;
  aa.Tq = d.T;
  aa.Tk = d.T;
  aa.rows = d.T;
  aa.W = d.W;
  aa.wbar_ld = d.nc;
  aa.nc = d.nc;
  aa.scale_log2 = d.scale * 1.4426950408889634f;
  aa.sigma = d.sigma;
  aa.dtype = d.dtype;
  aa.dense = 1;
  void* vt = workspace;
  if ((e = dash::launch_vtranspose(v, vt, d.B, d.Hkv, d.T, d.D, d.nc, s)) != hipSuccess)
    return hip_fail(e, "V transpose launch");
  aa.vt = vt;
  if ((e = dash::launch_attend_mfma(aa, s)) != hipSuccess) return hip_fail(e, "dense launch");
  return ok();
}

}  // extern "C"
