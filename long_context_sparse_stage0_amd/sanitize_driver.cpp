// Host-only check of the C ABI's argument validation under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by sanitize_build.py; no GPU is touched: every call
// below fails validation before any HIP call, or is a workspace-size query).
//
// Exit status 0 when every call returned the expected status; the sanitizers abort on any
// memory or undefined-behaviour error in the validation, layout and error-string code.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../include/dash.h"

namespace {

int g_fail = 0;

void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, dash_last_error());
    ++g_fail;
  } else if (want != DASH_OK && std::strlen(dash_last_error()) == 0) {
    std::printf("FAIL %s: no error message\n", what);
    ++g_fail;
  }
}

dash_params base() {
  dash_params p;
  std::memset(&p, 0, sizeof(p));
  p.B = 1;
  p.Hq = 4;
  p.Hkv = 2;
  p.T = 256;
  p.D = 128;
  p.chunk_size = 64;
  p.alpha = 1.5f;
  p.gamma = 1.0f;
  p.sm_scale = 0.0f;
  p.enable_gqa = 1;
  p.dtype = DASH_BF16;
  p.sigma = 1.0f;
  return p;
}

}  // namespace

int main() {
  void* fake = reinterpret_cast<void*>(uintptr_t(1) << 20);        // aligned, never used
  void* mis = reinterpret_cast<void*>((uintptr_t(1) << 20) + 4);   // misaligned
  const size_t big = size_t(1) << 40;
  size_t n = 0;

  dash_params p = base();
  expect(dash_prefill_workspace_size(&p, &n), DASH_OK, "prefill workspace size");
  expect(dash_prefill_workspace_size(nullptr, &n), DASH_ERR_INVALID_ARG, "null params");
  expect(dash_prefill_workspace_size(&p, nullptr), DASH_ERR_INVALID_ARG, "null bytes");
  expect(dash_decode_workspace_size(&p, &n), DASH_OK, "decode workspace size");
  expect(dash_prefill_backward_workspace_size(&p, &n), DASH_OK, "backward workspace size");
  expect(dash_dense_causal_workspace_size(&p, &n), DASH_OK, "dense workspace size");

  struct Bad { const char* what; void (*edit)(dash_params*); int code; };
  const Bad bads[] = {
      {"Hq % Hkv", [](dash_params* q) { q->Hq = 6; q->Hkv = 4; }, DASH_ERR_SHAPE},
      {"gqa flag", [](dash_params* q) { q->enable_gqa = 0; }, DASH_ERR_SHAPE},
      {"G = 3", [](dash_params* q) { q->Hq = 12; q->Hkv = 4; }, DASH_ERR_UNSUPPORTED},
      {"D = 96", [](dash_params* q) { q->D = 96; }, DASH_ERR_UNSUPPORTED},
      {"chunk 128", [](dash_params* q) { q->chunk_size = 128; }, DASH_ERR_UNSUPPORTED},
      {"alpha 1", [](dash_params* q) { q->alpha = 1.0f; }, DASH_ERR_INVALID_ARG},
      {"alpha nan", [](dash_params* q) { q->alpha = NAN; }, DASH_ERR_INVALID_ARG},
      {"gamma 0", [](dash_params* q) { q->gamma = 0.0f; }, DASH_ERR_INVALID_ARG},
      {"scale inf", [](dash_params* q) { q->sm_scale = INFINITY; }, DASH_ERR_INVALID_ARG},
      {"T 0", [](dash_params* q) { q->T = 0; }, DASH_ERR_INVALID_ARG},
      {"B 0", [](dash_params* q) { q->B = 0; }, DASH_ERR_INVALID_ARG},
      {"dtype 7", [](dash_params* q) { q->dtype = 7; }, DASH_ERR_DTYPE},
      {"sigma -1", [](dash_params* q) { q->sigma = -1.0f; }, DASH_ERR_INVALID_ARG},
      {"topk -1", [](dash_params* q) { q->topk = -1; }, DASH_ERR_INVALID_ARG},
      {"T too long", [](dash_params* q) { q->T = 64 * 2049 + 1; }, DASH_ERR_UNSUPPORTED},
      {"huge B", [](dash_params* q) { q->B = 2147483647; }, DASH_OK},   // sizes only
  };
  for (const Bad& b : bads) {
    dash_params q = base();
    b.edit(&q);
    if (b.code == DASH_OK) {
      // a valid but huge shape: size queries must not overflow into a small number
      if (dash_prefill_workspace_size(&q, &n) == DASH_OK && n < (size_t(1) << 32)) {
        std::printf("FAIL %s: workspace size %zu\n", b.what, n);
        ++g_fail;
      }
      continue;
    }
    expect(dash_prefill_workspace_size(&q, &n), b.code, b.what);
    expect(dash_prefill(&q, fake, fake, fake, fake, fake, nullptr, nullptr, nullptr, fake, big,
                        nullptr), b.code, b.what);
    expect(dash_decode(&q, fake, fake, fake, (const int32_t*)fake, (const float*)fake, fake,
                       nullptr, fake, big, nullptr), b.code, b.what);
    expect(dash_prefill_backward(&q, fake, fake, fake, fake, fake, fake, (const float*)fake,
                                 fake, fake, fake, (float*)fake, fake, big, nullptr),
           b.code, b.what);
  }
  // pointers and workspaces
  p = base();
  expect(dash_prefill_workspace_size(&p, &n), DASH_OK, "size");
  expect(dash_prefill(&p, nullptr, fake, fake, fake, fake, nullptr, nullptr, nullptr, fake, n,
                      nullptr), DASH_ERR_INVALID_ARG, "null q");
  expect(dash_prefill(&p, mis, fake, fake, fake, fake, nullptr, nullptr, nullptr, fake, n,
                      nullptr), DASH_ERR_INVALID_ARG, "misaligned q");
  expect(dash_prefill(&p, fake, fake, fake, fake, fake, nullptr, nullptr, nullptr, nullptr, n,
                      nullptr), DASH_ERR_WORKSPACE, "null workspace");
  expect(dash_prefill(&p, fake, fake, fake, fake, fake, nullptr, nullptr, nullptr, fake, n - 1,
                      nullptr), DASH_ERR_WORKSPACE, "small workspace");
  expect(dash_prefill_stage(&p, 4, fake, fake, fake, fake, fake, nullptr, nullptr, nullptr, fake,
                            n, nullptr), DASH_ERR_INVALID_ARG, "stage 4");
  expect(dash_prefill_train(&p, fake, fake, fake, fake, fake, nullptr, fake, n, nullptr),
         DASH_ERR_INVALID_ARG, "train without lse");
  dash_params pt = base();
  pt.topk = 4;
  expect(dash_prefill_backward_workspace_size(&pt, &n), DASH_ERR_UNSUPPORTED, "backward topk");
  pt = base();
  pt.estimate_diagonal = 1;
  expect(dash_prefill_backward_workspace_size(&pt, &n), DASH_ERR_UNSUPPORTED, "backward diag");
  p = base();
  expect(dash_prefill_backward(&p, fake, fake, fake, fake, fake, fake, nullptr, fake, fake, fake,
                               (float*)fake, fake, big, nullptr), DASH_ERR_INVALID_ARG,
         "backward without lse");
  // decode entry points
  p = base();
  p.Hq = 32;
  p.T = 65792;
  expect(dash_decode_workspace_size(&p, &n), DASH_OK, "decode size");
  expect(dash_decode(&p, fake, fake, fake, nullptr, (const float*)fake, fake, nullptr, fake, n,
                     nullptr), DASH_ERR_INVALID_ARG, "null seq_lens");
  expect(dash_decode_paged(&p, fake, fake, fake, 4, nullptr, (const int32_t*)fake,
                           (const float*)fake, fake, nullptr, fake, n, nullptr),
         DASH_ERR_INVALID_ARG, "null block table");
  expect(dash_append_chunk(&p, fake, fake, (const int32_t*)fake, (float*)fake, nullptr, nullptr),
         DASH_ERR_INVALID_ARG, "null n_summarized");
  dash_params pb = base();
  pb.B = 64;
  pb.Hq = 32;
  pb.T = 64 * 2049;
  expect(dash_decode_noalloc(&pb, fake, fake, fake, (const int32_t*)fake, (const float*)fake,
                             fake, nullptr, nullptr), DASH_ERR_WORKSPACE, "no-alloc oversize");
  // a long message must be truncated safely
  dash_params pl = base();
  pl.dtype = 123456789;
  expect(dash_prefill_workspace_size(&pl, &n), DASH_ERR_DTYPE, "dtype message");
  std::printf("%s: %d failure(s)\n", g_fail ? "FAILED" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
