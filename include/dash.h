/*
 * dash.h -- C ABI of the MI355X (gfx950) DashAttention forward library (libdash.so).
 *
 * The method (arXiv 2605.18753, "DashAttention: Differentiable and Adaptive Sparse
 * Hierarchical Attention"), as summarised on gist.science ("Technische Zusammenfassung",
 * "Methodik"), the aixai.ru blog ("Трёхстадийная архитектура") and the liuzhao09 reading
 * note (section 2, "核心方法"):
 *   Stage 0  every complete 64-token chunk of keys is summarised by a scaled dot-product
 *            attention of a learned per-head query (head_cls) over the chunk's keys;
 *   Stage 1  each query scores the chunk summaries and alpha-entmax(gamma * scores) gives a
 *            sparse block distribution; the distributions of the query heads that share a
 *            KV head are averaged into one shared support, packed as a bit mask in 64-bit
 *            words;
 *   Stage 2  token-level softmax attention over the active chunks only, with the Stage 1
 *            block weight entering the token logits as a log-prior, plus the query's own
 *            (diagonal) chunk, which has no summary yet.
 * The interface -- queries, keys, values, a per-head classification vector head_cls,
 * chunk_size, estimate_diagonal, enable_gqa and an optional active_blocks mask -- follows
 * the aiexpert.news article on the authors' release (paragraph on the Triton package).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers unless stated; tensors are dense, row-major,
 *     with the shapes given below; they must be 16-byte aligned.  The caller owns all
 *     memory; the library never allocates device memory and keeps no state besides the
 *     loaded kernels, a thread-local error string and a per-device cache of the CU count
 *     (read once, to size decode launches).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *     returns without waiting.  Arguments are validated on the host first; on any
 *     failure nothing is launched and a negative dash_status is returned, with a message
 *     in dash_last_error().  Faults inside kernels surface at the caller's next
 *     synchronisation.
 *   - kv(h) = h / (Hq / Hkv): consecutive query heads share a KV head (enable_gqa).
 *   - Only complete chunks are summarised.  Row t routes over chunks c < t / C and always
 *     attends causally inside its own chunk with log-prior 0.
 *   - Beyond the method's defaults: a prior strength sigma, a top-k comparison router
 *     (topk) in place of entmax, and paged K/V caches for decoding (dash_decode_paged,
 *     dash_append_chunk_paged).
 */
#ifndef DASH_H_
#define DASH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DASH_OK = 0,
  DASH_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad alpha/gamma/scale, T <= 0 */
  DASH_ERR_SHAPE = -2,       /* head counts inconsistent, sizes too large */
  DASH_ERR_DTYPE = -3,       /* unknown dtype */
  DASH_ERR_UNSUPPORTED = -4, /* valid per the method, not built here (D, C, G, flags) */
  DASH_ERR_WORKSPACE = -5,   /* workspace pointer null or smaller than required */
  DASH_ERR_HIP = -6          /* a HIP runtime call or launch failed */
} dash_status;

typedef enum { DASH_BF16 = 0, DASH_FP32 = 1 } dash_dtype;

typedef struct dash_params {
  int32_t B;          /* batch */
  int32_t Hq;         /* query heads */
  int32_t Hkv;        /* key/value heads; Hq % Hkv == 0 */
  int32_t T;          /* prefill: sequence length; decode/append: cache capacity T_max */
  int32_t D;          /* head dim: 64 or 128 */
  int32_t chunk_size; /* tokens per chunk: 64 (the only size the pages use) */
  float alpha;        /* entmax alpha, finite and > 1; 1.5 at inference */
  float gamma;        /* Stage 1 logit factor (the "Stage 1 factor"), finite > 0 */
  float sm_scale;     /* logit scale of Stages 0-2; <= 0 selects 1/sqrt(D) */
  int32_t enable_gqa; /* 0: Hq must equal Hkv; 1: Hq % Hkv == 0 */
  int32_t dtype;      /* dash_dtype of q, k, v, head_cls and out */
  int32_t estimate_diagonal; /* 0: the own (diagonal) chunk takes no part in routing.  1
                         (dash_prefill, dash_decode_diag and dash_decode_paged_diag with
                         entmax routing, T <= 64 * 2048; with topk > 0 DASH_ERR_UNSUPPORTED;
                         dash_decode and dash_decode_paged, which take no head_cls, return
                         DASH_ERR_INVALID_ARG):
                         the own chunk is summarised by Stage 0's formula over its keys up to
                         the query and joins each head's alpha-entmax normalisation as one more
                         entry (aiexpert.news, interface paragraph: a diagonal correction of
                         the normalisation); its weight is then dropped and the routed chunks
                         keep theirs.  The own chunk is attended at prior 1 either way */
  float sigma;        /* prior strength, finite >= 0: keys of a routed chunk c get the logit
                         bias sigma * log w_bar_c.  1 is the prior itself, 0 a uniform prior
                         over the active chunks (gist.science, "Stufe 2": a hyperparameter
                         sigma weighs the routing values against a uniform baseline) */
  int32_t topk;       /* 0: alpha-entmax routing (the method).  k > 0: a top-k comparison
                         router instead -- per row and KV head, the chunks whose score summed
                         over the G heads is at least the k-th largest (every routed chunk
                         when there are at most k), each with weight 1 (no prior).  Not on the
                         pages as part of the method: they compare against top-k routers
                         (NSA, InfLLMv2; aixai.ru, experiments).  bf16 only */
} dash_params;

/* Version of this ABI (major * 100 + minor). */
int dash_abi_version(void);

/* Message describing the last non-OK status returned on this thread ("" if none). */
const char* dash_last_error(void);

/* ---------------------------------------------------------------------------------
 * Causal prefill (all three stages): gist.science, "Methodik" and "Stufe 0"-"Stufe 2"
 * (chunk summaries by a learned query's scaled dot-product attention over each complete
 * chunk; alpha-entmax over the query-vs-summary logits, averaged over the query heads of a
 * KV head into one shared support; softmax attention over the active chunks' tokens with
 * the log of the block weight added to their logits, plus the own chunk); aixai.ru,
 * "Трёхстадийная архитектура" (three stages, 64-bit mask words walked in one pass).
 *   q        [B, Hq, T, D]   dtype
 *   k, v     [B, Hkv, T, D]  dtype
 *   head_cls [Hkv, D]        dtype   (one classifier query per KV head)
 *   out      [B, Hq, T, D]   dtype   written
 * Optional outputs (NULL = not wanted):
 *   active_blocks [B, Hkv, T, W] uint64, W = ceil(ceil(T/C) / 64): bit (c % 64) of word
 *                 c / 64 is set iff the head-averaged weight of chunk c for row t is > 0
 *                 (LSB first).  Bits for c >= t / C are 0.
 *   block_weights [B, Hkv, T, ceil(T/C)] float32: the head-averaged entmax weights,
 *                 0 where inactive (debug/analysis; costs a full clear).
 *   summary_out   [B, Hkv, ceil(T/C), D] float32: Stage 0 summaries of every complete
 *                 chunk (a partial last chunk is left untouched); lets decode continue.
 * workspace: device buffer of at least dash_prefill_workspace_size() bytes, 256-byte
 * aligned, not shared with a concurrent call.
 * ------------------------------------------------------------------------------- */
/* Workspace queries return a dash_status like every other entry point and write the size
 * to *bytes, so an invalid parameter set is reported the same way everywhere. */
int dash_prefill_workspace_size(const dash_params* p, size_t* bytes);
int dash_prefill(const dash_params* p, const void* q, const void* k, const void* v,
                 const void* head_cls, void* out, uint64_t* active_blocks,
                 float* block_weights, float* summary_out, void* workspace,
                 size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Training: the forward that keeps what the backward pass needs, and the backward pass.
 * The pages' central claim is that the hierarchy is differentiable end to end: the routing
 * distribution is alpha-entmax, whose Jacobian exists almost everywhere, so gradients flow
 * from the token-level attention through the routing back to the chunk summaries and
 * Stage 0's classifier query (gist.science, "Stufe 1", remark on differentiability, and
 * "Hauptbeiträge"; aixai.ru, the section on why top-k routing breaks gradients).  The entmax
 * Jacobian is that of Peters, Niculae and Martins (2019), to which aixai.ru's FAQ points.
 *
 * dash_prefill_train: dash_prefill (same arguments, same out) that also writes
 *   lse [B, Hq, T] float32: for each head and row, the natural log of the sum over the
 *   row's attended keys of exp(logit), logit = sm_scale <q, k_j> + the key's log-prior.
 * dash_prefill_backward: gradients of a loss L given dout = dL/dout [B, Hq, T, D] (dtype),
 *   the forward's q, k, v, head_cls, out and lse, and the same dash_params:
 *   dq [B, Hq, T, D], dk, dv [B, Hkv, T, D] (dtype), dhead_cls [Hkv, D] (float32),
 *   all written (not accumulated).  Stage 0 and Stage 1 are recomputed from q, k and
 *   head_cls with the forward's kernels, so the routing is the forward's.  A chunk whose
 *   entmax argument sits exactly on the threshold gets the one-sided gradient with the
 *   chunk outside the support.  Alpha-entmax routing only: topk > 0 or
 *   estimate_diagonal = 1 is DASH_ERR_UNSUPPORTED.  workspace: at least
 *   dash_prefill_backward_workspace_size() bytes, 256-byte aligned.
 * ------------------------------------------------------------------------------- */
int dash_prefill_train(const dash_params* p, const void* q, const void* k, const void* v,
                       const void* head_cls, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream);
int dash_prefill_backward_workspace_size(const dash_params* p, size_t* bytes);
int dash_prefill_backward(const dash_params* p, const void* q, const void* k, const void* v,
                          const void* head_cls, const void* out, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv, float* dhead_cls,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Profiling aid: run one step of dash_prefill alone (stage 0: the chunk summaries; 1:
 * routing; 2: sparse attention; 3: the chunk-transposed copy of V that bf16 Stage 2 reads,
 * a no-op for fp32), reading the intermediates that a complete dash_prefill call with the
 * same arguments and workspace left behind.  Used to time each kernel separately; stages
 * 0, 3, 1, 2 in that order give the results of the full call. */
int dash_prefill_stage(const dash_params* p, int stage, const void* q, const void* k,
                       const void* v, const void* head_cls, void* out,
                       uint64_t* active_blocks, float* block_weights, float* summary_out,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * One incremental decoding step (one new token per sequence): the incremental decoding
 * with a cache of chunk representations that gist.science names among the main
 * contributions ("Hauptbeiträge") and the liuzhao09 note describes in section 2 (the
 * summary of a complete chunk is computed once, cached and reused by every later query;
 * gist.science "Stufe 0").  Stages 1 and 2 then run for the single new query row.
 *   p->T          cache capacity T_max
 *   q             [B, Hq, D]            dtype, the new token's queries
 *   k_cache, v_cache [B, Hkv, T_max, D] dtype, holding seq_lens[b] valid tokens, the new
 *                 token included (the caller writes it at index seq_lens[b] - 1 first)
 *   seq_lens      [B] int32 (device): 1 <= seq_lens[b] <= T_max
 *   summary_cache [B, Hkv, ceil(T_max/C), D] float32 holding the summaries of every
 *                 chunk c < (seq_lens[b] - 1) / C (see dash_append_chunk)
 *   out           [B, Hq, D] dtype written
 *   active_blocks optional [B, Hkv, W] uint64, W = ceil(ceil(T_max/C) / 64)
 * The query sits at t = seq_lens[b] - 1: decode row t equals prefill row t of the same
 * sequence.  A sequence whose seq_lens entry is out of range gets NaN outputs and no
 * memory outside its cache rows is touched.
 * ------------------------------------------------------------------------------- */
int dash_decode_workspace_size(const dash_params* p, size_t* bytes);
int dash_decode(const dash_params* p, const void* q, const void* k_cache,
                const void* v_cache, const int32_t* seq_lens, const float* summary_cache,
                void* out, uint64_t* active_blocks, void* workspace,
                size_t workspace_bytes, void* stream);

/* dash_decode with the KV heads' head_cls [Hkv, D] (dtype, device), which
 * estimate_diagonal = 1 needs: the own chunk of the query at t is summarised over its keys
 * i_t C .. t of k_cache (Stage 0's formula) and joins each head's alpha-entmax
 * normalisation (aiexpert.news, interface paragraph), exactly as in dash_prefill.  With
 * estimate_diagonal = 0 it equals dash_decode.  Errors as dash_decode; a NULL head_cls with
 * the flag set is DASH_ERR_INVALID_ARG (so is the flag in dash_decode and dash_decode_paged),
 * the flag with topk > 0 or T_max > 64 * 2048 is DASH_ERR_UNSUPPORTED. */
int dash_decode_diag(const dash_params* p, const void* q, const void* k_cache,
                     const void* v_cache, const void* head_cls, const int32_t* seq_lens,
                     const float* summary_cache, void* out, uint64_t* active_blocks,
                     void* workspace, size_t workspace_bytes, void* stream);

/* dash_decode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the step's scratch (mask,
 * weights, work lists, scores and split-K partials) lives in a fixed 32 MiB device array
 * inside the library, one per GPU, held until the process ends; this call allocates
 * nothing.  Shapes whose dash_decode_workspace_size() exceeds 32 MiB are rejected with
 * DASH_ERR_WORKSPACE before anything is launched (the 64K-token, batch-16, 32/2-head
 * decode needs about 20 MiB).  Every call on one GPU uses the same array, so calls that
 * may overlap on one GPU (different streams, different host threads) race: serialise them.
 * Nothing in the array needs clearing between calls.  Other arguments, results and errors
 * as dash_decode. */
int dash_decode_noalloc(const dash_params* p, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* seq_lens,
                        const float* summary_cache, void* out, uint64_t* active_blocks,
                        void* stream);

/* ---------------------------------------------------------------------------------
 * Chunk-summary cache append.  A summary, once its chunk is complete, is frozen and
 * cached (gist.science, "Stufe 0", efficiency remark): for each b this summarises every
 * chunk c with n_summarized[b] <= c < seq_lens[b] / C into summary_cache and then sets
 * n_summarized[b] = max(n_summarized[b], seq_lens[b] / C).  Call it after a decode step
 * whose token completed a chunk, and once to build the cache of a prompt.
 *   k_cache [B, Hkv, T_max, D] dtype; head_cls [Hkv, D] dtype;
 *   seq_lens [B] int32 (device); summary_cache [B, Hkv, ceil(T_max/C), D] float32;
 *   n_summarized [B] int32 (device, in/out).
 * ------------------------------------------------------------------------------- */
int dash_append_chunk(const dash_params* p, const void* k_cache, const void* head_cls,
                      const int32_t* seq_lens, float* summary_cache,
                      int32_t* n_summarized, void* stream);

/* ---------------------------------------------------------------------------------
 * Paged caches: dash_decode and dash_append_chunk over a shared pool of pages, for
 * continuous batching (the pages' incremental decoding with a chunk-representation cache,
 * gist.science "Hauptbeiträge" and "Stufe 0"; the paging is this library's layout).  A
 * page holds one chunk of every KV head; p->T is the logical capacity T_max per sequence.
 *   k_pages, v_pages [num_pages, Hkv, C, D] bf16 (caller-owned; dtype must be DASH_BF16)
 *   block_table      [B, ceil(T_max/C)] int32 (device): page of chunk c of sequence b;
 *                    entries for chunks past a sequence's length are never read
 * Everything else, the workspace and the results are as for dash_decode /
 * dash_append_chunk; the summary cache stays per sequence.  A page id outside
 * [0, num_pages) is never dereferenced: decode reads its keys and values as zeros and
 * append leaves that chunk's summary untouched (the output is then meaningless).
 * Errors: DASH_ERR_INVALID_ARG for a NULL block_table or num_pages <= 0,
 * DASH_ERR_UNSUPPORTED for fp32.
 * ------------------------------------------------------------------------------- */
int dash_decode_paged(const dash_params* p, const void* q, const void* k_pages,
                      const void* v_pages, int32_t num_pages, const int32_t* block_table,
                      const int32_t* seq_lens, const float* summary_cache, void* out,
                      uint64_t* active_blocks, void* workspace, size_t workspace_bytes,
                      void* stream);
/* dash_decode_paged with head_cls [Hkv, D] (bf16), for estimate_diagonal = 1, as
 * dash_decode_diag: the own chunk's keys are read from its page (an id outside the pool
 * reads as zero keys). */
int dash_decode_paged_diag(const dash_params* p, const void* q, const void* k_pages,
                           const void* v_pages, int32_t num_pages, const int32_t* block_table,
                           const void* head_cls, const int32_t* seq_lens,
                           const float* summary_cache, void* out, uint64_t* active_blocks,
                           void* workspace, size_t workspace_bytes, void* stream);
int dash_append_chunk_paged(const dash_params* p, const void* k_pages, int32_t num_pages,
                            const int32_t* block_table, const void* head_cls,
                            const int32_t* seq_lens, float* summary_cache,
                            int32_t* n_summarized, void* stream);

/* ---------------------------------------------------------------------------------
 * Dense causal softmax attention with the same layout (the comparator the pages time
 * against: FlashAttention-3 in their Table 5).  Uses p->B, Hq, Hkv, T, D, sm_scale,
 * enable_gqa, dtype (bf16 only).
 *   q [B, Hq, T, D], k, v [B, Hkv, T, D], out [B, Hq, T, D].
 * ------------------------------------------------------------------------------- */
int dash_dense_causal_workspace_size(const dash_params* p, size_t* bytes);
int dash_dense_causal(const dash_params* p, const void* q, const void* k, const void* v,
                      void* out, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DASH_H_ */
