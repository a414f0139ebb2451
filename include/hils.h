/*
 * hils.h — C ABI of the HiLS (Hierarchical Landmark Sparse) attention forward
 * pass for AMD Instinct MI355X (gfx950).
 *
 * The operation is defined in "Hierarchical Sparse Attention Done Right:
 * Toward Infinite Context Modeling" (Hu et al., arXiv 2607.02980):
 *   - section 2.1: chunks c(j) = floor(j/S); aligned window boundary
 *     l(i) = floor((i-W+1)/S)*S; candidate chunks C_i = {0..l(i)/S-1};
 *     token logits s_ij = q_i.k_j/sqrt(d); window mass Z_{i,swa};
 *   - section 3, Proposition 3.1 and the landmark text: per-chunk summary
 *     (k'_c, b'_c) from Attn(q'_c, K_c, K_c), b'_c the entropy of the
 *     landmark query's attention over the chunk;
 *   - section 3, routing equation: s_hat_ic = q_i.k'_c/sqrt(d) + b'_c, the
 *     top-K chunks of C_i, and the fused mass Z_hat_i;
 *   - section 3, hierarchical-softmax equation: independent softmax inside
 *     every selected chunk and inside the window, fused by a softmax over the
 *     chunk scores (the window's logit is log Z_{i,swa});
 *   - section 4.1: low-rank query calibration (a routing query q_hat used only
 *     in s_hat) and GQA shared selection (per-head normalised chunk weights,
 *     maximum over the heads of a group, one top-K per group).
 *
 * Conventions for every entry point
 *   - All tensors are caller-owned DEVICE memory, contiguous, head-major:
 *       q, q_route, out : [B][Hq][N][d]         (decode: [B][Hq][1][d])
 *       k, v            : [B][Hkv][N][d]        (decode: the KV cache, N = capacity)
 *       lm_q            : [B][Hq][floor(N/S)][d]  one landmark query per chunk per q head
 *       k_sum           : [B][Hq][floor(N/S)][d]  summary keys, element type = dtype
 *       b_sum           : [B][Hq][floor(N/S)]     entropy biases, fp32
 *       sel             : [B][Hkv][N][K] int32   (decode: [B][Hkv][K]) selected chunk
 *                         ids of each query, ascending, -1 padded when |C_i| < K
 *     Element type of q/q_route/k/v/lm_q/k_sum/out is cfg->dtype (bf16 or fp32).
 *     Query head h uses KV head h / (Hq/Hkv).  Tokens and chunks are 0-based.
 *   - The library allocates no device memory.  Scratch comes from the caller's
 *     workspace `ws` of at least hils_workspace_bytes() bytes (256-byte aligned).
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 *     No entry point synchronises the host.  Outputs are valid once the stream
 *     reaches the enqueued work.  The library keeps no global mutable state
 *     (apart from the opt-in kernel-timing record below): calls on different
 *     streams with different buffers are independent.
 *   - Errors: arguments are validated before anything is enqueued; on a
 *     non-OK return nothing has been enqueued (except HILS_E_HIP, which reports
 *     a launch failure), and outputs are undefined.  No C++ exception crosses
 *     this boundary.
 */
#ifndef HILS_H
#define HILS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HILS_ABI_VERSION 1

typedef enum {
  HILS_OK = 0,
  HILS_E_ARG = 1,          /* invalid argument (shape, null pointer, misalignment) */
  HILS_E_UNSUPPORTED = 2,  /* valid but not implemented (e.g. d > 256, S > 64) */
  HILS_E_WORKSPACE = 3,    /* workspace too small */
  HILS_E_HIP = 4           /* HIP runtime / launch error */
} hils_status;

typedef enum { HILS_BF16 = 0, HILS_F32 = 1 } hils_dtype;

typedef enum {
  HILS_SCORE_SURROGATE = 0,     /* Proposition 3.1 summary (k'_c, b'_c) — the method */
  HILS_SCORE_LANDMARK_KEY = 1,  /* ablation "w/o Prop. 3.1" (Table 5): lm row is k'_c, b'_c = 0 */
  HILS_SCORE_EXACT = 2,         /* naive-BSA exact chunk log-mass log sum_{j in chunk} exp(s_ij)
                                   (section 2.1), from the token query q: an O(N^2 d) test mode,
                                   prefill only (generic kernels); no summaries, lm_q unused */
  HILS_SCORE_MEAN_POOL = 3      /* mean-pooled key (section 2.2 equation; ablation "w/ mean
                                   pooling", Table 5): k'_c = mean of the chunk's keys,
                                   b'_c = ln S (Proposition 3.1 at a zero landmark query);
                                   lm_q unused */
} hils_score_mode;

/* flags */
#define HILS_FLAG_GENERIC 1u   /* prefill: force the generic (vector-ALU) kernels */
#define HILS_FLAG_UNION 2u     /* prefill, MFMA path: attention by query block over the
                                  union of the block's chunks (section 4.2 of the
                                  pages) instead of the default per-chunk buckets */

typedef struct hils_cfg {
  int32_t B;      /* batch */
  int32_t N;      /* prefill: sequence length; decode: KV-cache capacity */
  int32_t Hq;     /* query heads */
  int32_t Hkv;    /* key/value heads; Hq % Hkv == 0 */
  int32_t d;      /* head dim, 1..256 */
  int32_t S;      /* chunk size, 1..64 */
  int32_t W;      /* window size >= 1 */
  int32_t K;      /* top-K chunks, 1..128 */
  int32_t dtype;  /* hils_dtype */
  int32_t mode;   /* hils_score_mode */
  float scale;    /* logit scale; 0 selects 1/sqrt(d) */
  uint32_t flags; /* HILS_FLAG_* */
} hils_cfg;

/* Bytes of workspace hils_prefill (is_decode = 0) or hils_decode (is_decode = 1)
 * needs for this configuration; 0 when the configuration is invalid. */
size_t hils_workspace_bytes(const hils_cfg* cfg, int is_decode);

/* Chunk summaries for chunks c0 <= c < c1 (section 3, Proposition 3.1):
 *   p_j = softmax_{j in chunk c}(scale * lm_q[b,h,c] . k[b,h/G,j]),
 *   k_sum[b,h,c] = sum_j p_j k_j (rounded once, to nearest-even, to dtype),
 *   b_sum[b,h,c] = -sum_j p_j log p_j (rounded once to fp32).
 * Computed in double precision.  Mode LANDMARK_KEY copies lm_q into k_sum and
 * writes b_sum = 0.  Requires 0 <= c0 <= c1 <= floor(N/S).  Used to build or
 * extend a decode summary cache as chunks complete. */
hils_status hils_summarize(const hils_cfg* cfg, const void* k, const void* lm_q,
                           int32_t c0, int32_t c1, void* k_sum, float* b_sum, void* stream);

/* Prefill: HiLS output for every position of every sequence.
 *   q_route  : routing query (low-rank query calibration, section 4.1) used only
 *              in the chunk scores; NULL means q.
 *   out      : [B][Hq][N][d], dtype.
 *   sel      : optional output of the selected chunk ids (NULL: kept in workspace).
 *   k_sum, b_sum : optional outputs of the summaries of all floor(N/S) chunks
 *              (both NULL or both non-NULL).
 * Requires 1 <= K, 1 <= W, N >= 1. */
hils_status hils_prefill(const hils_cfg* cfg, const void* q, const void* q_route,
                         const void* k, const void* v, const void* lm_q, void* out,
                         int32_t* sel, void* k_sum, float* b_sum,
                         void* ws, size_t ws_bytes, void* stream);

/* Single-step decode: for each sequence b the new token is already in the
 * cache at position T_b - 1 (T_b = seqlen[b], 1 <= T_b <= N, device int32[B]),
 * and the query q[b,:,0,:] is that token's query.  k_sum/b_sum hold the
 * summaries of every complete chunk (from hils_summarize); only chunks
 * c < |C_{T_b-1}| are read.  out: [B][Hq][1][d]; sel optional [B][Hkv][K].
 * B * Hq above 65535 returns HILS_E_UNSUPPORTED (also for the multi-query and
 * paged decode below). */
hils_status hils_decode(const hils_cfg* cfg, const void* q, const void* q_route,
                        const void* k_cache, const void* v_cache, const int32_t* seqlen,
                        const void* k_sum, const float* b_sum, void* out, int32_t* sel,
                        void* ws, size_t ws_bytes, void* stream);

/* Allocation-free single-step decode, for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, result and errors
 * as hils_decode without ws/ws_bytes; the scratch comes from a buffer of
 * HILS_NOALLOC_SCRATCH_BYTES that the library keeps in device memory, one per
 * GPU it runs on (held until the process ends; its address is looked up once
 * per device, on the first call with that device current).  The call
 * allocates nothing.  Configurations whose decode workspace
 * (hils_workspace_bytes(cfg, 1)) exceeds HILS_NOALLOC_SCRATCH_BYTES return
 * HILS_E_WORKSPACE before anything is enqueued.  Every call on one GPU shares
 * that GPU's buffer: calls that overlap in time on one GPU (different streams
 * or host threads without ordering between them) race and give undefined
 * results; calls on one stream are ordered and safe.  The buffer keeps the
 * last call's contents; the decode kernels need no zeroed scratch. */
#define HILS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hils_status hils_decode_noalloc(const hils_cfg* cfg, const void* q, const void* q_route,
                                const void* k_cache, const void* v_cache, const int32_t* seqlen,
                                const void* k_sum, const float* b_sum, void* out, int32_t* sel,
                                void* stream);

/* Multi-query decode: M new tokens of each sequence (draft or verification
 * tokens, 1 <= M <= HILS_MAX_DECODE_QUERIES) are already in the cache at
 * positions T_b - M .. T_b - 1 (T_b = seqlen[b] >= M), and query m is the
 * query of the token at position T_b - M + m.  Each query is the prefill row
 * at its own position (section 3; causal among the new tokens: its window ends
 * at its own position, and its candidate chunks are the complete chunks
 * before its window).  Layouts:
 *   q, q_route, out : [B][Hq][M][d];   sel (optional) : [B][Hkv][M][K].
 * k_sum/b_sum as for hils_decode.  The chunk-summary read, the dominant
 * traffic, is shared by up to 4 queries of a sequence.  A position below 0
 * (seqlen < M) is evaluated at position 0.  M = 1 is hils_decode.  Workspace:
 * hils_decode_multi_workspace_bytes(cfg, M) (0 for an invalid cfg or M). */
#define HILS_MAX_DECODE_QUERIES 16
size_t hils_decode_multi_workspace_bytes(const hils_cfg* cfg, int32_t M);
hils_status hils_decode_multi(const hils_cfg* cfg, int32_t M, const void* q, const void* q_route,
                              const void* k_cache, const void* v_cache, const int32_t* seqlen,
                              const void* k_sum, const float* b_sum, void* out, int32_t* sel,
                              void* ws, size_t ws_bytes, void* stream);

/* Paged KV cache with one chunk per page (the pages' serving setup, section
 * 7.1: KV page size equal to the chunk size S).  Physical page p holds
 *   k_pages, v_pages : [num_pages][Hkv][S][d]   the S tokens of one chunk,
 *   lm_pages         : [num_pages][Hq][d]       that chunk's landmark queries,
 *   k_sum_pages      : [num_pages][Hq][d]       its summary keys (dtype),
 *   b_sum_pages      : [num_pages][Hq]          its entropy biases (fp32).
 * page_table [B][max_pages] int32 maps chunk c of sequence b to its page; only
 * the entries of chunks that hold tokens of the sequence are read, and page
 * ids are clamped into [0, num_pages) on the device, so any table content
 * stays in bounds (a wrong id gives a wrong result, never a fault).
 * cfg->N is the per-sequence token capacity (N <= max_pages * S).
 *
 * hils_summarize_paged: summaries (as hils_summarize) of the npages pages
 * listed in pages[] (device int32), written into their own page slots.
 * hils_decode_paged: as hils_decode, with every KV, summary and window access
 * going through the page table; the workspace is hils_workspace_bytes(cfg, 1).
 * Both enqueue kernels only (no allocation, no memset, no host sync), so a
 * decode step can be captured into a HIP graph and replayed. */
hils_status hils_summarize_paged(const hils_cfg* cfg, const void* k_pages, const void* lm_pages,
                                 const int32_t* pages, int32_t npages, int32_t num_pages,
                                 void* k_sum_pages, float* b_sum_pages, void* stream);
hils_status hils_decode_paged(const hils_cfg* cfg, const void* q, const void* q_route,
                              const void* k_pages, const void* v_pages, int32_t num_pages,
                              const int32_t* page_table, int32_t max_pages, const int32_t* seqlen,
                              const void* k_sum_pages, const float* b_sum_pages, void* out,
                              int32_t* sel, void* ws, size_t ws_bytes, void* stream);

/* Prefill backward (training through HiLS attention).  Gradients of
 * L = sum(dout * out) of hils_prefill, with the top-K selection held fixed (the
 * forward's sel [B][Hkv][N][K]; a hard choice has no gradient) and every other
 * step differentiated (section 3): the chunk-level fusion softmax into the
 * chunk scores and the window log-mass, the chunk and window softmaxes into
 * q, k, v, the routing equation into q_route (or q), k'_c and b'_c, and the
 * Proposition 3.1 summary softmax into the landmark queries and k (modes
 * LANDMARK_KEY: dlm = dk'; MEAN_POOL: dk += dk'/S, no dlm; EXACT unsupported).
 *   dout            : [B][Hq][N][d], dtype;
 *   k_sum, b_sum    : the forward's summaries, or both NULL to recompute them;
 *   dq, dk, dv      : fp32 outputs shaped like q, k, v (fully written);
 *   dq_route        : fp32 [B][Hq][N][d] iff q_route is given (the token query
 *                     then gets only the attention part);
 *   dlm             : fp32 [B][Hq][N/S][d] (may be NULL in MEAN_POOL mode).
 * The kernels use no floating-point atomics, so results are deterministic.
 * Supports d <= 128 (a multiple of 64 for bf16, of 32 for fp32), S <= 64,
 * G <= 8, K <= 128 and windows whose G head rows of logits fit in LDS
 * (otherwise HILS_E_UNSUPPORTED, and hils_prefill_backward_workspace_bytes
 * returns 0).  For bf16 with d in {64, 128} and S a multiple of 16 the
 * attention products run on the matrix cores in query slices whose per-slice
 * partials fit 4 GiB of workspace; the environment variable
 * HILS_BWD_SLICE_QUERIES, a positive query count, caps the slice (the
 * workspace query and the call must see the same value).
 */
size_t hils_prefill_backward_workspace_bytes(const hils_cfg* cfg);
hils_status hils_prefill_backward(const hils_cfg* cfg, const void* q, const void* q_route,
                                  const void* k, const void* v, const void* lm_q, const void* dout,
                                  const int32_t* sel, const void* k_sum, const float* b_sum,
                                  float* dq, float* dq_route, float* dk, float* dv, float* dlm,
                                  void* ws, size_t ws_bytes, void* stream);

const char* hils_strerror(hils_status status);
int hils_abi_version(void);

/* Kernel timing for measurement tools (not part of the method).
 * hils_profile_enable(1): from then on every kernel the library enqueues is
 * bracketed by two HIP events recorded on its stream.  hils_profile_read()
 * copies the names (static strings) and durations in milliseconds of the
 * kernels enqueued since the previous read into names[]/ms[] (at most cap
 * entries), returns how many kernels were recorded (which may exceed cap),
 * and forgets them; the caller must have synchronised the streams first.
 * While enabled the library keeps this process-wide record (guarded by a
 * mutex); hils_profile_enable(0) turns it off and releases the events. */
void hils_profile_enable(int on);
int hils_profile_read(const char** names, float* ms, int cap);

#ifdef __cplusplus
}
#endif
#endif /* HILS_H */
