/*
 * dsa.h — C ABI of the DeepSeek Sparse Attention (DSA) hot path for AMD
 * Instinct MI355X (gfx950).
 *
 * The path has three stages (ouchyi.pink post on DSA, the DSA paragraph;
 * tenelement.pl article "DeepSeek V3.2-Exp Cuts Long-Context Costs with
 * DeepSeek Sparse Attention (DSA) While Maintaining Benchmark Parity",
 * section "Architektura DeepSeek V3.2-Exp: Od MoE do DSA"):
 *
 *   1. dsa_indexer     — the lightning indexer: a few FP8 heads score every
 *                        cached token for each query row,
 *                          I[t,s] = k_scale[s] * sum_j (w[t,j]*q_scale[t]) * ReLU(q8[t,j] . k8[s])
 *   2. dsa_topk        — keep k tokens per query row (k = 2048 on the pages,
 *                        whatever the context length),
 *   3. dsa_sparse_attn — softmax attention over only the kept tokens, in MQA
 *                        form: all query heads read one shared latent KV row
 *                        per token (same article, same section; degnora.com
 *                        "DeepSeekV3, Farkı Ne?", section "MLA — Multi-Latent
 *                        Attention").
 *   dsa_decode (one query per sequence) and dsa_prefill (query rows per
 *   sequence) chain the three without any host round trip between the stages (sider.ai "Sparse attention that isn't
 *   sparse thinking", sections "Uyarılar" and "Dağıtım Gerçekliği": selection
 *   that bounces between CPU and GPU, or launch overhead, eats the gain).
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller; the library
 *   never allocates, frees, copies to the host or synchronises.  All work is
 *   enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 *   buffers must stay alive until that work has completed.
 * - Query rows are grouped by sequence.  Sequence b has seq_lens[b] cached
 *   tokens; its query rows are its LAST nq_b tokens, so row i of sequence b
 *   sits at position p = seq_lens[b] - nq_b + i and sees tokens 0..p
 *   (causal, itself included).  With q_start == NULL there is exactly one
 *   query row per sequence (row b, position seq_lens[b]-1): decode.
 * - Caches are contiguous per sequence or paged.  Token s of sequence b is
 *   token row r of a cache, where r = b*seq_stride + s when block_table is
 *   NULL, else r = block_table[b*max_blocks + s/block_size]*block_size +
 *   s%block_size.  Its bytes start at data + r*row_stride.  One batch (and so
 *   one block table) describes all caches of a call.
 * - Scalars: FP8 is OCP e4m3fn bytes; bf16 is passed as its 16-bit pattern.
 * - Errors: arguments are validated on the host before anything is enqueued;
 *   a non-OK status leaves every output untouched and dsa_last_error()
 *   (thread-local) describes it.  DSA_ERR_HIP reports a failed launch.
 *   Device faults surface at the caller's next synchronisation.  Nothing is
 *   printed, thrown or aborted across this interface.
 * - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,        /* a required pointer is NULL */
  DSA_ERR_SHAPE = 2,       /* inconsistent sizes, strides or bounds */
  DSA_ERR_UNSUPPORTED = 3, /* valid, but no kernel for these sizes */
  DSA_ERR_ALIGN = 4,       /* pointer or stride not aligned as required */
  DSA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than dsa_workspace_size() */
  DSA_ERR_HIP = 6          /* a HIP launch failed */
} dsa_status;

/* Token rows of one cache (index keys, key scales, latent KV, separate V). */
typedef struct dsa_cache {
  const void* data;   /* device pointer to token row 0 */
  int64_t row_stride; /* bytes between consecutive token rows */
  int64_t seq_stride; /* contiguous caches: token rows between sequences (unused when paged) */
} dsa_cache;

/* Batch geometry: sequences, query rows and (optionally) the page table. */
typedef struct dsa_batch {
  int32_t num_seqs;           /* B >= 1 */
  int32_t num_rows;           /* T: total query rows (== B when q_start is NULL) */
  int32_t max_q;              /* host bound on nq_b (1 when q_start is NULL) */
  int32_t max_len;            /* host bound on seq_lens[b]; sizes grids and checks ld */
  const int32_t* seq_lens;    /* device [B]: 1 <= seq_lens[b] <= max_len */
  const int32_t* q_start;     /* device [B+1] row offsets, or NULL (one row per sequence) */
  const int32_t* block_table; /* device [B, max_blocks] physical block ids, or NULL */
  int32_t max_blocks;         /* paged: entries per table row */
  int32_t block_size;         /* paged: tokens per block, a power of two >= 16 */
} dsa_batch;

/*
 * dsa_indexer — lightning-indexer scores for every query row and every token
 * it may see (ouchyi.pink post, DSA paragraph: few heads, FP8, cheap;
 * tenelement.pl article, section "Architektura DeepSeek V3.2-Exp: Od MoE do
 * DSA": logits per context token with a ReLU).
 *   q8      [T, H_I, d_I] e4m3fn, row-major
 *   q_scale [T] fp32 per-token dequantisation scale, or NULL (= 1)
 *   w       [T, H_I] fp32 head weights, 16-byte aligned
 *   kidx    d_I e4m3fn bytes per token; data and row_stride 16-byte aligned
 *   kscale  one fp32 per token (row_stride >= 4), or NULL (= 1)
 *   scores  [T, ld] fp32 out: scores[t*ld + s] for s <= p_t; entries past
 *           p_t are unspecified.  ld >= max_len.
 * Supported: H_I a multiple of 4 in [4, 64], d_I in {32, 128}.
 */
dsa_status dsa_indexer(const dsa_batch* batch, const uint8_t* q8, const float* q_scale,
                       const float* w, const dsa_cache* kidx, const dsa_cache* kscale,
                       int H_I, int d_I, float* scores, int64_t ld, void* stream);

/*
 * dsa_topk — per query row, the first min(k, p+1) tokens in the order
 * (score descending, token index ascending; -0.0 equals +0.0), written in
 * ascending token order and padded with -1 (ouchyi.pink post, DSA paragraph:
 * a fixed number of tokens per query; digitalreport.com.tr article "DeepSeek
 * V3.2-exp: daha ucuz uzun bağlamlı AI": fine-grained token selection).
 *   scores  [T, ld] fp32 as written by dsa_indexer (NaN not allowed)
 *   idx     [T, k] int32 out
 *   workspace: dsa_workspace_size(DSA_WS_TOPK, ...) bytes, 256-byte aligned
 * Supported: 1 <= k <= 4096.
 */
dsa_status dsa_topk(const dsa_batch* batch, const float* scores, int64_t ld, int k,
                    int32_t* idx, void* workspace, size_t ws_bytes, void* stream);

/*
 * dsa_sparse_attn — softmax attention of H query heads over the selected
 * tokens only, all heads sharing one KV row per token (MQA over the latent
 * cache; tenelement.pl article, section "Architektura DeepSeek V3.2-Exp: Od
 * MoE do DSA"; degnora.com "DeepSeekV3, Farkı Ne?", section "MLA —
 * Multi-Latent Attention").
 *   q     [T, H, D] bf16
 *   kv    D bf16 per token (K is the whole row); 16-byte aligned rows
 *   v     D_v bf16 per token, or NULL: V is the first D_v dims of the kv row
 *         (a separate V cache is supported for D = 64 only)
 *   idx   [T, k] int32 token indices; -1, and any index outside [0, p_t],
 *         marks an unused slot
 *   out   [T, H, D_v] bf16;  lse [T, H] fp32 natural-log softmax denominator, or NULL
 *   workspace: dsa_workspace_size(DSA_WS_ATTN, ...) bytes (0 is valid when it says 0)
 * A row whose k slots are all -1 gets out = 0 and lse = -inf.
 * Supported: (D, D_v) in {(64, 64), (576, 512)}, 1 <= H <= 128, 1 <= k <= 4096.
 */
dsa_status dsa_sparse_attn(const dsa_batch* batch, const uint16_t* q, const dsa_cache* kv,
                           const dsa_cache* v, int H, int D, int D_v, float scale,
                           const int32_t* idx, int k, uint16_t* out, float* lse,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * dsa_decode — the whole path for one query per sequence (q_start must be
 * NULL), enqueued back to back with no host synchronisation: indexer scores
 * (kept in the workspace), top-k, sparse attention.
 * Arguments as in the three calls above; idx_out [B, k] receives the
 * selected indices when not NULL.  Workspace: dsa_workspace_size(
 * DSA_WS_DECODE, ...) bytes, 256-byte aligned.
 * Short contexts: when batch->max_len <= k every query selects all of its
 * tokens (the selection is then independent of the scores), so the indexer
 * is skipped, the identity selections are written and the attention is
 * dense (tenelement.pl article, "Architektura DeepSeek V3.2-Exp: Od MoE do
 * DSA": dense attention at short lengths).
 */
dsa_status dsa_decode(const dsa_batch* batch, const uint8_t* q8, const float* q_scale,
                      const float* w, const dsa_cache* kidx, const dsa_cache* kscale,
                      int H_I, int d_I, int k, const uint16_t* q, const dsa_cache* kv,
                      const dsa_cache* v, int H, int D, int D_v, float scale,
                      uint16_t* out, float* lse, int32_t* idx_out,
                      void* workspace, size_t ws_bytes, void* stream);

/*
 * dsa_prefill — the same fused path for a batch of query rows per sequence
 * (q_start must be set): indexer over every causal (row, token) pair, top-k,
 * sparse attention, on one stream.  Arguments as in dsa_decode; out, lse and
 * idx_out have num_rows rows.  Workspace: dsa_workspace_size(
 * DSA_WS_PREFILL, ...) bytes, 256-byte aligned (it holds the [num_rows,
 * max_len] score matrix).  The short-context shortcut of dsa_decode applies:
 * with max_len <= k no scores are computed and the attention is dense causal.
 * Errors: as dsa_decode; DSA_ERR_SHAPE when q_start is NULL.
 */
dsa_status dsa_prefill(const dsa_batch* batch, const uint8_t* q8, const float* q_scale,
                       const float* w, const dsa_cache* kidx, const dsa_cache* kscale,
                       int H_I, int d_I, int k, const uint16_t* q, const dsa_cache* kv,
                       const dsa_cache* v, int H, int D, int D_v, float scale,
                       uint16_t* out, float* lse, int32_t* idx_out,
                       void* workspace, size_t ws_bytes, void* stream);

/*
 * dsa_prefill_streaming — dsa_prefill without the [num_rows, max_len] score
 * matrix: the top-k selection streams out of the indexer (sider.ai "Sparse
 * attention that isn't sparse thinking", section "Matematik, Minimalist
 * Sürüm": selection that stays cache-aware).  Per row, a threshold on the
 * order (score desc, token asc) is taken from the scores of every 32nd token;
 * the indexer then keeps only the (score, token) pairs at or above it, and the
 * exact top-k is selected among those.  A row left with fewer than k such
 * pairs, or more than the candidate capacity, is recomputed exactly (slower,
 * same result).  The selection, and therefore out/lse/idx_out, equals
 * dsa_prefill's bit for bit.  Arguments and errors as dsa_prefill, plus
 * DSA_ERR_UNSUPPORTED unless d_I = 128, k <= 2048 and max_len <= 262144.
 * Workspace: dsa_workspace_size(DSA_WS_PREFILL_STREAM, ...) bytes, 256-byte
 * aligned: O(num_rows * (max_len / 32 + 56 * rank)) with rank = max(64,
 * ceil(k/16)), instead of num_rows * max_len scores.  Stage events as
 * dsa_prefill (the indexer stage covers the sampled and the filtered pass).
 */
dsa_status dsa_prefill_streaming(const dsa_batch* batch, const uint8_t* q8, const float* q_scale,
                                 const float* w, const dsa_cache* kidx, const dsa_cache* kscale,
                                 int H_I, int d_I, int k, const uint16_t* q, const dsa_cache* kv,
                                 const dsa_cache* v, int H, int D, int D_v, float scale,
                                 uint16_t* out, float* lse, int32_t* idx_out,
                                 void* workspace, size_t ws_bytes, void* stream);

/*
 * dsa_set_stage_events — opt-in stage timing for the NEXT dsa_decode,
 * dsa_prefill, dsa_prefill_streaming or dsa_indexer_warmup call on this
 * thread (for profiling
 * tools; the stages are the ones the pages name: indexer, selection, core
 * attention).  `events` holds `count` >= 4 hipEvent_t handles created by the
 * caller (at most 6 are used); that call records them on its stream:
 *   dsa_decode / dsa_prefill / dsa_prefill_streaming (4 events):
 *     events[0] before the indexer (after the workspace clear),
 *     events[1] after the indexer, events[2] after the top-k,
 *     events[3] after the attention (and its split combine);
 *   dsa_indexer_warmup (the first min(count, 6)):
 *     events[0] before the indexer, events[1] after it, events[2] after the
 *     dense log-sum-exp pass, events[3] after the target/KL pass,
 *     events[4] after dq/dw, events[5] after dk.
 * The registration is consumed by that one call.  NULL clears it.
 * Errors: DSA_ERR_SHAPE if count < 4, DSA_ERR_NULL if one of the first
 * min(count, 6) is NULL.  A failed record returns DSA_ERR_HIP from the call.
 */
dsa_status dsa_set_stage_events(void* const* events, int count);

/*
 * dsa_indexer_warmup — the indexer's warm-up objective and its gradients
 * (tenelement.pl article "DeepSeek V3.2-Exp Cuts Long-Context Costs with
 * DeepSeek Sparse Attention (DSA) While Maintaining Benchmark Parity",
 * section "Proces Treningu DSA: Od Warm-up do Sparsity": with the main model
 * frozen, the indexer is fitted by a KL divergence to the dense attention
 * distribution summed over the heads).  For query row t at position p:
 *   target  a[s] = (1/H) sum_h softmax_s(scale * q[t,h] . K[s]),  s <= p
 *   model   P[s] = softmax_s(I[t,s]),  I = the dsa_indexer score
 *   loss[t] = sum_s a[s] (log a[s] - log P[s])
 * and, for the pointers that are not NULL, the gradients of sum_t loss[t]
 * with respect to the dequantised indexer query q_scale*q8 (dq), the head
 * weights (dw) and the dequantised index keys k_scale*k8 (dk).  ReLU'(0) is
 * taken as 0.  The dense side (q, kv) gets no gradient (it is frozen).
 *   q, kv   as dsa_sparse_attn with D = 576 (K is the whole row; V is unused)
 *   q8, q_scale, w, kidx, kscale   as dsa_indexer, d_I = 128, H_I in {32, 64}
 *   loss    [T] fp32 out
 *   dq      [T, H_I, 128] fp32 out, or NULL
 *   dw      [T, H_I] fp32 out, or NULL
 *   dk      [B, max_len, 128] fp32 out (token s of sequence b at row
 *           b*max_len + s; tokens at or past seq_lens[b] get 0), or NULL;
 *           16-byte aligned
 *   workspace: dsa_workspace_size(DSA_WS_WARMUP, batch, 0, H, 0) bytes,
 *           256-byte aligned
 * Batch: q_start must be set (rows per sequence, as dsa_prefill) and the
 * caches contiguous (block_table NULL), else DSA_ERR_SHAPE / DSA_ERR_UNSUPPORTED.
 * Supported: D = 576, H a multiple of 16 in [16, 128].  Results are
 * deterministic (fixed-order reductions, no float atomics).
 */
dsa_status dsa_indexer_warmup(const dsa_batch* batch, const uint16_t* q, const dsa_cache* kv, int H, int D,
                              float scale, const uint8_t* q8, const float* q_scale, const float* w,
                              const dsa_cache* kidx, const dsa_cache* kscale, int H_I, int d_I,
                              float* loss, float* dq, float* dw, float* dk,
                              void* workspace, size_t ws_bytes, void* stream);

/*
 * dsa_set_attn_splits — tuning and testing hook for the attention stage of the
 * calls that follow on this thread (dsa_sparse_attn, dsa_decode, dsa_prefill,
 * dsa_prefill_streaming, and dsa_workspace_size for them): the k selected
 * slots of each query row are divided among `nsplit` workgroups whose
 * partial softmax results are merged by their log-sum-exp (the split-K form
 * of the online softmax).  0 restores the automatic choice.  A count above
 * what the slots allow is clamped (at most one split per 64 slots).  The
 * result equals the unsplit one up to the rounding of the partials; set the
 * same value before sizing and before calling.
 * Errors: DSA_ERR_SHAPE if nsplit is outside [0, 4096].
 */
dsa_status dsa_set_attn_splits(int nsplit);

/*
 * dsa_set_indexer_fp8 — tuning and testing hook for the streaming prefill
 * (dsa_prefill_streaming) calls that follow on this thread.  1: the filtered
 * indexer pass contracts the FP8 query and key bytes on the FP8 matrix-core
 * form (the pages' FP8 lightning indexer: ouchyi.pink post, DSA paragraph;
 * tenelement.pl "DeepSeek V3.2-Exp Cuts Long-Context Costs", section
 * "Architektura DeepSeek V3.2-Exp: Od MoE do DSA"); each candidate keeps its
 * FP8 estimate and error bound, and only the candidates whose bounds straddle
 * the row's k-th score are scored exactly afterwards; 0 (the default, the
 * faster one on gfx950): every pair is scored exactly in the filtered pass.
 * The selection is the same either way.
 * Errors: DSA_ERR_SHAPE if `on` is not 0 or 1.
 */
dsa_status dsa_set_indexer_fp8(int on);

/*
 * dsa_decode_noalloc — dsa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Arguments, results and errors as dsa_decode, without
 * the workspace: it uses a static device array of
 * dsa_noalloc_scratch_bytes() bytes (256 MiB) instead, one per GPU, held
 * from the library's first use of that GPU until the process ends.  The
 * first call on a device looks the array up (hipGetSymbolAddress, with that
 * device current); no call allocates or frees memory.
 *   DSA_ERR_WORKSPACE when dsa_workspace_size(DSA_WS_DECODE, ...) for the
 *   batch exceeds the array (use dsa_decode with a caller workspace then).
 * All calls on one GPU share its array, which keeps the last call's contents
 * (everything that must start at zero is cleared by each call): calls that
 * overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller.
 */
dsa_status dsa_decode_noalloc(const dsa_batch* batch, const uint8_t* q8, const float* q_scale,
                              const float* w, const dsa_cache* kidx, const dsa_cache* kscale,
                              int H_I, int d_I, int k, const uint16_t* q, const dsa_cache* kv,
                              const dsa_cache* v, int H, int D, int D_v, float scale,
                              uint16_t* out, float* lse, int32_t* idx_out, void* stream);

/* Size in bytes of dsa_decode_noalloc's static scratch array (host-only). */
size_t dsa_noalloc_scratch_bytes(void);

/* Which call dsa_workspace_size() sizes. */
enum { DSA_WS_TOPK = 1, DSA_WS_ATTN = 2, DSA_WS_DECODE = 3, DSA_WS_PREFILL = 4, DSA_WS_WARMUP = 5,
       DSA_WS_PREFILL_STREAM = 6 };

/*
 * Workspace bytes `entry` needs for this batch (host-only; no device call).
 * H and D_v matter for DSA_WS_ATTN / DSA_WS_DECODE / DSA_WS_PREFILL /
 * DSA_WS_PREFILL_STREAM only (the last also needs k <= 2048);
 * DSA_WS_WARMUP takes H (the dense heads) and ignores k and D_v.  Returns 0 when the
 * call needs none, and (size_t)-1 for invalid arguments.
 */
size_t dsa_workspace_size(int entry, const dsa_batch* batch, int k, int H, int D_v);

/* Text for the last non-OK status returned on this thread ("" if none). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
