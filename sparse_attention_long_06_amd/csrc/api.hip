// C ABI of the DSA hot path: host-side validation, workspace layout and the
// launch sequence of each entry point.  Every argument check happens before
// the first HIP call, so an invalid call has no device side effects.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "dsa.h"
#include "dsa_kernels.h"

using namespace dsa;

namespace {

thread_local std::string g_err;
constexpr int kMaxStageEvents = 6;
thread_local hipEvent_t g_stage_events[kMaxStageEvents] = {};
thread_local int g_stage_count = 0;
thread_local bool g_stage_armed = false;
thread_local int g_force_splits = 0;   // dsa_set_attn_splits: 0 = the planner's choice
thread_local bool g_indexer_fp8 = false;  // dsa_set_indexer_fp8

dsa_status fail(dsa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

dsa_status ok() {
  g_err.clear();
  return DSA_OK;
}

#define CHECK(cond, status, ...) \
  do {                           \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

#define LAUNCH(expr, what)                                                              \
  do {                                                                                  \
    const hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e_)); \
  } while (0)

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
int ilog2(int64_t x) { int r = 0; while ((int64_t(1) << r) < x) ++r; return r; }

dsa_status check_batch(const dsa_batch* b) {
  CHECK(b, DSA_ERR_NULL, "batch is NULL");
  CHECK(b->seq_lens, DSA_ERR_NULL, "batch->seq_lens is NULL");
  CHECK(b->num_seqs >= 1 && b->num_seqs <= 65535, DSA_ERR_SHAPE, "num_seqs %d outside [1, 65535]", b->num_seqs);
  CHECK(b->max_len >= 1, DSA_ERR_SHAPE, "max_len %d < 1", b->max_len);
  if (!b->q_start) {
    CHECK(b->num_rows == b->num_seqs, DSA_ERR_SHAPE,
          "num_rows %d != num_seqs %d with one query row per sequence", b->num_rows, b->num_seqs);
  } else {
    CHECK(b->num_rows >= 0, DSA_ERR_SHAPE, "num_rows %d < 0", b->num_rows);
    CHECK(b->max_q >= 1 && b->max_q <= b->max_len, DSA_ERR_SHAPE, "max_q %d outside [1, max_len]", b->max_q);
  }
  if (b->block_table) {
    CHECK(pow2(b->block_size) && b->block_size >= 16 && b->block_size <= (1 << 20), DSA_ERR_SHAPE,
          "block_size %d is not a power of two in [16, 2^20]", b->block_size);
    CHECK(b->max_blocks >= 1 && (int64_t)b->max_blocks * b->block_size >= b->max_len, DSA_ERR_SHAPE,
          "max_blocks %d * block_size %d < max_len %d", b->max_blocks, b->block_size, b->max_len);
  }
  return DSA_OK;
}

dsa_status check_cache(const dsa_batch* b, const dsa_cache* c, const char* name, int64_t row_bytes, size_t align) {
  CHECK(c && c->data, DSA_ERR_NULL, "%s cache is NULL", name);
  CHECK(c->row_stride >= row_bytes, DSA_ERR_SHAPE, "%s row_stride %lld < %lld bytes", name,
        (long long)c->row_stride, (long long)row_bytes);
  CHECK(aligned(c->data, align) && c->row_stride % (int64_t)align == 0, DSA_ERR_ALIGN,
        "%s data/row_stride not %zu-byte aligned", name, align);
  if (!b->block_table)
    CHECK(c->seq_stride >= b->max_len, DSA_ERR_SHAPE, "%s seq_stride %lld < max_len %d", name,
          (long long)c->seq_stride, b->max_len);
  return DSA_OK;
}

Geo make_geo(const dsa_batch* b) {
  Geo g;
  g.seq_lens = b->seq_lens;
  g.q_start = b->q_start;
  g.block_table = b->block_table;
  g.max_blocks = b->max_blocks;
  g.block_shift = b->block_table ? ilog2(b->block_size) : 0;
  g.num_seqs = b->num_seqs;
  g.num_rows = b->num_rows;
  return g;
}

Cache make_cache(const dsa_cache* c) {
  Cache r;
  r.data = c ? static_cast<const char*>(c->data) : nullptr;
  r.row_stride = c ? c->row_stride : 0;
  r.seq_stride = c ? c->seq_stride : 0;
  return r;
}

// ---------------------------------------------------------------- workspace plans

struct TopkPlan {
  bool split = false;
  int nslices = 0, slice = 0;
  size_t off_hist = 0, off_hist2 = 0, off_meta = 0, off_slice = 0, off_lists = 0, bytes = 0;
  size_t zero_words = 0;  // the two histograms, from off_hist
};

TopkPlan plan_topk(int T, int max_len, int k) {
  TopkPlan p;
  if (T > kTopkSplitMaxRows || max_len <= k || T == 0) return p;
  p.split = true;
  // slices per row: ~512 workgroups over the batch, and at least 16 per row so
  // that rows shorter than max_len (mixed-length batches) still spread out
  const int target = max((kTopkSplitMaxRows + T - 1) / T, 16);
  int slice = (int)round_up((max_len + target - 1) / target, 1024);
  if (slice < 1024) slice = 1024;
  int ns = (max_len + slice - 1) / slice;
  if (ns > kTopkMaxSlices) {
    slice = (int)round_up((max_len + kTopkMaxSlices - 1) / kTopkMaxSlices, 1024);
    ns = (max_len + slice - 1) / slice;
  }
  p.slice = slice;
  p.nslices = ns;
  size_t o = 0;
  p.off_hist = o; o += (size_t)T * kBins1 * 4;
  p.off_hist2 = o; o += (size_t)T * kBins1 * 4;
  p.zero_words = o / 4;
  p.off_meta = o; o += (size_t)T * 16;
  p.off_slice = o; o += (size_t)T * ns * 4;
  o = (size_t)round_up((int64_t)o, 256);
  p.off_lists = o; o += (size_t)T * ns * slice * 8;
  p.bytes = (size_t)round_up((int64_t)o, 256);
  return p;
}

struct AttnPlan {
  int nsplit = 1, per_split = 0;
  size_t off_o = 0, off_lse = 0, bytes = 0;
};

AttnPlan plan_attn(int T, int k, int H, int D_v) {
  AttnPlan p;
  const int blocks = (k + kAttnBlock - 1) / kAttnBlock;
  int ns = 1;
  if (g_force_splits > 0) {
    ns = g_force_splits < blocks ? g_force_splits : blocks;
  } else if (T > 0 && T < 256) {
    while (ns < blocks && (int64_t)T * ns < 256) ns *= 2;
    if (ns > blocks) ns = blocks;
  }
  while ((k + ns - 1) / ns > kAttnMaxSplit) ++ns;
  int per = (int)round_up((k + ns - 1) / ns, kAttnBlock);
  ns = (k + per - 1) / per;
  p.nsplit = ns;
  p.per_split = per;
  if (ns > 1) {
    size_t o = 0;
    p.off_o = o; o += (size_t)T * ns * H * D_v * 2;
    o = (size_t)round_up((int64_t)o, 256);
    p.off_lse = o; o += (size_t)T * ns * H * 4;
    p.bytes = (size_t)round_up((int64_t)o, 256);
  }
  return p;
}

// Workspace of the fused entry points (dsa_decode, dsa_prefill) over T query
// rows.  When every row sees at most k tokens (max_len <= k) the selection is
// every prior token: no scores, no indexer, and the top-k launch only writes
// the identity lists.
// Decode indexer chunking: about 2048 workgroups over the batch (short enough
// chunks that the last wave of workgroups leaves little of the device idle).
int decode_chunk(int max_len, int num_seqs) {
  const int64_t c = round_up(((int64_t)max_len * num_seqs + 2047) / 2048, 16);
  return (int)(c < 256 ? 256 : (c > kIdxDecodeChunk ? kIdxDecodeChunk : c));
}

// The fused decode's chunk-candidate selection: per chunk of kCandChunk
// tokens of a row its candidate list (key, token), count and cut key.
struct CandPlan {
  bool ok = false;
  int nchunks = 0;
  size_t off_cand = 0, off_cnt = 0, off_cut = 0, bytes = 0;
};

CandPlan plan_cand(int B, int max_len, int k) {
  CandPlan p;
  if (max_len <= k) return p;
  p.nchunks = (max_len + kCandChunk - 1) / kCandChunk;
  if (p.nchunks > kCandMaxChunks || (int64_t)B * p.nchunks >= ((int64_t)1 << 31)) return p;
  p.ok = true;
  size_t o = 0;
  p.off_cand = o; o += (size_t)B * p.nchunks * kCandChunk * 8;
  o = (size_t)round_up((int64_t)o, 256);
  p.off_cnt = o; o += (size_t)B * p.nchunks * 4;
  o = (size_t)round_up((int64_t)o, 256);
  p.off_cut = o; o += (size_t)B * p.nchunks * 4;
  p.bytes = (size_t)round_up((int64_t)o, 256);
  return p;
}

struct FusedPlan {
  bool dense = false;
  int64_t ld = 0;
  TopkPlan tk;
  CandPlan cd;          // decode only; shares the top-k region with tk
  AttnPlan at;
  size_t off_scores = 0, off_topk = 0, off_idx = 0, off_attn = 0, bytes = 0;
};

FusedPlan plan_fused(int T, int max_len, int k, int H, int D_v, bool decode) {
  FusedPlan p;
  p.dense = max_len <= k;
  p.ld = p.dense ? 0 : round_up(max_len, 4);
  if (!p.dense) p.tk = plan_topk(T, max_len, k);
  if (!p.dense && decode) p.cd = plan_cand(T, max_len, k);
  p.at = plan_attn(T, k, H, D_v);
  size_t o = 0;
  p.off_scores = o; o += (size_t)T * p.ld * 4;
  o = (size_t)round_up((int64_t)o, 256);
  p.off_topk = o; o += p.tk.bytes > p.cd.bytes ? p.tk.bytes : p.cd.bytes;
  p.off_idx = o; o += (size_t)round_up((int64_t)T * k * 4, 256);
  p.off_attn = o; o += p.at.bytes;
  p.bytes = o;
  return p;
}

// Workspace of dsa_prefill_streaming: the compacted sampled keys, the sampled
// score matrix [T, ceil(max_len / kStreamStride)], per-row thresholds and list headers,
// the candidate lists [T, cap] and their segment records; no [T, max_len]
// score matrix.
struct StreamPlan {
  bool dense = false;
  int umax = 0, cap = 0, rank = 0;
  int64_t ld_samp = 0;
  AttnPlan at;
  size_t off_keys = 0, off_scale = 0, off_samp = 0, off_thr = 0, off_info = 0, off_redo = 0, off_cnt = 0,
         off_lists = 0, off_segs = 0, off_idx = 0, off_attn = 0, bytes = 0;
};

StreamPlan plan_stream(int B, int T, int max_len, int k, int H, int D_v) {
  StreamPlan p;
  p.dense = max_len <= k;
  p.at = plan_attn(T, k, H, D_v);
  size_t o = 0;
  auto take = [&](size_t& off, size_t n) {
    off = o;
    o = (size_t)round_up((int64_t)(o + n), 256);
  };
  if (!p.dense) {
    p.umax = (max_len + kStreamStride - 1) / kStreamStride;
    p.ld_samp = round_up(p.umax, 4);
    p.cap = stream_cap(k);
    p.rank = stream_rank(k);
    take(p.off_keys, (size_t)B * p.umax * 128);
    take(p.off_scale, (size_t)B * p.umax * 4);
    take(p.off_samp, (size_t)T * p.ld_samp * 4);
    take(p.off_thr, (size_t)T * 8);
    take(p.off_info, (size_t)T * 8);
    take(p.off_redo, (size_t)T * 4);
    take(p.off_cnt, 4);
    take(p.off_lists, (size_t)T * p.cap * 8);
    take(p.off_segs, (size_t)T * kStreamMaxSegs * 8);
  }
  take(p.off_idx, (size_t)T * k * 4);
  take(p.off_attn, p.at.bytes);
  p.bytes = o;
  return p;
}

// Workspace of dsa_indexer_warmup: the [T, ld] score matrix (overwritten by
// dI), the per-head dense log-sum-exps and the per-chunk key-gradient partials.
struct WarmPlan {
  int64_t ld = 0;
  int row_chunk = 0, nchunk = 0;
  size_t off_scores = 0, off_lse = 0, off_dk = 0, off_pairs = 0, bytes = 0;
};

WarmPlan plan_warmup(int T, int B, int max_len, int max_q, int H) {
  WarmPlan p;
  p.ld = round_up(max_len, 4);
  // at most 16 chunks of rows per key tile, at least 64 rows each
  p.row_chunk = (int)round_up((max_q + 15) / 16, 4);
  if (p.row_chunk < 64) p.row_chunk = 64;
  p.nchunk = (max_q + p.row_chunk - 1) / p.row_chunk;
  size_t o = 0;
  p.off_scores = o; o += (size_t)T * p.ld * 4;
  o = (size_t)round_up((int64_t)o, 256);
  p.off_lse = o; o += (size_t)T * H * 4;
  o = (size_t)round_up((int64_t)o, 256);
  p.off_dk = o; o += (size_t)p.nchunk * B * max_len * 128 * 4;
  o = (size_t)round_up((int64_t)o, 256);
  p.off_pairs = o; o += (size_t)(B + 1) * 4;
  p.bytes = (size_t)round_up((int64_t)o, 256);
  return p;
}

// ---------------------------------------------------------------- launch sequences

dsa_status run_indexer(const dsa_batch* b, const uint8_t* q8, const float* q_scale, const float* w,
                       const dsa_cache* kidx, const dsa_cache* kscale, int H_I, int d_I, float* scores,
                       int64_t ld, uint32_t* hist, hipStream_t s) {
  IndexerArgs a;
  a.g = make_geo(b);
  a.kidx = make_cache(kidx);
  a.ksc = make_cache(kscale);
  a.q8 = q8;
  a.q_scale = q_scale;
  a.w = w;
  a.scores = scores;
  a.ld = ld;
  a.hist = hist;
  a.H_I = H_I;
  const bool decode = b->q_start == nullptr;
  if (decode) {
    a.chunk = decode_chunk(b->max_len, b->num_seqs);
    a.ntiles = 1;
  } else {
    a.chunk = kIdxPrefillChunk;
    a.ntiles = (b->max_q + kIdxPrefillRows - 1) / kIdxPrefillRows;
  }
  a.nchunks = (b->max_len + a.chunk - 1) / a.chunk;
  CHECK((int64_t)a.nchunks * a.ntiles < (int64_t)1 << 31, DSA_ERR_UNSUPPORTED, "indexer grid too large");
  LAUNCH(launch_indexer(a, d_I, decode, hist != nullptr, s), "indexer launch");
  return DSA_OK;
}

dsa_status run_topk(const dsa_batch* b, const float* scores, int64_t ld, int k, int32_t* idx,
                    const TopkPlan& p, char* ws, bool hist_ready, hipStream_t s) {
  TopkArgs a;
  a.g = make_geo(b);
  a.scores = scores;
  a.ld = ld;
  a.k = k;
  a.idx = idx;
  a.hist = nullptr;
  a.hist2 = nullptr;
  a.meta = nullptr;
  a.slice_cnt = nullptr;
  a.lists = nullptr;
  a.slice = p.slice;
  a.nslices = p.nslices;
  if (!p.split) {
    LAUNCH(launch_topk_row(a, s), "top-k launch");
    return DSA_OK;
  }
  a.hist = reinterpret_cast<uint32_t*>(ws + p.off_hist);
  a.hist2 = reinterpret_cast<uint32_t*>(ws + p.off_hist2);
  a.meta = reinterpret_cast<uint32_t*>(ws + p.off_meta);
  a.slice_cnt = reinterpret_cast<uint32_t*>(ws + p.off_slice);
  a.lists = reinterpret_cast<uint2*>(ws + p.off_lists);
  if (!hist_ready) {
    LAUNCH(launch_zero(a.hist, (int64_t)p.zero_words, s), "workspace clear");
    LAUNCH(launch_topk_hist(a, s), "top-k histogram launch");
  }
  LAUNCH(launch_topk_split(a, s), "top-k launch");
  return DSA_OK;
}

dsa_status run_attn(const dsa_batch* b, const uint16_t* q, const dsa_cache* kv, const dsa_cache* v, int H,
                    int D, int D_v, float scale, const int32_t* idx, int k, uint16_t* out, float* lse,
                    const AttnPlan& p, char* ws, hipStream_t s) {
  AttnArgs a;
  a.g = make_geo(b);
  a.kv = make_cache(kv);
  a.v = make_cache((v && v->data) ? v : nullptr);
  a.q = q;
  a.idx = idx;
  a.k = k;
  a.H = H;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;
  a.nsplit = p.nsplit;
  a.per_split = p.per_split;
  a.part_o = p.nsplit > 1 ? reinterpret_cast<uint16_t*>(ws + p.off_o) : nullptr;
  a.part_lse = p.nsplit > 1 ? reinterpret_cast<float*>(ws + p.off_lse) : nullptr;
  LAUNCH(launch_attn(a, D, D_v, s), "attention launch");
  if (p.nsplit > 1) {
    CombineArgs c;
    c.part_o = a.part_o;
    c.part_lse = a.part_lse;
    c.out = out;
    c.lse = lse;
    c.T = b->num_rows;
    c.H = H;
    c.D_v = D_v;
    c.nsplit = p.nsplit;
    LAUNCH(launch_combine(c, s), "attention combine launch");
  }
  return DSA_OK;
}

dsa_status check_indexer_args(const dsa_batch* b, const uint8_t* q8, const float* w, const dsa_cache* kidx,
                              const dsa_cache* kscale, int H_I, int d_I) {
  CHECK(q8 && w, DSA_ERR_NULL, "q8 or w is NULL");
  CHECK(H_I >= 4 && H_I <= 64 && H_I % 4 == 0, DSA_ERR_UNSUPPORTED, "H_I %d not a multiple of 4 in [4, 64]", H_I);
  CHECK(aligned(w, 16), DSA_ERR_ALIGN, "w not 16-byte aligned");
  CHECK(d_I == 32 || d_I == 128, DSA_ERR_UNSUPPORTED, "d_I %d not in {32, 128}", d_I);
  CHECK(aligned(q8, 16), DSA_ERR_ALIGN, "q8 not 16-byte aligned");
  dsa_status st = check_cache(b, kidx, "index-key", d_I, 16);
  if (st != DSA_OK) return st;
  if (kscale && kscale->data) {
    st = check_cache(b, kscale, "key-scale", 4, 4);
    if (st != DSA_OK) return st;
  }
  return DSA_OK;
}

dsa_status check_attn_args(const dsa_batch* b, const uint16_t* q, const dsa_cache* kv, const dsa_cache* v, int H,
                           int D, int D_v, float scale, int k) {
  CHECK(q, DSA_ERR_NULL, "q is NULL");
  CHECK((D == 576 && D_v == 512) || (D == 64 && D_v == 64), DSA_ERR_UNSUPPORTED,
        "(D, D_v) = (%d, %d) not in {(576, 512), (64, 64)}", D, D_v);
  CHECK(H >= 1 && H <= (D == 64 ? 64 : 128), DSA_ERR_UNSUPPORTED, "H %d outside [1, %d]", H, D == 64 ? 64 : 128);
  CHECK(k >= 1 && k <= 4096, DSA_ERR_UNSUPPORTED, "k %d outside [1, 4096]", k);
  CHECK(isfinite(scale), DSA_ERR_SHAPE, "scale is not finite");
  CHECK(aligned(q, 16), DSA_ERR_ALIGN, "q not 16-byte aligned");
  dsa_status st = check_cache(b, kv, "kv", (int64_t)D * 2, 16);
  if (st != DSA_OK) return st;
  if (v && v->data) {
    CHECK(D == 64, DSA_ERR_UNSUPPORTED, "a separate V cache is supported for D = 64 only");
    st = check_cache(b, v, "v", (int64_t)D_v * 2, 16);
    if (st != DSA_OK) return st;
  }
  return DSA_OK;
}

}  // namespace

// Records `msg` as this thread's last error and returns `s` (for the other
// source files of the library).
dsa_status dsa_record_error(dsa_status s, const char* msg) { return fail(s, "%s", msg); }

// ====================================================================== C ABI

extern "C" const char* dsa_last_error(void) { return g_err.c_str(); }

extern "C" dsa_status dsa_set_attn_splits(int nsplit) {
  CHECK(nsplit >= 0 && nsplit <= 4096, DSA_ERR_SHAPE, "nsplit %d outside [0, 4096]", nsplit);
  g_force_splits = nsplit;
  return ok();
}

extern "C" dsa_status dsa_set_indexer_fp8(int on) {
  CHECK(on == 0 || on == 1, DSA_ERR_SHAPE, "dsa_set_indexer_fp8 takes 0 or 1, got %d", on);
  g_indexer_fp8 = on == 1;
  return ok();
}

extern "C" dsa_status dsa_set_stage_events(void* const* events, int count) {
  if (!events) {
    g_stage_armed = false;
    return ok();
  }
  CHECK(count >= 4, DSA_ERR_SHAPE, "need at least 4 stage events, got %d", count);
  const int n = count < kMaxStageEvents ? count : kMaxStageEvents;
  for (int i = 0; i < n; ++i) CHECK(events[i], DSA_ERR_NULL, "stage event %d is NULL", i);
  for (int i = 0; i < n; ++i) g_stage_events[i] = static_cast<hipEvent_t>(events[i]);
  g_stage_count = n;
  g_stage_armed = true;
  return ok();
}

extern "C" size_t dsa_workspace_size(int entry, const dsa_batch* batch, int k, int H, int D_v) {
  if (check_batch(batch) != DSA_OK) return (size_t)-1;
  if (entry == DSA_WS_WARMUP) {
    if (H < 1 || !batch->q_start) return (size_t)-1;
    return plan_warmup(batch->num_rows, batch->num_seqs, batch->max_len, batch->max_q, H).bytes;
  }
  if (k < 1 || k > 4096) return (size_t)-1;
  switch (entry) {
    case DSA_WS_TOPK:
      return plan_topk(batch->num_rows, batch->max_len, k).bytes;
    case DSA_WS_ATTN:
      if (H < 1 || D_v < 1) return (size_t)-1;
      return plan_attn(batch->num_rows, k, H, D_v).bytes;
    case DSA_WS_DECODE:
      if (H < 1 || D_v < 1 || batch->q_start) return (size_t)-1;
      return plan_fused(batch->num_rows, batch->max_len, k, H, D_v, true).bytes;
    case DSA_WS_PREFILL:
      if (H < 1 || D_v < 1 || !batch->q_start) return (size_t)-1;
      return plan_fused(batch->num_rows, batch->max_len, k, H, D_v, false).bytes;
    case DSA_WS_PREFILL_STREAM:
      if (H < 1 || D_v < 1 || !batch->q_start || k > kStreamMaxK) return (size_t)-1;
      return plan_stream(batch->num_seqs, batch->num_rows, batch->max_len, k, H, D_v).bytes;
    default:
      return (size_t)-1;
  }
}

extern "C" dsa_status dsa_indexer(const dsa_batch* batch, const uint8_t* q8, const float* q_scale,
                                  const float* w, const dsa_cache* kidx, const dsa_cache* kscale, int H_I,
                                  int d_I, float* scores, int64_t ld, void* stream) {
  dsa_status st = check_batch(batch);
  if (st != DSA_OK) return st;
  st = check_indexer_args(batch, q8, w, kidx, kscale, H_I, d_I);
  if (st != DSA_OK) return st;
  CHECK(scores, DSA_ERR_NULL, "scores is NULL");
  CHECK(ld >= batch->max_len, DSA_ERR_SHAPE, "ld %lld < max_len %d", (long long)ld, batch->max_len);
  if (batch->num_rows == 0) return ok();
  st = run_indexer(batch, q8, q_scale, w, kidx, kscale, H_I, d_I, scores, ld, nullptr,
                   static_cast<hipStream_t>(stream));
  return st == DSA_OK ? ok() : st;
}

extern "C" dsa_status dsa_topk(const dsa_batch* batch, const float* scores, int64_t ld, int k, int32_t* idx,
                               void* workspace, size_t ws_bytes, void* stream) {
  dsa_status st = check_batch(batch);
  if (st != DSA_OK) return st;
  CHECK(scores && idx, DSA_ERR_NULL, "scores or idx is NULL");
  CHECK(k >= 1 && k <= 4096, DSA_ERR_UNSUPPORTED, "k %d outside [1, 4096]", k);
  CHECK(ld >= batch->max_len, DSA_ERR_SHAPE, "ld %lld < max_len %d", (long long)ld, batch->max_len);
  CHECK(ld % 4 == 0 && aligned(scores, 16), DSA_ERR_ALIGN, "scores must be 16-byte aligned with ld % 4 == 0");
  const TopkPlan p = plan_topk(batch->num_rows, batch->max_len, k);
  if (p.bytes) {
    CHECK(workspace, DSA_ERR_WORKSPACE, "top-k needs %zu workspace bytes, got NULL", p.bytes);
    CHECK(ws_bytes >= p.bytes, DSA_ERR_WORKSPACE, "top-k needs %zu workspace bytes, got %zu", p.bytes, ws_bytes);
    CHECK(aligned(workspace, 256), DSA_ERR_ALIGN, "workspace not 256-byte aligned");
  }
  if (batch->num_rows == 0) return ok();
  st = run_topk(batch, scores, ld, k, idx, p, static_cast<char*>(workspace), false,
                static_cast<hipStream_t>(stream));
  return st == DSA_OK ? ok() : st;
}

extern "C" dsa_status dsa_sparse_attn(const dsa_batch* batch, const uint16_t* q, const dsa_cache* kv,
                                      const dsa_cache* v, int H, int D, int D_v, float scale, const int32_t* idx,
                                      int k, uint16_t* out, float* lse, void* workspace, size_t ws_bytes,
                                      void* stream) {
  dsa_status st = check_batch(batch);
  if (st != DSA_OK) return st;
  st = check_attn_args(batch, q, kv, v, H, D, D_v, scale, k);
  if (st != DSA_OK) return st;
  CHECK(idx && out, DSA_ERR_NULL, "idx or out is NULL");
  const AttnPlan p = plan_attn(batch->num_rows, k, H, D_v);
  if (p.bytes) {
    CHECK(workspace, DSA_ERR_WORKSPACE, "attention needs %zu workspace bytes, got NULL", p.bytes);
    CHECK(ws_bytes >= p.bytes, DSA_ERR_WORKSPACE, "attention needs %zu workspace bytes, got %zu", p.bytes, ws_bytes);
    CHECK(aligned(workspace, 256), DSA_ERR_ALIGN, "workspace not 256-byte aligned");
  }
  if (batch->num_rows == 0) return ok();
  st = run_attn(batch, q, kv, v, H, D, D_v, scale, idx, k, out, lse, p, static_cast<char*>(workspace),
                static_cast<hipStream_t>(stream));
  return st == DSA_OK ? ok() : st;
}

namespace {

// The fused path over all rows of the batch, enqueued on one stream:
// indexer -> top-k -> attention (+ split combine), or, when no row sees more
// than k tokens, identity selections -> attention.  One query per sequence
// (decode) selects through per-chunk candidates (launch_topk_chunk, then
// launch_topk_cand); other batches use the histogram top-k.
dsa_status run_fused(const dsa_batch* batch, const uint8_t* q8, const float* q_scale, const float* w,
                     const dsa_cache* kidx, const dsa_cache* kscale, int H_I, int d_I, int k, const uint16_t* q,
                     const dsa_cache* kv, const dsa_cache* v, int H, int D, int D_v, float scale, uint16_t* out,
                     float* lse, int32_t* idx_out, const FusedPlan& p, char* ws, hipStream_t s) {
  float* scores = reinterpret_cast<float*>(ws + p.off_scores);
  char* tws = ws + p.off_topk;
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + p.off_idx);
  const bool timed = g_stage_armed;
  g_stage_armed = false;
  auto mark = [&](int i) -> hipError_t { return timed ? hipEventRecord(g_stage_events[i], s) : hipSuccess; };
  const bool decode = batch->q_start == nullptr;
  dsa_status st;
  if (!p.dense && decode && p.cd.ok) {
    // decode: indexer scores -> per-chunk candidates -> each row's top-k
    // among its chunks' candidates
    LAUNCH(mark(0), "stage event");
    st = run_indexer(batch, q8, q_scale, w, kidx, kscale, H_I, d_I, scores, p.ld, nullptr, s);
    if (st != DSA_OK) return st;
    LAUNCH(mark(1), "stage event");
    CandArgs c;
    c.g = make_geo(batch);
    c.scores = scores;
    c.ld = p.ld;
    c.k = k;
    c.nchunks = p.cd.nchunks;
    c.cand = reinterpret_cast<uint2*>(tws + p.cd.off_cand);
    c.cand_cnt = reinterpret_cast<uint32_t*>(tws + p.cd.off_cnt);
    c.cand_cut = reinterpret_cast<uint32_t*>(tws + p.cd.off_cut);
    c.idx = idx;
    LAUNCH(launch_topk_chunk(c, s), "top-k launch");
    LAUNCH(launch_topk_cand(c, s), "top-k launch");
    LAUNCH(mark(2), "stage event");
  } else {
    uint32_t* hist = nullptr;
    if (!p.dense && decode && p.tk.split) {
      hist = reinterpret_cast<uint32_t*>(tws + p.tk.off_hist);
      LAUNCH(launch_zero(hist, (int64_t)p.tk.zero_words, s), "workspace clear");
    }
    LAUNCH(mark(0), "stage event");
    if (!p.dense) {
      st = run_indexer(batch, q8, q_scale, w, kidx, kscale, H_I, d_I, scores, p.ld, hist, s);
      if (st != DSA_OK) return st;
    }
    LAUNCH(mark(1), "stage event");
    st = run_topk(batch, scores, p.dense ? 4 : p.ld, k, idx, p.tk, tws, hist != nullptr, s);
    if (st != DSA_OK) return st;
    LAUNCH(mark(2), "stage event");
  }
  st = run_attn(batch, q, kv, v, H, D, D_v, scale, idx, k, out, lse, p.at, ws + p.off_attn, s);
  if (st != DSA_OK) return st;
  LAUNCH(mark(3), "stage event");
  return DSA_OK;
}

dsa_status check_fused_bytes(const dsa_batch* batch, const uint8_t* q8, const float* w, const dsa_cache* kidx,
                             const dsa_cache* kscale, int H_I, int d_I, int k, const uint16_t* q,
                             const dsa_cache* kv, const dsa_cache* v, int H, int D, int D_v, float scale,
                             uint16_t* out, size_t need, void* workspace, size_t ws_bytes) {
  dsa_status st = check_indexer_args(batch, q8, w, kidx, kscale, H_I, d_I);
  if (st != DSA_OK) return st;
  st = check_attn_args(batch, q, kv, v, H, D, D_v, scale, k);
  if (st != DSA_OK) return st;
  CHECK(out, DSA_ERR_NULL, "out is NULL");
  CHECK(workspace, DSA_ERR_WORKSPACE, "the fused path needs %zu workspace bytes, got NULL", need);
  CHECK(ws_bytes >= need, DSA_ERR_WORKSPACE, "the fused path needs %zu workspace bytes, got %zu", need, ws_bytes);
  CHECK(aligned(workspace, 256), DSA_ERR_ALIGN, "workspace not 256-byte aligned");
  return DSA_OK;
}

// The streaming prefill path (dsa_prefill_streaming), enqueued on one stream:
// sampled keys -> sampled scores -> row thresholds -> filtered indexer ->
// finalize (+ recompute of the rows it lists) -> attention.
dsa_status run_stream(const dsa_batch* batch, const uint8_t* q8, const float* q_scale, const float* w,
                      const dsa_cache* kidx, const dsa_cache* kscale, int H_I, int k, const uint16_t* q,
                      const dsa_cache* kv, const dsa_cache* v, int H, int D, int D_v, float scale, uint16_t* out,
                      float* lse, int32_t* idx_out, const StreamPlan& p, char* ws, hipStream_t s) {
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + p.off_idx);
  const bool timed = g_stage_armed;
  g_stage_armed = false;
  auto mark = [&](int i) -> hipError_t { return timed ? hipEventRecord(g_stage_events[i], s) : hipSuccess; };
  StreamArgs sa;
  sa.g = make_geo(batch);
  sa.kidx = make_cache(kidx);
  sa.ksc = make_cache((kscale && kscale->data) ? kscale : nullptr);
  sa.q8 = q8;
  sa.q_scale = q_scale;
  sa.w = w;
  sa.H_I = H_I;
  sa.k = k;
  sa.cap = p.cap;
  sa.rank = p.rank;
  sa.umax = p.umax;
  sa.samp_keys = ws + p.off_keys;
  sa.samp_scale = reinterpret_cast<float*>(ws + p.off_scale);
  sa.samp = reinterpret_cast<const float*>(ws + p.off_samp);
  sa.ld_samp = p.ld_samp;
  sa.thr = reinterpret_cast<unsigned long long*>(ws + p.off_thr);
  sa.rowinfo = reinterpret_cast<unsigned long long*>(ws + p.off_info);
  sa.lists = reinterpret_cast<uint2*>(ws + p.off_lists);
  sa.segs = reinterpret_cast<const uint2*>(ws + p.off_segs);
  sa.redo = reinterpret_cast<int*>(ws + p.off_redo);
  sa.redo_count = reinterpret_cast<uint32_t*>(ws + p.off_cnt);
  sa.idx = idx;
  sa.fp8 = g_indexer_fp8;
  LAUNCH(mark(0), "stage event");
  if (!p.dense) {
    LAUNCH(launch_stream_gather(sa, s), "sampled-key gather launch");
    // the prefill indexer over the compacted sampled keys (key u = token u << kStreamShift,
    // every kStreamStride-th token)
    IndexerArgs ia;
    ia.g = sa.g;
    ia.g.block_table = nullptr;
    ia.g.block_shift = 0;
    ia.kidx = Cache{sa.samp_keys, 128, p.umax};
    ia.ksc = sa.ksc.data ? Cache{reinterpret_cast<const char*>(sa.samp_scale), 4, p.umax} : Cache{nullptr, 0, 0};
    ia.q8 = q8;
    ia.q_scale = q_scale;
    ia.w = w;
    ia.scores = reinterpret_cast<float*>(ws + p.off_samp);
    ia.ld = p.ld_samp;
    ia.hist = nullptr;
    ia.H_I = H_I;
    ia.chunk = kIdxPrefillChunk;
    ia.ntiles = (batch->max_q + kIdxPrefillRows - 1) / kIdxPrefillRows;
    ia.nchunks = (p.umax + ia.chunk - 1) / ia.chunk;
    ia.kshift = kStreamShift;
    LAUNCH(launch_indexer(ia, 128, false, false, s), "sampled indexer launch");
    LAUNCH(launch_stream_threshold(sa, s), "threshold launch");
    IndexerArgs fa;
    fa.g = sa.g;
    fa.kidx = sa.kidx;
    fa.ksc = sa.ksc;
    fa.q8 = q8;
    fa.q_scale = q_scale;
    fa.w = w;
    fa.scores = nullptr;
    fa.ld = 0;
    fa.hist = nullptr;
    fa.H_I = H_I;
    fa.chunk = kIdxPrefillChunk;
    fa.ntiles = ia.ntiles;
    fa.nchunks = (batch->max_len + fa.chunk - 1) / fa.chunk;
    fa.thr = sa.thr;
    fa.rowinfo = sa.rowinfo;
    fa.lists = reinterpret_cast<uint2*>(ws + p.off_lists);
    fa.segs = reinterpret_cast<uint2*>(ws + p.off_segs);
    fa.cap = p.cap;
    fa.fp8 = g_indexer_fp8;
    CHECK((int64_t)fa.nchunks * fa.ntiles < (int64_t)1 << 31, DSA_ERR_UNSUPPORTED, "indexer grid too large");
    LAUNCH(launch_indexer_stream(fa, s), "filtered indexer launch");
  }
  LAUNCH(mark(1), "stage event");
  if (p.dense) {
    dsa_status st = run_topk(batch, nullptr, 4, k, idx, TopkPlan{}, nullptr, false, s);
    if (st != DSA_OK) return st;
  } else {
    LAUNCH(launch_stream_finalize(sa, s), "streaming finalize launch");
  }
  LAUNCH(mark(2), "stage event");
  dsa_status st = run_attn(batch, q, kv, v, H, D, D_v, scale, idx, k, out, lse, p.at, ws + p.off_attn, s);
  if (st != DSA_OK) return st;
  LAUNCH(mark(3), "stage event");
  return DSA_OK;
}

dsa_status check_fused(const dsa_batch* batch, const uint8_t* q8, const float* w, const dsa_cache* kidx,
                       const dsa_cache* kscale, int H_I, int d_I, int k, const uint16_t* q, const dsa_cache* kv,
                       const dsa_cache* v, int H, int D, int D_v, float scale, uint16_t* out, const FusedPlan& p,
                       void* workspace, size_t ws_bytes) {
  return check_fused_bytes(batch, q8, w, kidx, kscale, H_I, d_I, k, q, kv, v, H, D, D_v, scale, out, p.bytes,
                           workspace, ws_bytes);
}

}  // namespace

extern "C" dsa_status dsa_decode(const dsa_batch* batch, const uint8_t* q8, const float* q_scale, const float* w,
                                 const dsa_cache* kidx, const dsa_cache* kscale, int H_I, int d_I, int k,
                                 const uint16_t* q, const dsa_cache* kv, const dsa_cache* v, int H, int D, int D_v,
                                 float scale, uint16_t* out, float* lse, int32_t* idx_out, void* workspace,
                                 size_t ws_bytes, void* stream) {
  dsa_status st = check_batch(batch);
  if (st != DSA_OK) return st;
  CHECK(batch->q_start == nullptr, DSA_ERR_SHAPE, "dsa_decode takes one query per sequence (q_start must be NULL)");
  const FusedPlan p = plan_fused(batch->num_rows, batch->max_len, k, H, D_v, true);
  st = check_fused(batch, q8, w, kidx, kscale, H_I, d_I, k, q, kv, v, H, D, D_v, scale, out, p, workspace, ws_bytes);
  if (st != DSA_OK) return st;
  if (batch->num_rows == 0) return ok();
  st = run_fused(batch, q8, q_scale, w, kidx, kscale, H_I, d_I, k, q, kv, v, H, D, D_v, scale, out, lse, idx_out, p,
                 static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
  return st == DSA_OK ? ok() : st;
}

extern "C" dsa_status dsa_prefill(const dsa_batch* batch, const uint8_t* q8, const float* q_scale, const float* w,
                                  const dsa_cache* kidx, const dsa_cache* kscale, int H_I, int d_I, int k,
                                  const uint16_t* q, const dsa_cache* kv, const dsa_cache* v, int H, int D, int D_v,
                                  float scale, uint16_t* out, float* lse, int32_t* idx_out, void* workspace,
                                  size_t ws_bytes, void* stream) {
  dsa_status st = check_batch(batch);
  if (st != DSA_OK) return st;
  CHECK(batch->q_start != nullptr, DSA_ERR_SHAPE, "dsa_prefill takes query rows per sequence (q_start must be set)");
  const FusedPlan p = plan_fused(batch->num_rows, batch->max_len, k, H, D_v, false);
  st = check_fused(batch, q8, w, kidx, kscale, H_I, d_I, k, q, kv, v, H, D, D_v, scale, out, p, workspace, ws_bytes);
  if (st != DSA_OK) return st;
  if (batch->num_rows == 0) return ok();
  st = run_fused(batch, q8, q_scale, w, kidx, kscale, H_I, d_I, k, q, kv, v, H, D, D_v, scale, out, lse, idx_out, p,
                 static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
  return st == DSA_OK ? ok() : st;
}

extern "C" dsa_status dsa_prefill_streaming(const dsa_batch* batch, const uint8_t* q8, const float* q_scale,
                                            const float* w, const dsa_cache* kidx, const dsa_cache* kscale, int H_I,
                                            int d_I, int k, const uint16_t* q, const dsa_cache* kv,
                                            const dsa_cache* v, int H, int D, int D_v, float scale, uint16_t* out,
                                            float* lse, int32_t* idx_out, void* workspace, size_t ws_bytes,
                                            void* stream) {
  dsa_status st = check_batch(batch);
  if (st != DSA_OK) return st;
  CHECK(batch->q_start != nullptr, DSA_ERR_SHAPE,
        "dsa_prefill_streaming takes query rows per sequence (q_start must be set)");
  CHECK(d_I == 128, DSA_ERR_UNSUPPORTED, "dsa_prefill_streaming supports d_I = 128 (got %d)", d_I);
  CHECK(k >= 1 && k <= kStreamMaxK, DSA_ERR_UNSUPPORTED, "dsa_prefill_streaming supports k in [1, %d] (got %d)",
        kStreamMaxK, k);
  CHECK(batch->max_len <= kStreamMaxLen, DSA_ERR_UNSUPPORTED, "dsa_prefill_streaming supports max_len <= %d (got %d)",
        kStreamMaxLen, batch->max_len);
  const StreamPlan p = plan_stream(batch->num_seqs, batch->num_rows, batch->max_len, k, H, D_v);
  st = check_fused_bytes(batch, q8, w, kidx, kscale, H_I, d_I, k, q, kv, v, H, D, D_v, scale, out, p.bytes,
                         workspace, ws_bytes);
  if (st != DSA_OK) return st;
  if (batch->num_rows == 0) return ok();
  st = run_stream(batch, q8, q_scale, w, kidx, kscale, H_I, k, q, kv, v, H, D, D_v, scale, out, lse, idx_out, p,
                  static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
  return st == DSA_OK ? ok() : st;
}

extern "C" dsa_status dsa_indexer_warmup(const dsa_batch* batch, const uint16_t* q, const dsa_cache* kv, int H,
                                         int D, float scale, const uint8_t* q8, const float* q_scale,
                                         const float* w, const dsa_cache* kidx, const dsa_cache* kscale, int H_I,
                                         int d_I, float* loss, float* dq, float* dw, float* dk, void* workspace,
                                         size_t ws_bytes, void* stream) {
  dsa_status st = check_batch(batch);
  if (st != DSA_OK) return st;
  CHECK(batch->q_start != nullptr, DSA_ERR_SHAPE, "dsa_indexer_warmup takes query rows per sequence (q_start must be set)");
  CHECK(batch->block_table == nullptr, DSA_ERR_UNSUPPORTED, "dsa_indexer_warmup supports contiguous caches only");
  st = check_indexer_args(batch, q8, w, kidx, kscale, H_I, d_I);
  if (st != DSA_OK) return st;
  CHECK(d_I == 128 && (H_I == 32 || H_I == 64), DSA_ERR_UNSUPPORTED,
        "warm-up objective supports d_I = 128 with H_I in {32, 64} (got d_I %d, H_I %d)", d_I, H_I);
  CHECK(q && loss, DSA_ERR_NULL, "q or loss is NULL");
  CHECK(D == 576, DSA_ERR_UNSUPPORTED, "warm-up objective supports D = 576 (got %d)", D);
  CHECK(H >= 16 && H <= 128 && H % 16 == 0, DSA_ERR_UNSUPPORTED, "H %d not a multiple of 16 in [16, 128]", H);
  CHECK(isfinite(scale), DSA_ERR_SHAPE, "scale is not finite");
  CHECK(aligned(q, 16), DSA_ERR_ALIGN, "q not 16-byte aligned");
  CHECK(aligned(w, 16), DSA_ERR_ALIGN, "w not 16-byte aligned");
  CHECK(!dk || aligned(dk, 16), DSA_ERR_ALIGN, "dk not 16-byte aligned");
  st = check_cache(batch, kv, "kv", (int64_t)D * 2, 16);
  if (st != DSA_OK) return st;
  const WarmPlan p = plan_warmup(batch->num_rows, batch->num_seqs, batch->max_len, batch->max_q, H);
  CHECK(workspace, DSA_ERR_WORKSPACE, "warm-up needs %zu workspace bytes, got NULL", p.bytes);
  CHECK(ws_bytes >= p.bytes, DSA_ERR_WORKSPACE, "warm-up needs %zu workspace bytes, got %zu", p.bytes, ws_bytes);
  CHECK(aligned(workspace, 256), DSA_ERR_ALIGN, "workspace not 256-byte aligned");
  if (batch->num_rows == 0 && !dk) return ok();     // with dk set, the zero gradient is still written
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nmark = g_stage_armed ? g_stage_count : 0;
  g_stage_armed = false;
  auto mark = [&](int i) -> hipError_t { return i < nmark ? hipEventRecord(g_stage_events[i], s) : hipSuccess; };
  char* ws = static_cast<char*>(workspace);
  float* scores = reinterpret_cast<float*>(ws + p.off_scores);
  LAUNCH(mark(0), "stage event");
  if (batch->num_rows > 0) {
    st = run_indexer(batch, q8, q_scale, w, kidx, kscale, H_I, d_I, scores, p.ld, nullptr, s);
    if (st != DSA_OK) return st;
  }
  LAUNCH(mark(1), "stage event");
  WarmArgs a;
  a.g = make_geo(batch);
  a.kv = make_cache(kv);
  a.q = q;
  a.H = H;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.inv_H = 1.0f / (float)H;
  a.lse2 = reinterpret_cast<float*>(ws + p.off_lse);
  a.scores = scores;
  a.ld = p.ld;
  a.loss = loss;
  a.kidx = make_cache(kidx);
  a.ksc = make_cache((kscale && kscale->data) ? kscale : nullptr);
  a.q8 = q8;
  a.q_scale = q_scale;
  a.w = w;
  a.H_I = H_I;
  a.dq = dq;
  a.dw = dw;
  a.dk_part = reinterpret_cast<float*>(ws + p.off_dk);
  a.dk = dk;
  a.max_len = batch->max_len;
  a.row_chunk = p.row_chunk;
  a.nchunk = p.nchunk;
  a.pair_start = reinterpret_cast<int*>(ws + p.off_pairs);
  for (int stage = 0; stage < 4; ++stage) {
    LAUNCH(launch_warmup(a, stage, s), "warm-up launch");
    LAUNCH(mark(2 + stage), "stage event");
  }
  return ok();
}
