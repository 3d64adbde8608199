// Kernel argument blocks and host launchers of the DSA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa_common.h"

namespace dsa {

// ---------------------------------------------------------------- indexer
struct IndexerArgs {
  Geo g;
  Cache kidx;            // d_I FP8 bytes per token
  Cache ksc;             // fp32 per token; data == nullptr means 1
  const uint8_t* q8;     // [T, H_I, d_I]
  const float* q_scale;  // [T] or nullptr
  const float* w;        // [T, H_I]
  float* scores;         // [T, ld]
  int64_t ld;
  uint32_t* hist;        // [T, kBins1] first-pass top-k histogram (decode layout), or nullptr
  int H_I;
  int chunk;             // keys per workgroup
  int nchunks;           // key chunks per row tile
  int ntiles;            // row tiles per sequence
  // Prefill layout only.  kshift > 0: key u of the cache stands for token
  // u << kshift (a compacted sample of every 2^kshift-th token), so row t sees
  // keys u <= p_t >> kshift.
  int kshift = 0;
  // Streaming selection (filtered epilogue): scores are not stored; the pairs
  // (key, token) whose order (key desc, token asc) reaches the row threshold
  // go to per-row candidate lists in segments (see launch_indexer_stream).
  const unsigned long long* thr = nullptr;   // [T] (key << 32) | ~token of the row threshold
  unsigned long long* rowinfo = nullptr;     // [T] low 32: candidates reserved, high 32: segments
  uint2* lists = nullptr;                    // [T, cap] (key, token)
  uint2* segs = nullptr;                     // [T, kStreamMaxSegs] (chunk << 3 | flush, base << 16 | count)
  int cap = 0;
  // Filtered pass only: decide on FP8 matrix-core scores, keep on exact ones.
  bool fp8 = false;
};

// Rows of one workgroup in the prefill layout (4 waves x kIdxRowsPerWave rows).
constexpr int kIdxRowsPerWave = 2;
constexpr int kIdxPrefillRows = 4 * kIdxRowsPerWave;
constexpr int kIdxPrefillChunk = 1024;
constexpr int kIdxDecodeChunk = 2048;

hipError_t launch_indexer(const IndexerArgs& a, int d_I, bool decode_layout, bool with_hist,
                          hipStream_t stream);

// ---------------------------------------------------------------- streaming prefill selection
// The threshold of a row comes from the scores of every kStreamStride-th
// token; the filtered indexer keeps the pairs at or above it in LDS buffers of
// kStreamLds entries per (wave, row) and flushes them as segments.
constexpr int kStreamShift = 5;
constexpr int kStreamStride = 1 << kStreamShift;
constexpr int kStreamLds = 448;
constexpr int kStreamMaxSegs = 512;
constexpr int kStreamMaxK = 2048;
constexpr int kStreamMaxLen = 262144;

// Rank of the threshold among a row's sampled scores (about k/16, at least
// 64), and the candidate capacity per row (1.75 times the expected count
// kStreamStride * rank; 7168 for k = 2048).
__host__ __device__ constexpr int stream_rank(int k) { return (k + 15) / 16 > 64 ? (k + 15) / 16 : 64; }
__host__ __device__ constexpr int stream_cap(int k) { return 56 * stream_rank(k); }

hipError_t launch_indexer_stream(const IndexerArgs& a, hipStream_t stream);

struct StreamArgs {
  Geo g;
  Cache kidx;            // 128 FP8 bytes per token
  Cache ksc;             // fp32 per token; data == nullptr means 1
  const uint8_t* q8;     // [T, H_I, 128]
  const float* q_scale;  // [T] or nullptr
  const float* w;        // [T, H_I]
  int H_I;
  int k;
  int cap;               // stream_cap(k)
  int rank;              // stream_rank(k)
  int umax;              // sampled keys per sequence: ceil(max_len / kStreamStride)
  char* samp_keys;       // [B, umax, 128] compacted sampled keys
  float* samp_scale;     // [B, umax] their scales (when ksc.data)
  const float* samp;     // [T, ld_samp] sampled scores
  int64_t ld_samp;
  unsigned long long* thr;
  unsigned long long* rowinfo;
  uint2* lists;          // [T, cap]: the filtered pass's pairs (rewritten in place by the exactify launch)
  const uint2* segs;
  int* redo;             // [T] rows the finalize leaves to the fallback
  uint32_t* redo_count;
  int32_t* idx;          // [T, k]
  bool fp8 = false;      // the filtered pass ran on FP8 estimates (pairs carry their error bound)
};

hipError_t launch_stream_gather(const StreamArgs& a, hipStream_t stream);
hipError_t launch_stream_threshold(const StreamArgs& a, hipStream_t stream);
hipError_t launch_stream_finalize(const StreamArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- top-k
struct TopkArgs {
  Geo g;
  const float* scores;
  int64_t ld;
  int k;
  int32_t* idx;          // [T, k]
  uint32_t* hist;        // [T, kBins1]           (split mode) first-pass row histogram
  uint32_t* hist2;       // [T, kBins1]           (split mode) next 11 bits of the boundary bin
  uint32_t* meta;        // [T, 4]                (split mode) first-pass bin, count above it, count in it
  uint32_t* slice_cnt;   // [T, nslices]          (split mode)
  uint2* lists;          // [T, nslices * slice]  (split mode)
  int slice;             // keys per slice        (split mode)
  int nslices;
};

constexpr int kTopkMaxSlices = 64;
constexpr int kTopkSplitMaxRows = 512;

hipError_t launch_zero(uint32_t* p, int64_t n, hipStream_t stream);
// The fused decode's selection through chunk candidates: per chunk of
// kCandChunk tokens of a row, the tokens whose keys reach the boundary of the
// chunk's C-th largest key (C = cand_per_chunk), then the row's top-k among
// them (exact: a row whose candidates may miss part of its top-k is selected
// again from its scores).
constexpr int kCandChunk = 8192;
// Chunks per row above which the fused decode uses the histogram path instead.
constexpr int kCandMaxChunks = 1024;

// Candidates a chunk keeps at least: 1.25 times the chunk's expected share of
// the row's top-k plus 64 (a chunk holding more of the top-k than that is
// more than 12 standard deviations out on exchangeable scores; the selection
// then falls back to the row's full scores), or the whole chunk.
__host__ __device__ inline int cand_per_chunk(int k, int chunk, int n, int nk) {
  const long long c = (5ll * k * chunk + 4ll * n - 1) / (4ll * n) + 64;
  return c < nk ? (int)c : nk;
}

struct CandArgs {
  Geo g;
  const float* scores;   // [T, ld]
  int64_t ld;
  int k;
  int nchunks;           // chunk slots per row: ceil(max_len / kCandChunk)
  uint2* cand;           // [T, nchunks, kCandChunk] (key, token), token order
  uint32_t* cand_cnt;    // [T, nchunks] candidates kept
  uint32_t* cand_cut;    // [T, nchunks] largest key the chunk may have dropped, 0 when none
  int32_t* idx;          // [T, k]
};
// One workgroup per (row, chunk): the chunk's candidates.
hipError_t launch_topk_chunk(const CandArgs& a, hipStream_t stream);
// One workgroup per row: the row's top-k from its chunks' candidates.
hipError_t launch_topk_cand(const CandArgs& a, hipStream_t stream);
hipError_t launch_topk_hist(const TopkArgs& a, hipStream_t stream);
hipError_t launch_topk_split(const TopkArgs& a, hipStream_t stream);
hipError_t launch_topk_row(const TopkArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- attention
struct AttnArgs {
  Geo g;
  Cache kv;              // D bf16 per token
  Cache v;               // D_v bf16 per token; data == nullptr: first D_v dims of kv
  const uint16_t* q;     // [T, H, D]
  const int32_t* idx;    // [T, k]
  int k;
  int H;
  float scale_log2;      // softmax scale * log2(e)
  uint16_t* out;         // [T, H, D_v] bf16 (nsplit == 1)
  float* lse;            // [T, H] or nullptr (nsplit == 1)
  uint16_t* part_o;      // [T, nsplit, H, D_v] bf16, normalised per split (nsplit > 1)
  float* part_lse;       // [T, nsplit, H]      (nsplit > 1)
  int nsplit;
  int per_split;         // selected slots per split, a multiple of kAttnBlock, <= kAttnMaxSplit
};

constexpr int kAttnBlock = 64;      // selected rows staged per step
constexpr int kAttnMaxSplit = 2048; // selected slots one workgroup handles at most

struct CombineArgs {
  const uint16_t* part_o;
  const float* part_lse;
  uint16_t* out;
  float* lse;
  int T, H, D_v, nsplit;
};

// Whether launch_attn runs the 32-head-per-wave kernel for these shapes.
bool attn_uses_wide(int H, int D, int D_v, bool sepv, int per_split);

hipError_t launch_attn(const AttnArgs& a, int D, int D_v, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- indexer warm-up objective
struct WarmArgs {
  Geo g;                 // contiguous caches, query rows per sequence
  Cache kv;              // 576 bf16 per token (K = the whole latent row)
  const uint16_t* q;     // [T, H, 576] bf16
  int H;                 // a multiple of 16 in [16, 128]
  float scale_log2;      // softmax scale * log2(e)
  float inv_H;
  float* lse2;           // [T, H] log2-sum-exp2 of the scaled dense logits
  float* scores;         // [T, ld] indexer scores in, dI out (entries s <= p_t)
  int64_t ld;
  float* loss;           // [T]
  Cache kidx;            // 128 FP8 bytes per token
  Cache ksc;             // fp32 per token or data == nullptr (= 1)
  const uint8_t* q8;     // [T, H_I, 128]
  const float* q_scale;  // [T] or nullptr
  const float* w;        // [T, H_I]
  int H_I;               // 32 or 64
  float* dq;             // [T, H_I, 128] or nullptr
  float* dw;             // [T, H_I] or nullptr
  float* dk_part;        // [nchunk, B, max_len, 128] per-chunk partials
  float* dk;             // [B, max_len, 128] or nullptr
  int max_len;
  int row_chunk;         // query rows per dk chunk
  int nchunk;
  int* pair_start;       // [B + 1] first row pair of each sequence (the dense passes take two rows each)
};

// stage 0: dense log-sum-exp pass; 1: target, KL and dI; 2: dq and dw; 3: dk
hipError_t launch_warmup(const WarmArgs& a, int stage, hipStream_t stream);

}  // namespace dsa
