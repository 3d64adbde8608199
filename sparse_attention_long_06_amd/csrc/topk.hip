// Per-row top-k selection on gfx950 (ouchyi.pink post on DSA, the DSA
// paragraph: a fixed budget of tokens per query; digitalreport.com.tr article
// "DeepSeek V3.2-exp: daha ucuz uzun bağlamlı AI": fine-grained token
// selection; sider.ai "Sparse attention that isn't sparse thinking", section
// "Matematik, Minimalist Sürüm": selection has to be vectorised and
// cache-aware to pay off).
//
// Order: score descending, then token index ascending; -0.0 ties +0.0.  The
// result is the ascending list of the first min(k, n) tokens in that order,
// padded with -1.
//
// Method: radix select on an order-preserving 32-bit key (11 + 11 + 10 bits).
// Every pass over memory issues kUnr chunks of loads per thread before
// consuming any, so a pass costs about one memory latency, not one per chunk.
// Each pass histograms the keys that share the prefix found so far (LDS
// atomics), and a block scan over the bins finds the bin holding the k-th
// key.  The final pass is an ordered compaction: per 4-element thread chunks,
// one block scan of packed (greater, equal) counts gives every kept token its
// output slot, so indices come out ascending and ties at the threshold go to
// the lowest indices.  A pass stops refining as soon as the whole boundary
// bin is needed.
//
// Two kernels:
//   row mode   one workgroup per row; after the first pass the candidates
//              (keys at or above the boundary bin) are compacted into LDS and
//              the remaining passes run there.
//   split mode for a few long rows (decode): S workgroups per row each
//              compact their slice's candidates into global memory, using the
//              row histogram that the indexer (or topk_hist_kernel) built;
//              a second launch, one workgroup per row, concatenates the lists
//              and finishes the selection (the launch boundary orders the
//              memory, with no fences or tickets inside a kernel).
#include "dsa_common.h"
#include "dsa_kernels.h"
#include "select_blocks.h"

namespace dsa {

// ---------------------------------------------------------------- row mode

constexpr int kRowNT = 512;
constexpr int kRowCap = 8192;
constexpr int kRowPer = kRowCap / kRowNT;          // register-held candidates per thread
constexpr int kRowUnr = 4;                         // load batches of the passes over a row's scores
static_assert(kRowPer <= 32 && kUnr * kRowNT / 64 >= 4 * kRowNT / 64, "candidate mask; range words after the scan words");
static_assert(kRowCap >= kBins1, "the key array holds the second histogram");

__global__ void __launch_bounds__(kRowNT) topk_row_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kBins1];
  __shared__ uint32_t tmp[kUnr * kRowNT / 64];
  __shared__ BinSel res;
  __shared__ uint32_t lkey[kRowCap];
  __shared__ int lidx[kRowCap];

  const int t = blockIdx.x;
  int b, pos;
  row_seq_pos(a.g, t, b, pos);
  const int n = pos + 1;
  int32_t* out = a.idx + (int64_t)t * a.k;
  const uint32_t k = (uint32_t)a.k;
  if (n <= a.k) {
    write_identity(out, n, a.k, threadIdx.x, kRowNT);
    return;
  }
  const RowSrc row{a.scores + (int64_t)t * a.ld, n, 0};
  auto to_out = [&](uint32_t slot, uint32_t, int id) { out[slot] = id; };

  hist_pass<kRowNT, kRowUnr>(row, hist, 0u, 0, 32 - kBins1Bits, kBins1Bits);
  const BinSel s1 = select_bin<kRowNT>(hist, kBins1, k, tmp, &res);
  const uint32_t need = k - s1.above;
  if (s1.cnt == need) {
    compact<kRowNT, kRowUnr>(row, s1.bin, kBins1Bits, need, k, tmp, to_out);
    return;
  }
  const uint32_t m = s1.above + s1.cnt;
  if (m <= (uint32_t)kRowCap) {
    // the m keys at or above the boundary bin, in token order, into LDS; then
    // into registers (kRowPer consecutive ones per thread) as offsets from
    // their smallest, for the register radix passes and one ordered
    // compaction.  The first pass's histogram (cleared here) and the key
    // array (free once the keys are in registers) are the two histograms.
    compact<kRowNT, kRowUnr>(row, s1.bin, kBins1Bits, s1.cnt, m, tmp,
                    [&](uint32_t slot, uint32_t key, int id) { lkey[slot] = key; lidx[slot] = id; });
    for (int i = threadIdx.x; i < kBins1; i += kRowNT) hist[i] = 0u;
    lds_barrier();
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int i0 = threadIdx.x * kRowPer;
    const int nv = max(0, min(kRowPer, (int)m - i0));
    uint32_t key[kRowPer];
    int id[kRowPer];
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    // every slot read (i0 + kRowPer <= kRowCap), so the reads issue together
    // instead of one guarded read after another; slots past m are masked
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) {
      key[j] = lkey[i0 + j];
      id[j] = lidx[i0 + j];
    }
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) {
      key[j] = j < nv ? key[j] : 0u;
      id[j] = j < nv ? id[j] : -1;
      if (j < nv) {
        lo = min(lo, key[j]);
        hi = max(hi, key[j]);
      }
    }
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    // (tmp[2NW..4NW): the compaction scan below writes tmp[0..NW) with no
    // barrier in between when no radix pass runs)
    if (lane == 0) {
      tmp[2 * kRowNT / 64 + wid] = lo;
      tmp[3 * kRowNT / 64 + wid] = hi;
    }
    lds_barrier();                                 // keys in registers (LDS keys free), ranges in
    lo = 0xFFFFFFFFu;
    hi = 0u;
#pragma unroll
    for (int w = 0; w < kRowNT / 64; ++w) {
      lo = min(lo, tmp[2 * kRowNT / 64 + w]);
      hi = max(hi, tmp[3 * kRowNT / 64 + w]);
    }
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) key[j] -= lo;
    uint32_t P = 0, need2 = k, cb = m;
    int pbits = hi > lo ? __clz(hi - lo) : 32;
    const uint32_t vm = nv >= 32 ? 0xFFFFFFFFu : (1u << nv) - 1u;
    reg_radix<kRowNT, kRowPer>(key, vm, hist, lkey, &res, P, pbits, need2, cb);
    // ordered compaction: every key above prefix P, and the first need2 at it
    uint32_t gm = 0u, em = 0u;
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) {
      const uint32_t pre = key_prefix(key[j], pbits);
      gm |= (j < nv && pre > P ? 1u : 0u) << j;
      em |= (j < nv && pre == P ? 1u : 0u) << j;
    }
    uint32_t tot2;
    const uint32_t ex = block_exclusive_scan<kRowNT>((uint32_t)__popc(gm) | ((uint32_t)__popc(em) << 16), tmp, tot2);
    uint32_t gr = ex & 0xFFFFu, er = ex >> 16;
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) {
      if ((gm >> j) & 1u) {
        out[gr + min(er, need2)] = id[j];
        ++gr;
      } else if ((em >> j) & 1u) {
        if (er < need2) out[gr + er] = id[j];
        ++er;
      }
    }
  } else {
    refine_and_emit<kRowNT, kRowUnr>(row, s1.bin, kBins1Bits, need, s1.cnt, hist, tmp, &res, k, to_out);
  }
}

// ---------------------------------------------------------------- split mode

constexpr int kSplitNT = 256;
constexpr int kFinalNT = 512;
constexpr int kSplitCap = 8192;

__global__ void __launch_bounds__(kSplitNT) topk_hist_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kBins1];
  const int sl = blockIdx.x, t = blockIdx.y;
  int b, pos;
  row_seq_pos(a.g, t, b, pos);
  const int n = pos + 1;
  if (n <= a.k) return;
  const int beg = sl * a.slice, end = min(n, beg + a.slice);
  if (beg >= end) return;
  const RowSrc src{a.scores + (int64_t)t * a.ld + beg, end - beg, beg};
  hist_pass<kSplitNT>(src, hist, 0u, 0, 32 - kBins1Bits, kBins1Bits);
  uint32_t* gh = a.hist + (int64_t)t * kBins1;
  for (int i = threadIdx.x; i < kBins1; i += kSplitNT) {
    const uint32_t c = hist[i];
    if (c) atomicAdd(gh + i, c);
  }
}

// Phase 1 of split mode: each slice compacts its candidates (keys in the
// first-pass boundary bin or above, read off the complete row histogram) into
// its own list region, in index order, and records how many it wrote.
__global__ void __launch_bounds__(kSplitNT) topk_slice_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kBins1];
  __shared__ uint32_t tmp[kUnr * kSplitNT / 64];
  __shared__ BinSel res;

  const int sl = blockIdx.x, t = blockIdx.y;
  int b, pos;
  row_seq_pos(a.g, t, b, pos);
  const int n = pos + 1;
  const uint32_t k = (uint32_t)a.k;
  if (n <= a.k) {
    if (sl == 0) write_identity(a.idx + (int64_t)t * a.k, n, a.k, threadIdx.x, kSplitNT);
    return;
  }
  // The slice's first NT*4*kUnr scores are requested before the row
  // histogram, so the two memory latencies overlap instead of adding up.
  const int beg = sl * a.slice, end = min(n, beg + a.slice);
  const RowSrc src{a.scores + (int64_t)t * a.ld + beg, max(end - beg, 0), beg};
  constexpr int kFirst = kSplitNT * 4 * kUnr;
  uint32_t key[kUnr][4];
  int id[kUnr][4];
  bool ok[kUnr][4];
  const bool full = src.size() >= kFirst;     // uniform
  float4 raw[kUnr];
  if (full) {
#pragma unroll
    for (int u = 0; u < kUnr; ++u) raw[u] = *reinterpret_cast<const float4*>(src.p + (u * kSplitNT + threadIdx.x) * 4);
  }

  load_hist<kSplitNT>(a.hist + (int64_t)t * kBins1, hist);
  lds_barrier();
  const BinSel s1 = select_bin<kSplitNT>(hist, kBins1, k, tmp, &res);

  if (full) {
#pragma unroll
    for (int u = 0; u < kUnr; ++u) {
      const int i = (u * kSplitNT + threadIdx.x) * 4;
      key[u][0] = score_key(raw[u].x); key[u][1] = score_key(raw[u].y);
      key[u][2] = score_key(raw[u].z); key[u][3] = score_key(raw[u].w);
#pragma unroll
      for (int j = 0; j < 4; ++j) { id[u][j] = beg + i + j; ok[u][j] = true; }
    }
  } else {
    load_batch<kSplitNT>(src, 0, key, id, ok);
  }

  if (sl == 0 && threadIdx.x == 0)
    reinterpret_cast<uint4*>(a.meta)[t] = make_uint4(s1.bin, s1.above, s1.cnt, 0u);

  // Candidates go to this slice's list; those in the boundary bin also count
  // their next 11 key bits into the row's second-level histogram (a few
  // hundred scattered atomics per slice, straight to global memory).
  uint2* mylist = a.lists + ((int64_t)t * a.nslices + sl) * a.slice;
  uint32_t* gh2 = a.hist2 + (int64_t)t * kBins1;
  auto to_list = [&](uint32_t slot, uint32_t kk, int ii) {
    mylist[slot] = make_uint2(kk, (uint32_t)ii);
    if ((kk >> (32 - kBins1Bits)) == s1.bin) atomicAdd(gh2 + ((kk >> (32 - 2 * kBins1Bits)) & (kBins1 - 1)), 1u);
  };
  uint32_t gt = 0, eq = 0;
  compact_batch<kSplitNT>(key, id, ok, s1.bin, 32 - kBins1Bits, 0xFFFFFFFFu, tmp, gt, eq, to_list);
  for (int base = kFirst; base < src.size(); base += kFirst) {     // slices longer than one batch
    load_batch<kSplitNT>(src, base, key, id, ok);
    compact_batch<kSplitNT>(key, id, ok, s1.bin, 32 - kBins1Bits, 0xFFFFFFFFu, tmp, gt, eq, to_list);
  }
  if (threadIdx.x == 0) a.slice_cnt[(int64_t)t * a.nslices + sl] = gt + eq;
}

// Phase 2 of split mode (next launch, so every slice's list is visible): one
// workgroup per row concatenates the slices' lists in slice order (= index
// order), refines the boundary bin and emits the selection.
__global__ void __launch_bounds__(kFinalNT) topk_finalize_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kBins1];
  __shared__ uint32_t tmp[kUnr * kFinalNT / 64];
  __shared__ BinSel res;
  __shared__ uint32_t lkey[kSplitCap];
  __shared__ int lidx[kSplitCap];
  __shared__ uint32_t cnt[kTopkMaxSlices];
  __shared__ uint32_t offs[kTopkMaxSlices + 1];

  const int t = blockIdx.x;
  int b, pos;
  row_seq_pos(a.g, t, b, pos);
  const int n = pos + 1;
  const uint32_t k = (uint32_t)a.k;
  if (n <= a.k) return;                         // phase 1 wrote the identity selection
  load_hist<kFinalNT>(a.hist2 + (int64_t)t * kBins1, hist);
  const uint4 s1 = reinterpret_cast<const uint4*>(a.meta)[t];   // first-pass bin, above, count
  if (threadIdx.x < a.nslices) cnt[threadIdx.x] = a.slice_cnt[(int64_t)t * a.nslices + threadIdx.x];
  lds_barrier();
  if (threadIdx.x == 0) {
    uint32_t o = 0;
    for (int s = 0; s < a.nslices; ++s) {
      offs[s] = o;
      o += cnt[s];
    }
    offs[a.nslices] = o;
  }
  // second level: the 11 key bits after the first-pass bin, histogrammed by
  // the slices over the boundary-bin elements (its barriers publish offs)
  uint32_t need = k - s1.y;
  uint32_t P = s1.x, cnt_p = s1.z;
  int pbits = kBins1Bits;
  const BinSel s2 = select_bin<kFinalNT>(hist, kBins1, need, tmp, &res);
  if (cnt_p != need) {
    P = (P << kBins1Bits) | s2.bin;
    pbits = 2 * kBins1Bits;
    need -= s2.above;
    cnt_p = s2.cnt;
  }
  const uint32_t m = offs[a.nslices];
  int32_t* out = a.idx + (int64_t)t * a.k;
  auto to_out = [&](uint32_t slot, uint32_t, int id) { out[slot] = id; };
  const uint2* rowlists = a.lists + (int64_t)t * a.nslices * a.slice;
  const SegSrc gs{rowlists, offs, a.nslices, a.slice};
  if (m <= (uint32_t)kSplitCap) {
    // Stage the concatenated lists slice by slice: 32 threads per slice copy
    // its (key, index) pairs two at a time (16-byte loads, kUnr in flight
    // per thread) to their place after the earlier slices' candidates.
    constexpr int GROUPS = kFinalNT / 32;
    const int l32 = threadIdx.x & 31;
    for (int sl = threadIdx.x >> 5; sl < a.nslices; sl += GROUPS) {
      const uint4* src = reinterpret_cast<const uint4*>(rowlists + (int64_t)sl * a.slice);
      const uint32_t o = offs[sl], c = cnt[sl];
      const uint32_t npairs = (c + 1) >> 1;         // an odd count reads one unused entry of its region
      for (uint32_t p0 = 0; p0 < npairs; p0 += 32 * kUnr) {
        uint4 v[kUnr];
#pragma unroll
        for (int u = 0; u < kUnr; ++u) {
          const uint32_t pp = p0 + u * 32 + l32;
          v[u] = pp < npairs ? src[pp] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kUnr; ++u) {
          const uint32_t e = 2 * (p0 + u * 32 + l32);
          if (e < c) {
            lkey[o + e] = v[u].x;
            lidx[o + e] = (int)v[u].y;
          }
          if (e + 1 < c) {
            lkey[o + e + 1] = v[u].z;
            lidx[o + e + 1] = (int)v[u].w;
          }
        }
      }
    }
    lds_barrier();
    const LdsSrc ls{lkey, lidx, (int)m};
    refine_and_emit<kFinalNT>(ls, P, pbits, need, cnt_p, hist, tmp, &res, k, to_out);
  } else {
    refine_and_emit<kFinalNT>(gs, P, pbits, need, cnt_p, hist, tmp, &res, k, to_out);
  }
}

// ---------------------------------------------------------------- chunk-candidate mode (fused decode)
//
// Two launches after the indexer has written a row's scores:
//
//   chunk   one workgroup per (row, chunk of kCandChunk tokens) keeps the
//           chunk's keys whose top 22 bits reach the boundary of its C-th
//           largest key (C = cand_per_chunk), in token order, with the
//           largest key it may have dropped (its cut).  Every workgroup of
//           the launch is resident at once, so this costs about one read of
//           the scores plus a few LDS passes.
//   merge   one workgroup per row stages the chunks' lists in LDS and selects
//           the row's top-k among them.  A dropped element can only belong to
//           the top-k (or tie its k-th key) when its chunk's cut reaches the
//           k-th key; then the row is selected again from its full scores, so
//           the result is always exact.
//
// Keys are ranked within [lo, hi] of the staged candidates: the radix passes
// run over key - lo from its highest possibly set bit, which spreads the
// candidates (all from the upper tail of the row) over the histogram bins
// instead of piling them into the few bins their top 11 bits share.

// ---- launch 1: per-chunk candidates

constexpr int kChunkNT = 512;
constexpr int kChunkPer = kCandChunk / kChunkNT;   // consecutive scores per thread
static_assert(kChunkPer % 4 == 0 && kChunkPer <= 32, "float4 loads, 32-bit keep mask");

__global__ void __launch_bounds__(kChunkNT) topk_chunk_kernel(CandArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[2][kBins1];
  __shared__ uint32_t tmp[kChunkNT / 64];
  __shared__ BinSel res;

  const int t = blockIdx.x / a.nchunks;
  const int ch = blockIdx.x - t * a.nchunks;
  int b, pos;
  row_seq_pos(a.g, t, b, pos);
  const int n = pos + 1;
  const int kbeg = ch * kCandChunk;
  if (n <= a.k || kbeg >= n) return;          // uniform over the workgroup
  const int nk = min(kCandChunk, n - kbeg);
  const float* src = a.scores + (int64_t)t * a.ld + kbeg;
  const int64_t slot0 = (int64_t)t * a.nchunks + ch;
  uint2* out = a.cand + slot0 * kCandChunk;

  // consecutive scores per thread (16-byte aligned: ld and kbeg are multiples of 4)
  const int i0 = threadIdx.x * kChunkPer;
  const int nv = max(0, min(kChunkPer, nk - i0));
  uint32_t key[kChunkPer];
  if (nv == kChunkPer) {
    float4 v[kChunkPer / 4];
#pragma unroll
    for (int j = 0; j < kChunkPer / 4; ++j) v[j] = *reinterpret_cast<const float4*>(src + i0 + 4 * j);
#pragma unroll
    for (int j = 0; j < kChunkPer / 4; ++j) {
      key[4 * j] = score_key(v[j].x);
      key[4 * j + 1] = score_key(v[j].y);
      key[4 * j + 2] = score_key(v[j].z);
      key[4 * j + 3] = score_key(v[j].w);
    }
  } else if (nv > 0) {
    // the ragged end: every load in bounds (clamped to the last score) and
    // issued before any is used, instead of one guarded load after another
    float v[kChunkPer];
#pragma unroll
    for (int j = 0; j < kChunkPer; ++j) v[j] = src[i0 + min(j, nv - 1)];
#pragma unroll
    for (int j = 0; j < kChunkPer; ++j) key[j] = j < nv ? score_key(v[j]) : 0u;
  } else {
#pragma unroll
    for (int j = 0; j < kChunkPer; ++j) key[j] = 0u;
  }

  uint32_t vm = 0u;
#pragma unroll
  for (int j = 0; j < kChunkPer; ++j) vm |= (j < nv ? 1u : 0u) << j;

  // keep the keys whose top `pbits` bits are >= P: two 11-bit passes leave
  // the C largest plus the rest of their 22-bit boundary bin.  (Ranking
  // inside a window below the chunk's largest key spreads the LDS atomics
  // better, but the reduction that finds that key cost more than it saved.)
  uint32_t P = 0;
  int pbits = 0;
  const uint32_t C = (uint32_t)cand_per_chunk(a.k, kCandChunk, n, nk);
  if (C < (uint32_t)nk) {
    for (int i = threadIdx.x; i < 2 * kBins1; i += kChunkNT) (&hist[0][0])[i] = 0u;
    lds_barrier();
    uint32_t need = C, cnt = (uint32_t)nk;
    reg_radix<kChunkNT, kChunkPer>(key, vm, hist[0], hist[1], &res, P, pbits, need, cnt, 2 * kBins1Bits);
  }
  uint32_t keep = 0u;
#pragma unroll
  for (int j = 0; j < kChunkPer; ++j) keep |= (((vm >> j) & 1u) && key_prefix(key[j], pbits) >= P ? 1u : 0u) << j;
  uint32_t tot;
  uint32_t o = block_exclusive_scan<kChunkNT>((uint32_t)__popc(keep), tmp, tot);
#pragma unroll
  for (int j = 0; j < kChunkPer; ++j)
    if ((keep >> j) & 1u) out[o++] = make_uint2(key[j], (uint32_t)(kbeg + i0 + j));
  if (threadIdx.x == 0) {
    a.cand_cnt[slot0] = tot;
    // dropped keys have a top-pbits prefix below P: at most (P << (32 - pbits)) - 1
    a.cand_cut[slot0] = (pbits > 0 && P > 0u) ? (P << (32 - pbits)) - 1u : 0u;
  }
}

hipError_t launch_topk_chunk(const CandArgs& a, hipStream_t stream) {
  const int64_t nb = (int64_t)a.g.num_rows * a.nchunks;
  if (nb <= 0 || nb >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_chunk_kernel, dim3((unsigned)nb), dim3(kChunkNT), 0, stream, a);
  return hipGetLastError();
}

// ---- launch 2: each row's top-k among its chunks' candidates

constexpr int kCandNT = 1024;
constexpr int kCandCap = 8192;                     // candidates held on chip; more are read in place
constexpr int kCandPer = kCandCap / kCandNT;       // register-held candidates per thread
constexpr int kCandLoad = 8;                       // staged entries per thread and batch
constexpr int kCandUnr = 2;                        // load batches of the in-place and fallback passes
constexpr int kCandOut = 2048;                     // selections staged in LDS when k fits

// The candidate lists read in place (more candidates than LDS holds).
struct CandSrc {
  const uint2* lists;
  const uint32_t* offs;  // LDS [nch + 1]
  int nch;
  int stride;
  __device__ int size() const { return (int)offs[nch]; }
  __device__ __forceinline__ void load4(int i, uint32_t (&k)[4], int (&d)[4], bool (&ok)[4]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t pos = (uint32_t)(i + j);
      ok[j] = pos < offs[nch];
      k[j] = 0u;
      d[j] = -1;
      if (ok[j]) {
        int lo = 0, hi = nch - 1;  // last chunk with offs[c] <= pos
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (offs[mid] <= pos) lo = mid; else hi = mid - 1;
        }
        const uint2 e = lists[(int64_t)lo * stride + (pos - offs[lo])];
        k[j] = e.x;
        d[j] = (int)e.y;
      }
    }
  }
  __device__ __forceinline__ void load4_full(int i, uint32_t (&k)[4], int (&d)[4], bool (&ok)[4]) const { load4(i, k, d, ok); }
};

__global__ void __launch_bounds__(kCandNT) topk_cand_kernel(CandArgs a) {
  constexpr int NW = kCandNT / 64;
  __shared__ __attribute__((aligned(16))) uint32_t hist[2][kBins1];
  __shared__ uint32_t tmp[kUnr * NW];
  __shared__ uint32_t red[2 * NW];
  __shared__ BinSel res;
  __shared__ __attribute__((aligned(16))) uint32_t lkey[kCandCap];
  __shared__ __attribute__((aligned(16))) int lidx[kCandCap];
  __shared__ uint32_t offs[kCandMaxChunks + 1];
  __shared__ int obuf[kCandOut];

  const int t = blockIdx.x;
  int b, pos;
  row_seq_pos(a.g, t, b, pos);
  const int n = pos + 1;
  int32_t* out = a.idx + (int64_t)t * a.k;
  const uint32_t k = (uint32_t)a.k;
  if (n <= a.k) {
    write_identity(out, n, a.k, threadIdx.x, kCandNT);
    return;
  }
  const int nch = (n + kCandChunk - 1) / kCandChunk;
  const uint32_t* cnt = a.cand_cnt + (int64_t)t * a.nchunks;
  const uint32_t* cut = a.cand_cut + (int64_t)t * a.nchunks;
  const uint2* lists = a.cand + (int64_t)t * a.nchunks * kCandChunk;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;

  // chunk offsets (one block scan of per-thread chunk counts) and the
  // largest cut of the row, in one barrier pair
  uint32_t m, cutmax;
  {
    constexpr int PERC = (kCandMaxChunks + kCandNT - 1) / kCandNT;
    uint32_t c[PERC], sum = 0, cm = 0;
#pragma unroll
    for (int j = 0; j < PERC; ++j) {
      const int ch = threadIdx.x * PERC + j;
      c[j] = ch < nch ? cnt[ch] : 0u;
      cm = max(cm, ch < nch ? cut[ch] : 0u);
      sum += c[j];
    }
    const uint32_t x = wave_inclusive_scan(sum);
    cm = wave_max_u32(cm);
    if (lane == 63) tmp[wid] = x;
    if (lane == 0) red[wid] = cm;
    lds_barrier();
    uint32_t before = 0, tot = 0;
    cutmax = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t s = tmp[w];
      before += (w < wid) ? s : 0u;
      tot += s;
      cutmax = max(cutmax, red[w]);
    }
    uint32_t run = before + x - sum;
#pragma unroll
    for (int j = 0; j < PERC; ++j) {
      const int ch = threadIdx.x * PERC + j;
      if (ch < nch) offs[ch] = run;
      run += c[j];
    }
    if (threadIdx.x == 0) offs[nch] = tot;
    m = tot;
  }
  lds_barrier();                                   // offs is set; tmp / red are free again
  const bool obuf_ok = k <= (uint32_t)kCandOut;
  uint32_t mn = 0xFFFFFFFFu;                       // smallest key emitted (the k-th key)
  uint32_t sub = 0u;                               // keys are ranked as key - sub
  auto emit = [&](uint32_t slot, uint32_t key, int id) {
    if (obuf_ok) obuf[slot] = id; else out[slot] = id;
    mn = min(mn, key);
  };
  if (m <= (uint32_t)kCandCap) {
    // stage the lists in LDS in row order: tpc threads (a power of two) per
    // chunk, kCandLoad entries per thread and batch, every load of a batch
    // issued before any is stored, so one batch costs one memory latency
    int tpc = kCandNT;
    while (tpc > 1 && tpc * nch > kCandNT) tpc >>= 1;
    const int l = threadIdx.x & (tpc - 1);
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int ch = threadIdx.x / tpc; ch < nch; ch += kCandNT / tpc) {
      const uint32_t o = offs[ch], c = offs[ch + 1] - o;
      const uint2* src = lists + (int64_t)ch * kCandChunk;
      for (uint32_t base = 0; base < c; base += (uint32_t)(kCandLoad * tpc)) {
        uint2 e[kCandLoad];
#pragma unroll
        for (int j = 0; j < kCandLoad; ++j) {
          const uint32_t p = base + (uint32_t)(l + j * tpc);
          e[j] = p < c ? src[p] : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int j = 0; j < kCandLoad; ++j) {
          const uint32_t p = base + (uint32_t)(l + j * tpc);
          if (p < c) {
            lkey[o + p] = e[j].x;
            lidx[o + p] = (int)e[j].y;
            lo = min(lo, e[j].x);
            hi = max(hi, e[j].x);
          }
        }
      }
    }
    for (int i = threadIdx.x; i < 2 * kBins1; i += kCandNT) (&hist[0][0])[i] = 0u;
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    // (tmp[NW..2NW): the compaction scan below writes tmp[0..NW) with no
    // barrier in between when no radix pass runs)
    if (lane == 0) {
      tmp[NW + wid] = lo;
      red[wid] = hi;
    }
    lds_barrier();                                 // lists staged, histograms clear, ranges in
    lo = 0xFFFFFFFFu;
    hi = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      lo = min(lo, tmp[NW + w]);
      hi = max(hi, red[w]);
    }
    sub = lo;
    // thread-owned consecutive candidates, as key - lo: the passes start at
    // the highest bit that key - lo can have set
    const int i0 = threadIdx.x * kCandPer;
    const int nv = max(0, min(kCandPer, (int)m - i0));
    uint32_t key[kCandPer];
    int id[kCandPer];
    if (nv == kCandPer) {
#pragma unroll
      for (int q = 0; q < kCandPer / 4; ++q) {
        const uint4 kv = *reinterpret_cast<const uint4*>(lkey + i0 + 4 * q);
        const int4 iv = *reinterpret_cast<const int4*>(lidx + i0 + 4 * q);
        key[4 * q] = kv.x - sub; key[4 * q + 1] = kv.y - sub; key[4 * q + 2] = kv.z - sub; key[4 * q + 3] = kv.w - sub;
        id[4 * q] = iv.x; id[4 * q + 1] = iv.y; id[4 * q + 2] = iv.z; id[4 * q + 3] = iv.w;
      }
    } else {
      // every slot read (i0 + kCandPer <= kCandCap), slots past m masked
#pragma unroll
      for (int j = 0; j < kCandPer; ++j) {
        key[j] = lkey[i0 + j];
        id[j] = lidx[i0 + j];
      }
#pragma unroll
      for (int j = 0; j < kCandPer; ++j) {
        key[j] = j < nv ? key[j] - sub : 0u;
        id[j] = j < nv ? id[j] : -1;
      }
    }
    uint32_t P = 0, need = k, cb = m;
    int pbits = hi > lo ? __clz(hi - lo) : 32;
    const uint32_t vm = nv >= 32 ? 0xFFFFFFFFu : (1u << nv) - 1u;
    reg_radix<kCandNT, kCandPer>(key, vm, hist[0], hist[1], &res, P, pbits, need, cb);
    // ordered compaction: every key above prefix P, and the first `need` at it
    uint32_t gm = 0u, em = 0u;
#pragma unroll
    for (int j = 0; j < kCandPer; ++j) {
      const uint32_t pre = key_prefix(key[j], pbits);
      gm |= (j < nv && pre > P ? 1u : 0u) << j;
      em |= (j < nv && pre == P ? 1u : 0u) << j;
    }
    uint32_t tot2;
    const uint32_t ex = block_exclusive_scan<kCandNT>((uint32_t)__popc(gm) | ((uint32_t)__popc(em) << 16), tmp, tot2);
    uint32_t gr = ex & 0xFFFFu, er = ex >> 16;
#pragma unroll
    for (int j = 0; j < kCandPer; ++j) {
      if ((gm >> j) & 1u) {
        emit(gr + min(er, need), key[j], id[j]);
        ++gr;
      } else if ((em >> j) & 1u) {
        if (er < need) emit(gr + er, key[j], id[j]);
        ++er;
      }
    }
  } else {
    const CandSrc src{lists, offs, nch, kCandChunk};
    refine_and_emit<kCandNT, kCandUnr>(src, 0u, 0, k, m, hist[0], tmp, &res, k, emit);
  }
  mn = wave_min_u32(mn);
  if (lane == 0) red[wid] = mn;
  lds_barrier();                                   // obuf complete, minima in
  uint32_t kth = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < NW; ++w) kth = min(kth, red[w]);
  kth += sub;
  // a chunk whose cut reaches the k-th key may hide elements of the top-k
  // (or ties of it): then the row is selected again from its scores
  if (cutmax == 0u || cutmax < kth) {
    if (obuf_ok)
      for (int i = threadIdx.x; i < a.k; i += kCandNT) out[i] = obuf[i];
  } else {
    const RowSrc row{a.scores + (int64_t)t * a.ld, n, 0};
    hist_pass<kCandNT, kCandUnr>(row, hist[0], 0u, 0, 32 - kBins1Bits, kBins1Bits);
    const BinSel s1 = select_bin<kCandNT>(hist[0], kBins1, k, tmp, &res);
    refine_and_emit<kCandNT, kCandUnr>(row, s1.bin, kBins1Bits, k - s1.above, s1.cnt, hist[0], tmp, &res, k,
                                       [&](uint32_t slot, uint32_t, int id) { out[slot] = id; });
  }
}

hipError_t launch_topk_cand(const CandArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(topk_cand_kernel, dim3(a.g.num_rows), dim3(kCandNT), 0, stream, a);
  return hipGetLastError();
}

// Clears n words; 16-byte stores for the whole quads when p is 16-byte aligned.
__global__ void zero_u32_kernel(uint32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t done = 0;
  if ((reinterpret_cast<uintptr_t>(p) & 15) == 0) {
    uint4* q = reinterpret_cast<uint4*>(p);
    const int64_t nq = n >> 2;
    for (int64_t i = i0; i < nq; i += stride) q[i] = make_uint4(0u, 0u, 0u, 0u);
    done = nq << 2;
  }
  for (int64_t i = done + i0; i < n; i += stride) p[i] = 0u;
}

hipError_t launch_zero(uint32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t want = (n / 4 + 255) / 256 + 1;
  const int64_t blocks = want < 256 ? want : 256;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_topk_hist(const TopkArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(topk_hist_kernel, dim3(a.nslices, a.g.num_rows), dim3(kSplitNT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_topk_split(const TopkArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(topk_slice_kernel, dim3(a.nslices, a.g.num_rows), dim3(kSplitNT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_finalize_kernel, dim3(a.g.num_rows), dim3(kFinalNT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_topk_row(const TopkArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(topk_row_kernel, dim3(a.g.num_rows), dim3(kRowNT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
