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

  hist_pass<kRowNT>(row, hist, 0u, 0, 32 - kBins1Bits, kBins1Bits);
  const BinSel s1 = select_bin<kRowNT>(hist, kBins1, k, tmp, &res);
  const uint32_t need = k - s1.above;
  if (s1.cnt == need) {
    compact<kRowNT>(row, s1.bin, kBins1Bits, need, k, tmp, to_out);
    return;
  }
  const uint32_t m = s1.above + s1.cnt;
  if (m <= (uint32_t)kRowCap) {
    compact<kRowNT>(row, s1.bin, kBins1Bits, s1.cnt, m, tmp,
                    [&](uint32_t slot, uint32_t key, int id) { lkey[slot] = key; lidx[slot] = id; });
    lds_barrier();
    const LdsSrc ls{lkey, lidx, (int)m};
    refine_and_emit<kRowNT>(ls, s1.bin, kBins1Bits, need, s1.cnt, hist, tmp, &res, k, to_out);
  } else {
    refine_and_emit<kRowNT>(row, s1.bin, kBins1Bits, need, s1.cnt, hist, tmp, &res, k, to_out);
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
