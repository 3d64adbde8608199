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

namespace dsa {

struct BinSel {
  uint32_t bin, above, cnt;
};

// ---- element sources: size() and load4(i, ...) for i a multiple of 4

// load4_full(i, ...) may assume i + 3 < size(): callers use it for chunks
// that lie wholly inside the source, where it compiles to one branch-free
// vector load, so a batch of them is issued before the first result is
// awaited.  load4 handles the ragged end.
struct RowSrc {  // fp32 scores in global memory; token index = base + i
  const float* p;  // 16-byte aligned (score rows are, and slices start at multiples of 4)
  int n;
  int base;
  __device__ int size() const { return n; }
  __device__ __forceinline__ void load4_full(int i, uint32_t (&key)[4], int (&id)[4], bool (&ok)[4]) const {
    const float4 v = *reinterpret_cast<const float4*>(p + i);
    key[0] = score_key(v.x); key[1] = score_key(v.y);
    key[2] = score_key(v.z); key[3] = score_key(v.w);
#pragma unroll
    for (int j = 0; j < 4; ++j) { id[j] = base + i + j; ok[j] = true; }
  }
  __device__ __forceinline__ void load4(int i, uint32_t (&key)[4], int (&id)[4], bool (&ok)[4]) const {
    if (i + 3 < n) {
      load4_full(i, key, id, ok);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ok[j] = i + j < n;
        key[j] = ok[j] ? score_key(p[i + j]) : 0u;
        id[j] = base + i + j;
      }
    }
  }
};

struct LdsSrc {  // (key, index) pairs in LDS
  const uint32_t* key;
  const int* id;
  int n;
  __device__ int size() const { return n; }
  __device__ __forceinline__ void load4(int i, uint32_t (&k)[4], int (&d)[4], bool (&ok)[4]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ok[j] = i + j < n;
      k[j] = ok[j] ? key[i + j] : 0u;
      d[j] = ok[j] ? id[i + j] : -1;
    }
  }
  __device__ __forceinline__ void load4_full(int i, uint32_t (&k)[4], int (&d)[4], bool (&ok)[4]) const { load4(i, k, d, ok); }
};

struct SegSrc {  // per-slice (key, index) lists in global memory, concatenated in slice order
  const uint2* lists;   // slice s starts at lists + s * slice
  const uint32_t* offs; // LDS [nslices + 1] prefix of the slice counts
  int nslices;
  int slice;
  __device__ int size() const { return (int)offs[nslices]; }
  __device__ __forceinline__ void load4(int i, uint32_t (&k)[4], int (&d)[4], bool (&ok)[4]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t pos = (uint32_t)(i + j);
      ok[j] = pos < offs[nslices];
      k[j] = 0u;
      d[j] = -1;
      if (ok[j]) {
        int lo = 0, hi = nslices - 1;  // last slice with offs[s] <= pos
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (offs[mid] <= pos) lo = mid; else hi = mid - 1;
        }
        const uint2 e = lists[(int64_t)lo * slice + (pos - offs[lo])];
        k[j] = e.x;
        d[j] = (int)e.y;
      }
    }
  }
  __device__ __forceinline__ void load4_full(int i, uint32_t (&k)[4], int (&d)[4], bool (&ok)[4]) const { load4(i, k, d, ok); }
};

// ---- block-level building blocks (every thread of the block calls them)

// Chunks of NT*4 elements whose loads are issued together before any of
// them is consumed: global sources are latency-bound otherwise.
constexpr int kUnr = 8;

// kUnr chunks of 4 elements per thread starting at `base`; whole chunks go
// through load4_full (issued back to back), a ragged batch through load4.
template <int NT, class Src>
__device__ __forceinline__ void load_batch(const Src& src, int base, uint32_t (&key)[kUnr][4], int (&id)[kUnr][4],
                                           bool (&ok)[kUnr][4]) {
  if (base + NT * 4 * kUnr <= src.size()) {       // uniform
#pragma unroll
    for (int u = 0; u < kUnr; ++u) src.load4_full(base + (u * NT + threadIdx.x) * 4, key[u], id[u], ok[u]);
  } else {
#pragma unroll
    for (int u = 0; u < kUnr; ++u) src.load4(base + (u * NT + threadIdx.x) * 4, key[u], id[u], ok[u]);
  }
}

// Copy a kBins1-bin row histogram from global memory to LDS; every thread
// issues all of its (16-byte) loads before storing any.
template <int NT>
__device__ __forceinline__ void load_hist(const uint32_t* gh, uint32_t* hist) {
  constexpr int PER = kBins1 / (4 * NT);
  static_assert(PER >= 1 && kBins1 % (4 * NT) == 0, "histogram copy shape");
  uint4 v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) v[j] = reinterpret_cast<const uint4*>(gh)[j * NT + threadIdx.x];
#pragma unroll
  for (int j = 0; j < PER; ++j) reinterpret_cast<uint4*>(hist)[j * NT + threadIdx.x] = v[j];
}

// Histogram of bits [shift, shift+bits) of the keys whose top `pbits` bits equal P.
template <int NT, class Src>
__device__ __forceinline__ void hist_pass(const Src& src, uint32_t* hist, uint32_t P, int pbits, int shift, int bits) {
  const int nb = 1 << bits;
  for (int i = threadIdx.x; i < nb; i += NT) hist[i] = 0u;
  lds_barrier();
  const uint32_t mask = (uint32_t)nb - 1u;
  const int n = src.size();
  for (int base = 0; base < n; base += NT * 4 * kUnr) {
    uint32_t key[kUnr][4];
    int id[kUnr][4];
    bool ok[kUnr][4];
    load_batch<NT>(src, base, key, id, ok);
#pragma unroll
    for (int u = 0; u < kUnr; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (ok[u][j] && (pbits == 0 || (key[u][j] >> (32 - pbits)) == P))
          atomicAdd(&hist[(key[u][j] >> shift) & mask], 1u);
  }
  lds_barrier();
}

// The bin (scanning from the top) where the running count reaches `need`,
// how many keys lie in higher bins, and how many are in the bin.
template <int NT>
__device__ __forceinline__ BinSel select_bin(const uint32_t* hist, int nb, uint32_t need, uint32_t* tmp, BinSel* res) {
  const int per = (nb + NT - 1) / NT;
  uint32_t c = 0;
  for (int j = 0; j < per; ++j) {
    const int d = threadIdx.x * per + j;
    if (d < nb) c += hist[nb - 1 - d];
  }
  uint32_t tot;
  const uint32_t pre = block_exclusive_scan<NT>(c, tmp, tot);
  if (pre < need && need <= pre + c) {
    uint32_t run = pre;
    for (int j = 0; j < per; ++j) {
      const int d = threadIdx.x * per + j;
      if (d >= nb) break;
      const uint32_t h = hist[nb - 1 - d];
      if (run + h >= need) {
        res->bin = (uint32_t)(nb - 1 - d);
        res->above = run;
        res->cnt = h;
        break;
      }
      run += h;
    }
  }
  lds_barrier();
  const BinSel r = *res;
  lds_barrier();
  return r;
}

// Ordered compaction: in ascending source order, emit every element whose
// top-`pbits` key prefix is greater than P plus the first `need_eq` whose
// prefix equals P; emit(slot, key, index) gets consecutive slots.
//
// compact_batch does one batch already in registers (kUnr chunks of 4
// elements per thread, chunk u covering elements (u*NT + thread)*4 + j).  The
// kUnr packed (greater, equal) chunk counts are scanned together, one barrier
// pair per batch, and each thread then walks only its set bits, so the cost
// follows the few elements kept.  gt_base / eq_base (uniform) count the
// elements of earlier batches and are advanced past this one.  tmp holds
// kUnr * NT/64 words.
template <int NT, class Emit>
__device__ __forceinline__ void compact_batch(const uint32_t (&key)[kUnr][4], const int (&id)[kUnr][4],
                                              const bool (&ok)[kUnr][4], uint32_t P, int shift, uint32_t need_eq,
                                              uint32_t* tmp, uint32_t& gt_base, uint32_t& eq_base, Emit& emit) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t mg[kUnr], me[kUnr], inc[kUnr], own[kUnr];
#pragma unroll
  for (int u = 0; u < kUnr; ++u) {
    mg[u] = 0u;
    me[u] = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {        // branch-free: selects, no exec-mask juggling
      const uint32_t pre = key[u][j] >> shift;
      const uint32_t v = ok[u][j] ? 1u : 0u;
      mg[u] |= (v & (pre > P ? 1u : 0u)) << j;
      me[u] |= (v & (pre == P ? 1u : 0u)) << j;
    }
    own[u] = (uint32_t)__popc(mg[u]) | ((uint32_t)__popc(me[u]) << 16);
    inc[u] = wave_inclusive_scan(own[u]);
    if (lane == 63) tmp[u * NW + wid] = inc[u];
  }
  lds_barrier();
  uint32_t gt0[kUnr], eq0[kUnr];
  uint32_t rg = gt_base, re = eq_base;
#pragma unroll
  for (int u = 0; u < kUnr; ++u) {
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t c = tmp[u * NW + w];
      before += (w < wid) ? c : 0u;
      tot += c;
    }
    const uint32_t ex = before + inc[u] - own[u];
    gt0[u] = rg + (ex & 0xFFFFu);
    eq0[u] = re + (ex >> 16);
    rg += tot & 0xFFFFu;
    re += tot >> 16;
  }
  lds_barrier();
  gt_base = rg;
  eq_base = re;
#pragma unroll
  for (int u = 0; u < kUnr; ++u) {
    uint32_t mm = mg[u] | me[u], gt = gt0[u], eq = eq0[u];
    while (mm) {
      const int j = __builtin_ctz(mm);
      const uint32_t kk = j == 0 ? key[u][0] : j == 1 ? key[u][1] : j == 2 ? key[u][2] : key[u][3];
      const int ii = j == 0 ? id[u][0] : j == 1 ? id[u][1] : j == 2 ? id[u][2] : id[u][3];
      if ((mg[u] >> j) & 1u) {
        emit(gt + min(eq, need_eq), kk, ii);
        ++gt;
      } else {
        if (eq < need_eq) emit(gt + eq, kk, ii);
        ++eq;
      }
      mm &= mm - 1u;
    }
  }
}

// Whole-source ordered compaction; stops after the batch in which `target`
// elements are out.  Returns the number emitted (uniform).
template <int NT, class Src, class Emit>
__device__ __forceinline__ uint32_t compact(const Src& src, uint32_t P, int pbits, uint32_t need_eq,
                                            uint32_t target, uint32_t* tmp, Emit emit) {
  const int shift = 32 - pbits;
  uint32_t gt_base = 0, eq_base = 0;
  const int n = src.size();
  for (int base = 0; base < n; base += NT * 4 * kUnr) {
    uint32_t key[kUnr][4];
    int id[kUnr][4];
    bool ok[kUnr][4];
    load_batch<NT>(src, base, key, id, ok);
    compact_batch<NT>(key, id, ok, P, shift, need_eq, tmp, gt_base, eq_base, emit);
    if (gt_base + min(eq_base, need_eq) >= target) break;
  }
  return gt_base + min(eq_base, need_eq);
}

// Refine (P, pbits) until the boundary bin is needed whole or the key is
// exhausted, then emit the selection in source order.
template <int NT, class Src, class Emit>
__device__ __forceinline__ void refine_and_emit(const Src& src, uint32_t P, int pbits, uint32_t need, uint32_t cnt,
                                uint32_t* hist, uint32_t* tmp, BinSel* res, uint32_t target, Emit emit) {
  while (cnt != need && pbits < 32) {
    const int bits = (pbits + 11 <= 22) ? 11 : 32 - pbits;
    const int shift = 32 - pbits - bits;
    hist_pass<NT>(src, hist, P, pbits, shift, bits);
    const BinSel s = select_bin<NT>(hist, 1 << bits, need, tmp, res);
    P = (P << bits) | s.bin;
    pbits += bits;
    need -= s.above;
    cnt = s.cnt;
  }
  compact<NT>(src, P, pbits, need, target, tmp, emit);
}

__device__ __forceinline__ void write_identity(int32_t* out, int n, int k, int tid, int nt) {
  for (int i = tid; i < k; i += nt) out[i] = i < n ? i : -1;
}

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

__global__ void zero_u32_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_zero(uint32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  const int64_t blocks = want < 1024 ? want : 1024;
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
