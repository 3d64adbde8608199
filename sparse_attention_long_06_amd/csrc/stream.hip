// Streaming top-k selection for prefill on gfx950: the lightning indexer's
// scores are never stored as a [rows, tokens] matrix; only the (key, token)
// pairs that can still be among a row's top k leave the indexer (sider.ai
// "Sparse attention that isn't sparse thinking", section "Matematik,
// Minimalist Sürüm": candidate selection has to stay vectorised and
// cache-aware, or its memory traffic eats the gain; ouchyi.pink post, DSA
// paragraph: a fixed budget of k tokens per query).
//
// Order: score descending, then token ascending, i.e. the pair order of
// c(s) = (key(s) << 32) | ~s with key the order-preserving map of the score.
// The selection is the k largest c(s), s <= p, emitted in ascending s.
//
// Launches (stream order is the only synchronisation):
//   gather     every kStreamStride-th token's index key (and scale) of each
//              sequence, compacted, so the prefill indexer can score them;
//   [indexer over the compacted keys: the sampled scores]
//   threshold  per row, thr = the rank-th largest c over its sampled tokens
//              (or the lower edge of its 22-bit key bin when few samples share it);
//              rows with n <= cap take thr = 0 (every token), rows with
//              n <= k need none;
//   [filtered indexer: pairs with c >= thr go to segment lists]
//   exactify   (FP8 filter only) per row, the pairs' FP8 estimates become
//              exact keys where they decide the selection (see below);
//   finalize   per row, the segments sorted by (chunk, flush) give the
//              candidates in token order; the same radix select and ordered
//              compaction as the top-k kernels picks the k largest.
// Exactness: every token with c >= thr is a candidate.  When at least k are,
// the k-th largest c is >= thr, so the top k are all among them.  A row with
// fewer than k candidates, or more than cap (or too many segments), is listed
// by the finalize and recomputed by a fallback launch: scores in batches,
// radix passes and ordered compaction over the recomputed batches, nothing
// stored.
#include "dsa_common.h"
#include "dsa_kernels.h"
#include "idx_math.h"
#include "select_blocks.h"

namespace dsa {

namespace {

__global__ void __launch_bounds__(256) stream_gather_kernel(StreamArgs a) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int u = i >> 3, c = i & 7;                       // sampled token, 16-byte chunk of its key
  const int len = a.g.seq_lens[b];
  if (u >= (len + kStreamStride - 1) >> kStreamShift) return;
  const int s = u << kStreamShift;
  const v4i v = *reinterpret_cast<const v4i*>(token_ptr(a.g, a.kidx, b, s) + 16 * c);
  *reinterpret_cast<v4i*>(a.samp_keys + ((int64_t)b * a.umax + u) * 128 + 16 * c) = v;
  if (c == 0 && a.ksc.data)
    a.samp_scale[(int64_t)b * a.umax + u] = *reinterpret_cast<const float*>(token_ptr(a.g, a.ksc, b, s));
}

constexpr int kThrNT = 256;
constexpr int kThrMaxSamples = kStreamMaxLen / kStreamStride;

// Order keys in LDS; element i is sampled token i.
struct LdsKeySrc {
  const uint32_t* key;
  int n;
  __device__ int size() const { return n; }
  __device__ __forceinline__ void load4(int i, uint32_t (&k)[4], int (&d)[4], bool (&ok)[4]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ok[j] = i + j < n;
      k[j] = ok[j] ? key[i + j] : 0u;
      d[j] = i + j;
    }
  }
  __device__ __forceinline__ void load4_full(int i, uint32_t (&k)[4], int (&d)[4], bool (&ok)[4]) const { load4(i, k, d, ok); }
};

__global__ void __launch_bounds__(kThrNT) stream_threshold_kernel(StreamArgs a) {
  __shared__ uint32_t hist[kBins1];
  __shared__ uint32_t tmp[kUnr * kThrNT / 64];
  __shared__ BinSel res;
  __shared__ unsigned long long tmin;
  __shared__ __attribute__((aligned(16))) uint32_t skeys[kThrMaxSamples];

  const int t = blockIdx.x;
  int b, pos;
  row_seq_pos(a.g, t, b, pos);
  const int n = pos + 1;
  if (threadIdx.x == 0) a.rowinfo[t] = 0ull;
  if (t == 0 && threadIdx.x == 0) *a.redo_count = 0u;
  unsigned long long thr;
  if (n <= a.k) {
    thr = ~0ull;                                         // identity selection: keep nothing
  } else if (n <= a.cap) {
    thr = 0ull;                                          // every token is a candidate
  } else {
    // the rank-th largest pair order among the sampled tokens u <= p >> shift
    // (token u << shift); m > 1.75 * rank because n > cap.  The row's sampled
    // scores are read once (all loads in flight) into LDS as order keys.
    const int m = (pos >> kStreamShift) + 1;
    const float4* row = reinterpret_cast<const float4*>(a.samp + (int64_t)t * a.ld_samp);
    const int n4 = (m + 3) >> 2;
    constexpr int PER = kThrMaxSamples / (4 * kThrNT);
    float4 v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = u * kThrNT + (int)threadIdx.x;
      if (i < n4) v[u] = row[i];
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = u * kThrNT + (int)threadIdx.x;
      if (i < n4)
        reinterpret_cast<uint4*>(skeys)[i] = make_uint4(score_key(v[u].x), score_key(v[u].y), score_key(v[u].z),
                                                        score_key(v[u].w));
    }
    if (threadIdx.x == 0) tmin = ~0ull;
    lds_barrier();
    const LdsKeySrc src{skeys, m};
    // Two radix passes (22 key bits).  When the boundary bin then holds only a
    // few samples, its lower edge is the threshold (every token whose key
    // reaches it is kept: a few more candidates than the exact rank-th pair,
    // never fewer); otherwise (many equal keys) the exact rank-th pair order,
    // token index included, bounds the candidates.
    uint32_t P = 0u, need = (uint32_t)a.rank, cnt = (uint32_t)m;
    int pbits = 0;
    for (int pass = 0; pass < 2 && cnt != need; ++pass) {
      hist_pass<kThrNT>(src, hist, P, pbits, 32 - pbits - kBins1Bits, kBins1Bits);
      const BinSel sb = select_bin<kThrNT>(hist, kBins1, need, tmp, &res);
      P = (P << kBins1Bits) | sb.bin;
      pbits += kBins1Bits;
      need -= sb.above;
      cnt = sb.cnt;
    }
    if (cnt == need || cnt <= 8u) {
      thr = (unsigned long long)(P << (32 - pbits)) << 32;
    } else {
      refine_and_emit<kThrNT>(src, P, pbits, need, cnt, hist, tmp, &res, (uint32_t)a.rank,
                              [&](uint32_t, uint32_t key, int id) {
                                const uint32_t tok = (uint32_t)id << kStreamShift;
                                atomicMin(&tmin, ((unsigned long long)key << 32) | (uint32_t)~tok);
                              });
      lds_barrier();
      thr = tmin;
    }
  }
  if (threadIdx.x == 0) a.thr[t] = thr;
}

constexpr int kFinNT = 512;                              // finalize
constexpr int kFinPer = 7168 / kFinNT;                   // register-held candidates per thread
constexpr int kFinLoad = 8;                              // staged entries per thread and batch
constexpr int kRedoNT = 512;                             // fallback
constexpr int kRedoBatch = kRedoNT * 4 * kUnr;           // tokens per recomputed batch (fallback)
// LDS layout of the batch buffer on the candidate path: keys [cap], tokens
// [cap], then the segment tables
constexpr int kFinSegOff = 8 * 7168;
static_assert(stream_cap(kStreamMaxK) <= 7168, "candidate pairs must fit before the segment tables");
constexpr int kRedoGrid = 256;

// Scores of tokens [base, base + kRedoBatch) of row t (those < n) into sc,
// with the arithmetic of the prefill indexer in the same order, so that they
// equal the scores the indexer produces bit for bit.
template <int HT>
struct RowScorer {
  Wide<128> qa[HT];
  float wq[HT][4];

  __device__ void init(const StreamArgs& a, int t, int nl, int grp) {
    const float qs = a.q_scale ? a.q_scale[t] : 1.0f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 16 + nl;
      Frag<128> raw;
      if (h < a.H_I)
        load_frag<128, false>(raw, reinterpret_cast<const char*>(a.q8) + ((int64_t)t * a.H_I + h) * 128, grp);
      else
        zero_frag<128>(raw);
      qa[ht] = widen<128>(raw);
      const int hw = ht * 16 + grp * 4;
      const float4 w4 = hw < a.H_I ? *reinterpret_cast<const float4*>(a.w + (int64_t)t * a.H_I + hw)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
      wq[ht][0] = w4.x * qs;
      wq[ht][1] = w4.y * qs;
      wq[ht][2] = w4.z * qs;
      wq[ht][3] = w4.w * qs;
    }
  }

  __device__ void stage(const StreamArgs& a, int b, int n, int base, float* sc, int wave, int nl, int grp) const {
    const int nk = min(kRedoBatch, n - base);
    const int ngroups = (nk + 15) / 16;
    for (int gi = wave; gi < ngroups; gi += kRedoNT / 64) {
      const int s = base + gi * 16 + nl;
      const int sl = min(s, n - 1);
      Frag<128> kf;
      load_frag<128, false>(kf, token_ptr(a.g, a.kidx, b, sl), grp);
      const float ks = a.ksc.data ? *reinterpret_cast<const float*>(token_ptr(a.g, a.ksc, b, sl)) : 1.0f;
      const Wide<128> kb = widen<128>(kf);
      float part = 0.0f;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        const v4f acc = mfma_dot<128>(qa[ht], kb);
#pragma unroll
        for (int i = 0; i < 4; ++i) part = fmaf(wq[ht][i], relu(acc[i]), part);
      }
      part = group_sum(part);
      if (grp == 0 && s < n) sc[gi * 16 + nl] = part * ks;
    }
  }

  // Keys of the exact scores of tokens toks[0, nt) (LDS) into keys[] (LDS),
  // with the arithmetic of stage(); wave w takes groups of 16 tokens w, w +
  // nwaves, ..., gathering kGather groups' keys before scoring any of them.
  static constexpr int kGather = 4;
  __device__ void score_list(const StreamArgs& a, int b, const int* toks, int nt, uint32_t* keys, int wave,
                             int nwaves, int nl, int grp) const {
    const int ngroups = (nt + 15) / 16;
    for (int g0 = wave; g0 < ngroups; g0 += nwaves * kGather) {
      Frag<128> kf[kGather];
      float ks[kGather];
#pragma unroll
      for (int u = 0; u < kGather; ++u) {
        const int gi = g0 + u * nwaves;
        if (gi < ngroups) {                          // uniform over the wave
          const int s = toks[min(gi * 16 + nl, nt - 1)];
          load_frag<128, false>(kf[u], token_ptr(a.g, a.kidx, b, s), grp);
          ks[u] = a.ksc.data ? *reinterpret_cast<const float*>(token_ptr(a.g, a.ksc, b, s)) : 1.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < kGather; ++u) {
        const int gi = g0 + u * nwaves;
        if (gi < ngroups) {
          const int i = gi * 16 + nl;
          const Wide<128> kb = widen<128>(kf[u]);
          float part = 0.0f;
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) {
            const v4f acc = mfma_dot<128>(qa[ht], kb);
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) part = fmaf(wq[ht][i4], relu(acc[i4]), part);
          }
          part = group_sum(part);
          if (grp == 0 && i < nt) keys[i] = score_key(part * ks[u]);
        }
      }
    }
  }
};

// ---- exact keys for the FP8 filter's candidates
//
// With the FP8 filter each pair carries its estimate's key and a bound m on
// |estimate - exact| (float bits >> 17, rounded up, above the 18-bit token),
// so the exact score lies in [L, U] = [estimate - m, estimate + m], both
// rounded outward.  With l_k and u_k the k-th largest L and U over the row's
// candidates:
//   L > u_k  the key is in the row's top k whatever the exact scores (fewer
//            than k other candidates can reach it, and every non-candidate
//            is below the threshold);
//   U < l_k  it is not (k candidates are strictly above it);
//   else     (the band) its exact score is computed from the index-key cache.
// The pairs are rewritten in place: key 0xFFFFFFFF for the first kind, 0 for
// the second (neither is the key of a finite score), the exact key for the
// band, the bare token; the finalize then selects exactly what it would have
// from exact keys.  Every pair the exact filter keeps is a candidate (its U
// reaches the threshold's key), so when l_k is above the threshold's key the
// row's top k are all candidates; otherwise, or when the band exceeds
// kExBand, the row's count is cleared and the finalize sends it to the
// fallback.
constexpr int kExNT = 512;
constexpr int kExPer = 7168 / kExNT;     // register-held candidates per thread
constexpr int kExBand = 2048;            // band keys rescored per row at most
static_assert(kExPer * kExNT >= 7168 && kExPer <= 32, "every candidate held in registers");

// The float next below (above) x, or -2^-126 (2^-126) for |x| < 2^-126: a
// rounded-to-nearest result stepped once this way bounds the exact value
// from below (above), also where a result was flushed to zero.
__device__ __forceinline__ float step_down(float x) {
  if (!(fabsf(x) >= 0x1p-126f)) return -0x1p-126f;
  const uint32_t u = __float_as_uint(x);
  return __uint_as_float(x > 0.0f ? u - 1u : u + 1u);
}
__device__ __forceinline__ float step_up(float x) {
  if (!(fabsf(x) >= 0x1p-126f)) return 0x1p-126f;
  const uint32_t u = __float_as_uint(x);
  return __uint_as_float(x > 0.0f ? u + 1u : u - 1u);
}

template <int HT>
__global__ void __launch_bounds__(kExNT) stream_exactify_kernel(StreamArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[2][kBins1];
  __shared__ uint32_t tmp[kExNT / 64];
  __shared__ uint32_t red[kExNT / 64];
  __shared__ BinSel res;
  __shared__ int btok[kExBand];
  __shared__ uint32_t bkey[kExBand];

  const int t = blockIdx.x;
  int b, pos;
  row_seq_pos(a.g, t, b, pos);
  const int n = pos + 1;
  const uint32_t k = (uint32_t)a.k;
  if (n <= a.k) return;
  const unsigned long long info = a.rowinfo[t];
  const uint32_t total = (uint32_t)info, nseg = (uint32_t)(info >> 32);
  if (!(total >= k && total <= (uint32_t)a.cap && nseg <= (uint32_t)kStreamMaxSegs)) return;  // the fallback's
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nl = lane & 15, grp = lane >> 4;
  RowScorer<HT> rs;
  rs.init(a, t, nl, grp);
  uint2* lists = a.lists + (int64_t)t * a.cap;
  const int i0 = threadIdx.x * kExPer;
  const int nv = max(0, min(kExPer, (int)total - i0));
  uint2 e[kExPer];
#pragma unroll
  for (int j = 0; j < kExPer; ++j) e[j] = lists[min(i0 + j, (int)total - 1)];   // all in flight
  uint32_t lk[kExPer], uk[kExPer];
#pragma unroll
  for (int j = 0; j < kExPer; ++j) {
    const float est = key_score(e[j].x);
    const float mg = __uint_as_float((e[j].y >> 18) << 17);
    lk[j] = score_key(step_down(est - mg));
    uk[j] = score_key(step_up(est + mg));
  }
  const uint32_t vm = nv >= 32 ? 0xFFFFFFFFu : (1u << nv) - 1u;
  // the k-th largest of the row's keys `key`: the radix passes end with the
  // k largest being those above prefix P and all those at it, or with P a
  // whole key; either way the k-th is the smallest key at prefix P
  auto kth = [&](const uint32_t (&key)[kExPer]) -> uint32_t {
    for (int i = threadIdx.x; i < 2 * kBins1; i += kExNT) (&hist[0][0])[i] = 0u;
    lds_barrier();
    uint32_t P = 0u, need = k, cnt = total;
    int pbits = 0;
    reg_radix<kExNT, kExPer>(key, vm, hist[0], hist[1], &res, P, pbits, need, cnt);
    uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < kExPer; ++j)
      if (((vm >> j) & 1u) && key_prefix(key[j], pbits) == P) mn = min(mn, key[j]);
    mn = wave_min_u32(mn);
    if (lane == 0) red[wid] = mn;
    lds_barrier();
    uint32_t r = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < kExNT / 64; ++w) r = min(r, red[w]);
    lds_barrier();                                   // red is free again
    return r;
  };
  const uint32_t lkth = kth(lk);
  const uint32_t ukth = kth(uk);
  uint32_t in = 0u, band = 0u;
#pragma unroll
  for (int j = 0; j < kExPer; ++j) {
    const bool v = (vm >> j) & 1u;
    in |= (v && lk[j] > ukth ? 1u : 0u) << j;
    band |= (v && !(lk[j] > ukth) && !(uk[j] < lkth) ? 1u : 0u) << j;
  }
  uint32_t nb;
  uint32_t bo = block_exclusive_scan<kExNT>((uint32_t)__popc(band), tmp, nb);
  const uint32_t thr_key = (uint32_t)(a.thr[t] >> 32);
  if (!(lkth > thr_key && nb <= (uint32_t)kExBand)) {       // uniform
    if (threadIdx.x == 0) a.rowinfo[t] = 0ull;              // the finalize lists the row for the fallback
    return;
  }
  const uint32_t bo0 = bo;
#pragma unroll
  for (int j = 0; j < kExPer; ++j)
    if ((band >> j) & 1u) btok[bo++] = (int)(e[j].y & 0x3FFFFu);
  lds_barrier();                                     // band tokens in
  rs.score_list(a, b, btok, (int)nb, bkey, wid, kExNT / 64, nl, grp);
  lds_barrier();                                     // band keys in
  bo = bo0;
#pragma unroll
  for (int j = 0; j < kExPer; ++j) {
    if (j < nv) {
      const uint32_t key = ((in >> j) & 1u) ? 0xFFFFFFFFu : ((band >> j) & 1u) ? bkey[bo++] : 0u;
      lists[i0 + j] = make_uint2(key, e[j].y & 0x3FFFFu);
    }
  }
}

__global__ void __launch_bounds__(kFinNT) stream_finalize_kernel(StreamArgs a) {
  __shared__ uint32_t hist[kBins1];
  __shared__ uint32_t tmp[kUnr * kFinNT / 64];
  __shared__ BinSel res;
  __shared__ __attribute__((aligned(16))) char big[kFinSegOff + 16 * kStreamMaxSegs];
  static_assert(kStreamMaxSegs <= 2 * kFinNT, "at most two segments per thread in the offset scan");
  static_assert(kUnr * kFinNT / 64 >= 4 * kFinNT / 64, "room for the range words after the scan words");
  static_assert(kFinPer * kFinNT >= 7168 && kFinPer <= 32, "every candidate held in registers");
  static_assert(4 * kStreamMaxSegs * 4 >= kBins1 * 4, "the second histogram fits the segment tables");

  const int t = blockIdx.x;
  int b, pos;
  row_seq_pos(a.g, t, b, pos);
  const int n = pos + 1;
  const uint32_t k = (uint32_t)a.k;
  int32_t* out = a.idx + (int64_t)t * a.k;
  if (n <= a.k) {
    write_identity(out, n, a.k, threadIdx.x, kFinNT);
    return;
  }
  const unsigned long long info = a.rowinfo[t];
  const uint32_t total = (uint32_t)info, nseg = (uint32_t)(info >> 32);
  if (!(total >= k && total <= (uint32_t)a.cap && nseg <= (uint32_t)kStreamMaxSegs)) {
    if (threadIdx.x == 0) a.redo[atomicAdd(a.redo_count, 1u)] = t;   // recomputed by the fallback launch
    return;
  }
  uint32_t* lkey = reinterpret_cast<uint32_t*>(big);
  int* lidx = reinterpret_cast<int*>(big + 4 * a.cap);
  uint32_t* skey = reinterpret_cast<uint32_t*>(big + kFinSegOff);
  uint32_t* sinfo = skey + kStreamMaxSegs;
  uint32_t* soff = sinfo + kStreamMaxSegs;
  int* sorder = reinterpret_cast<int*>(soff + kStreamMaxSegs);
  const uint2* segs = a.segs + (int64_t)t * kStreamMaxSegs;
  for (uint32_t i = threadIdx.x; i < nseg; i += kFinNT) {
    const uint2 e = segs[i];
    skey[i] = e.x;
    sinfo[i] = e.y;
  }
  lds_barrier();
  // segment keys (chunk << 3 | flush) are distinct: rank by counting
  for (uint32_t i = threadIdx.x; i < nseg; i += kFinNT) {
    const uint32_t ki = skey[i];
    uint32_t rnk = 0;
    for (uint32_t j = 0; j < nseg; ++j) rnk += skey[j] < ki ? 1u : 0u;
    sorder[rnk] = (int)i;
  }
  for (int i = threadIdx.x; i < kBins1; i += kFinNT) hist[i] = 0u;
  lds_barrier();
  // offsets in sorted order, two segments per thread
  uint32_t tot;
  const uint32_t j0 = 2 * threadIdx.x;
  const uint32_t c0 = j0 < nseg ? (sinfo[sorder[j0]] & 0xFFFFu) : 0u;
  const uint32_t c1 = j0 + 1 < nseg ? (sinfo[sorder[j0 + 1]] & 0xFFFFu) : 0u;
  const uint32_t ex = block_exclusive_scan<kFinNT>(c0 + c1, tmp, tot);
  if (j0 < nseg) soff[j0] = ex;
  if (j0 + 1 < nseg) soff[j0 + 1] = ex + c0;
  lds_barrier();
  // stage the segments in token order: tpc threads (a power of two) per
  // segment, kFinLoad entries per thread and batch, every load of a batch
  // issued before any is stored, so a batch costs one memory latency; each
  // thread keeps the smallest and largest key it staged
  const uint2* lists = a.lists + (int64_t)t * a.cap;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  {
    int tpc = kFinNT;
    while (tpc > 1 && tpc * (int)nseg > kFinNT) tpc >>= 1;
    const int l = threadIdx.x & (tpc - 1);
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (uint32_t sl = threadIdx.x / tpc; sl < nseg; sl += kFinNT / tpc) {
      const uint32_t inf = sinfo[sorder[sl]];
      const uint32_t base = inf >> 16, cnt = inf & 0xFFFFu, o = soff[sl];
      for (uint32_t e0 = 0; e0 < cnt; e0 += (uint32_t)(kFinLoad * tpc)) {
        uint2 v[kFinLoad];
#pragma unroll
        for (int u = 0; u < kFinLoad; ++u) {
          const uint32_t e = e0 + (uint32_t)(l + u * tpc);
          v[u] = e < cnt ? lists[base + e] : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kFinLoad; ++u) {
          const uint32_t e = e0 + (uint32_t)(l + u * tpc);
          if (e < cnt) {
            lkey[o + e] = v[u].x;
            lidx[o + e] = (int)v[u].y;
            lo = min(lo, v[u].x);
            hi = max(hi, v[u].x);
          }
        }
      }
    }
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    // (tmp[2NW..4NW): the compaction scan below writes tmp[0..NW) with no
    // barrier in between when no radix pass runs)
    if (lane == 0) {
      tmp[2 * kFinNT / 64 + wid] = lo;
      tmp[3 * kFinNT / 64 + wid] = hi;
    }
  }
  lds_barrier();                                   // candidates staged, ranges in; the segment tables are free
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int w = 0; w < kFinNT / 64; ++w) {
    lo = min(lo, tmp[2 * kFinNT / 64 + w]);
    hi = max(hi, tmp[3 * kFinNT / 64 + w]);
  }
  // thread-owned consecutive candidates, ranked as key - lo: the radix
  // passes start at the highest bit that key - lo can have set, which spreads
  // the candidates (all from the row's upper tail) over the bins
  const int i0 = threadIdx.x * kFinPer;
  const int nv = max(0, min(kFinPer, (int)total - i0));
  uint32_t key[kFinPer];
  int id[kFinPer];
  // every slot read (i0 + kFinPer <= 7168: inside the key and index arrays),
  // so the reads issue together; slots past the total are masked
#pragma unroll
  for (int j = 0; j < kFinPer; ++j) {
    key[j] = lkey[i0 + j];
    id[j] = lidx[i0 + j];
  }
#pragma unroll
  for (int j = 0; j < kFinPer; ++j) {
    key[j] = j < nv ? key[j] - lo : 0u;
    id[j] = j < nv ? id[j] : -1;
  }
  uint32_t P = 0, need = k, cb = total;
  int pbits = hi > lo ? __clz(hi - lo) : 32;
  const uint32_t vm = nv >= 32 ? 0xFFFFFFFFu : (1u << nv) - 1u;
  // hist (cleared before the staging) and the segment tables' space alternate
  reg_radix<kFinNT, kFinPer>(key, vm, hist, reinterpret_cast<uint32_t*>(big + kFinSegOff), &res, P, pbits, need, cb);
  // ordered compaction: every candidate above prefix P, and the first `need`
  // at it (the smallest tokens among equal keys)
  uint32_t gm = 0u, em = 0u;
#pragma unroll
  for (int j = 0; j < kFinPer; ++j) {
    const uint32_t pre = key_prefix(key[j], pbits);
    gm |= (j < nv && pre > P ? 1u : 0u) << j;
    em |= (j < nv && pre == P ? 1u : 0u) << j;
  }
  uint32_t tot2;
  const uint32_t ex2 = block_exclusive_scan<kFinNT>((uint32_t)__popc(gm) | ((uint32_t)__popc(em) << 16), tmp, tot2);
  uint32_t gr = ex2 & 0xFFFFu, er = ex2 >> 16;
#pragma unroll
  for (int j = 0; j < kFinPer; ++j) {
    if ((gm >> j) & 1u) {
      out[gr + min(er, need)] = id[j];
      ++gr;
    } else if ((em >> j) & 1u) {
      if (er < need) out[gr + er] = id[j];
      ++er;
    }
  }
}

// Rows the finalize could not select from their candidates: each is redone by
// one workgroup, recomputing its scores batch by batch for every radix pass
// and for the ordered compaction (nothing stored).  The grid is small and
// fixed; workgroup g takes listed rows g, g + grid, ...
template <int HT>
__global__ void __launch_bounds__(kRedoNT) stream_fallback_kernel(StreamArgs a) {
  __shared__ uint32_t hist[kBins1];
  __shared__ uint32_t tmp[kUnr * kRedoNT / 64];
  __shared__ BinSel res;
  __shared__ __attribute__((aligned(16))) float sc[kRedoBatch];

  const uint32_t nredo = *a.redo_count;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nl = lane & 15, grp = lane >> 4;
  const uint32_t k = (uint32_t)a.k;
  for (uint32_t r = blockIdx.x; r < nredo; r += gridDim.x) {
    const int t = a.redo[r];
    int b, pos;
    row_seq_pos(a.g, t, b, pos);
    const int n = pos + 1;
    int32_t* out = a.idx + (int64_t)t * a.k;
    RowScorer<HT> rs;
    rs.init(a, t, nl, grp);
    uint32_t P = 0u, need = k, cnt = (uint32_t)n;
    int pbits = 0;
    while (cnt != need && pbits < 32) {
      const int bits = (pbits + 11 <= 22) ? 11 : 32 - pbits;
      const int shift = 32 - pbits - bits;
      const int nb = 1 << bits;
      const uint32_t mask = (uint32_t)nb - 1u;
      for (int i = threadIdx.x; i < nb; i += kRedoNT) hist[i] = 0u;
      for (int base = 0; base < n; base += kRedoBatch) {
        rs.stage(a, b, n, base, sc, wave, nl, grp);
        lds_barrier();
        const int nk = min(kRedoBatch, n - base);
        for (int i = threadIdx.x; i < nk; i += kRedoNT) {
          const uint32_t key = score_key(sc[i]);
          if (pbits == 0 || (key >> (32 - pbits)) == P) atomicAdd(&hist[(key >> shift) & mask], 1u);
        }
        lds_barrier();
      }
      const BinSel s = select_bin<kRedoNT>(hist, nb, need, tmp, &res);
      P = (P << bits) | s.bin;
      pbits += bits;
      need -= s.above;
      cnt = s.cnt;
    }
    uint32_t gt = 0u, eq = 0u;
    for (int base = 0; base < n; base += kRedoBatch) {
      rs.stage(a, b, n, base, sc, wave, nl, grp);
      lds_barrier();
      uint32_t key[kUnr][4];
      int id[kUnr][4];
      bool ok[kUnr][4];
#pragma unroll
      for (int u = 0; u < kUnr; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = (u * kRedoNT + (int)threadIdx.x) * 4 + j;
          ok[u][j] = base + i < n;
          key[u][j] = ok[u][j] ? score_key(sc[i]) : 0u;
          id[u][j] = base + i;
        }
      // compact_batch's barriers also order these reads before the next stage's writes
      auto to_out = [&](uint32_t slot, uint32_t, int id) { out[slot] = id; };
      compact_batch<kRedoNT>(key, id, ok, P, 32 - pbits, need, tmp, gt, eq, to_out);
      if (gt + min(eq, need) >= k) break;
    }
    lds_barrier();                      // the next row's first stage overwrites sc
  }
}

}  // namespace

hipError_t launch_stream_gather(const StreamArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(((int64_t)a.umax * 8 + 255) / 256), (unsigned)a.g.num_seqs);
  hipLaunchKernelGGL(stream_gather_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_stream_threshold(const StreamArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(stream_threshold_kernel, dim3(a.g.num_rows), dim3(kThrNT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_stream_finalize(const StreamArgs& a, hipStream_t stream) {
  if (a.fp8) {
    switch ((a.H_I + 15) / 16) {
      case 1: hipLaunchKernelGGL(stream_exactify_kernel<1>, dim3(a.g.num_rows), dim3(kExNT), 0, stream, a); break;
      case 2: hipLaunchKernelGGL(stream_exactify_kernel<2>, dim3(a.g.num_rows), dim3(kExNT), 0, stream, a); break;
      case 3: hipLaunchKernelGGL(stream_exactify_kernel<3>, dim3(a.g.num_rows), dim3(kExNT), 0, stream, a); break;
      case 4: hipLaunchKernelGGL(stream_exactify_kernel<4>, dim3(a.g.num_rows), dim3(kExNT), 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    const hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
  hipLaunchKernelGGL(stream_finalize_kernel, dim3(a.g.num_rows), dim3(kFinNT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(a.g.num_rows < kRedoGrid ? a.g.num_rows : kRedoGrid);
  switch ((a.H_I + 15) / 16) {
    case 1: hipLaunchKernelGGL(stream_fallback_kernel<1>, grid, dim3(kRedoNT), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(stream_fallback_kernel<2>, grid, dim3(kRedoNT), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(stream_fallback_kernel<3>, grid, dim3(kRedoNT), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(stream_fallback_kernel<4>, grid, dim3(kRedoNT), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dsa
