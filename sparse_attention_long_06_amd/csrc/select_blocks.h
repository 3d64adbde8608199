// Block-level building blocks of the per-row top-k selection (gfx950, wave64):
// element sources, radix histogram passes, boundary-bin search and ordered
// compaction.  Order: score descending, then token index ascending, on the
// order-preserving 32-bit key of dsa_common.h; radix digits of 11 + 11 + 10
// bits.  Every routine is called by all NT threads of a workgroup.
#pragma once

#include "dsa_common.h"

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
// them is consumed: global sources are latency-bound otherwise.  The
// helpers below take the count as a template argument U (default kUnr);
// their LDS scratch `tmp` holds U * NT/64 words.
constexpr int kUnr = 8;

// U chunks of 4 elements per thread starting at `base`; whole chunks go
// through load4_full (issued back to back), a ragged batch through load4.
template <int NT, int U = kUnr, class Src>
__device__ __forceinline__ void load_batch(const Src& src, int base, uint32_t (&key)[U][4], int (&id)[U][4],
                                           bool (&ok)[U][4]) {
  if (base + NT * 4 * U <= src.size()) {       // uniform
#pragma unroll
    for (int u = 0; u < U; ++u) src.load4_full(base + (u * NT + threadIdx.x) * 4, key[u], id[u], ok[u]);
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) src.load4(base + (u * NT + threadIdx.x) * 4, key[u], id[u], ok[u]);
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
template <int NT, int U = kUnr, class Src>
__device__ __forceinline__ void hist_pass(const Src& src, uint32_t* hist, uint32_t P, int pbits, int shift, int bits) {
  const int nb = 1 << bits;
  for (int i = threadIdx.x; i < nb; i += NT) hist[i] = 0u;
  lds_barrier();
  const uint32_t mask = (uint32_t)nb - 1u;
  const int n = src.size();
  for (int base = 0; base < n; base += NT * 4 * U) {
    uint32_t key[U][4];
    int id[U][4];
    bool ok[U][4];
    load_batch<NT, U>(src, base, key, id, ok);
#pragma unroll
    for (int u = 0; u < U; ++u)
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
// compact_batch does one batch already in registers (U chunks of 4
// elements per thread, chunk u covering elements (u*NT + thread)*4 + j).  The
// U packed (greater, equal) chunk counts are scanned together, one barrier
// pair per batch, and each thread then walks only its set bits, so the cost
// follows the few elements kept.  gt_base / eq_base (uniform) count the
// elements of earlier batches and are advanced past this one.  tmp holds
// U * NT/64 words.
template <int NT, int U = kUnr, class Emit>
__device__ __forceinline__ void compact_batch(const uint32_t (&key)[U][4], const int (&id)[U][4],
                                              const bool (&ok)[U][4], uint32_t P, int shift, uint32_t need_eq,
                                              uint32_t* tmp, uint32_t& gt_base, uint32_t& eq_base, Emit& emit) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t mg[U], me[U], inc[U], own[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    mg[u] = 0u;
    me[u] = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {        // branch-free: selects, no exec-mask juggling
      const uint32_t pre = shift < 32 ? key[u][j] >> shift : 0u;   // shift 32: no prefix yet
      const uint32_t v = ok[u][j] ? 1u : 0u;
      mg[u] |= (v & (pre > P ? 1u : 0u)) << j;
      me[u] |= (v & (pre == P ? 1u : 0u)) << j;
    }
    own[u] = (uint32_t)__popc(mg[u]) | ((uint32_t)__popc(me[u]) << 16);
    inc[u] = wave_inclusive_scan(own[u]);
    if (lane == 63) tmp[u * NW + wid] = inc[u];
  }
  lds_barrier();
  uint32_t gt0[U], eq0[U];
  uint32_t rg = gt_base, re = eq_base;
#pragma unroll
  for (int u = 0; u < U; ++u) {
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
  for (int u = 0; u < U; ++u) {
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
template <int NT, int U = kUnr, class Src, class Emit>
__device__ __forceinline__ uint32_t compact(const Src& src, uint32_t P, int pbits, uint32_t need_eq,
                                            uint32_t target, uint32_t* tmp, Emit emit) {
  const int shift = 32 - pbits;
  uint32_t gt_base = 0, eq_base = 0;
  const int n = src.size();
  for (int base = 0; base < n; base += NT * 4 * U) {
    uint32_t key[U][4];
    int id[U][4];
    bool ok[U][4];
    load_batch<NT, U>(src, base, key, id, ok);
    compact_batch<NT, U>(key, id, ok, P, shift, need_eq, tmp, gt_base, eq_base, emit);
    if (gt_base + min(eq_base, need_eq) >= target) break;
  }
  return gt_base + min(eq_base, need_eq);
}

// Refine (P, pbits) until the boundary bin is needed whole or the key is
// exhausted, then emit the selection in source order.  pbits may start
// anywhere in [0, 32] (0: no prefix yet); each pass takes up to 11 more bits.
template <int NT, int U = kUnr, class Src, class Emit>
__device__ __forceinline__ void refine_and_emit(const Src& src, uint32_t P, int pbits, uint32_t need, uint32_t cnt,
                                uint32_t* hist, uint32_t* tmp, BinSel* res, uint32_t target, Emit emit) {
  while (cnt != need && pbits < 32) {
    const int bits = 32 - pbits < kBins1Bits ? 32 - pbits : kBins1Bits;
    const int shift = 32 - pbits - bits;
    hist_pass<NT, U>(src, hist, P, pbits, shift, bits);
    const BinSel s = select_bin<NT>(hist, 1 << bits, need, tmp, res);
    P = (P << bits) | s.bin;
    pbits += bits;
    need -= s.above;
    cnt = s.cnt;
  }
  compact<NT, U>(src, P, pbits, need, target, tmp, emit);
}

__device__ __forceinline__ void write_identity(int32_t* out, int n, int k, int tid, int nt) {
  for (int i = tid; i < k; i += nt) out[i] = i < n ? i : -1;
}

// Selection over register-held elements.  Elements stay in registers:
// a thread owns PER consecutive elements, so source order is (thread, slot)
// order and an ordered compaction needs one block scan.  The boundary bin of
// a histogram is found by wave 0 alone while the other waves clear the
// histogram of the next pass (two alternate), so a pass costs two barriers.

// Top `pbits` bits of a key (0 when pbits is 0).
__device__ __forceinline__ uint32_t key_prefix(uint32_t key, int pbits) {
  return pbits == 0 ? 0u : key >> (32 - pbits);
}

// Wave-wide min / max with DPP row shifts and row broadcasts (the pattern of
// wave_inclusive_scan; lanes with no source read the identity), then lane 63.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  constexpr int kId = -1;                          // 0xFFFFFFFF
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)x, 0x111, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)x, 0x112, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)x, 0x114, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)x, 0x118, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)x, 0x142, 0xa, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)x, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Wave 0 only: the bin of hist[0, nb) (nb <= kBins1, a power of two),
// scanning from the top, where the running count reaches `need`, the count
// above it and its own count, written to *res.  Two wave scans: lane l sums
// the `per` bins at descending positions per*l .. per*l + per - 1 (bin
// nb - 1 - position); then lanes 0 .. per-1 scan the bins of the lane whose
// range holds the boundary.
__device__ __forceinline__ void wave_select_bin(const uint32_t* hist, int nb, uint32_t need, BinSel* res) {
  static_assert(kBins1 == 64 * 32, "at most 32 bins per lane");
  const int lane = threadIdx.x & 63;
  const int per = nb >= 64 ? nb >> 6 : 1;
  uint32_t c = 0;
  if (per == 32) {
    const uint4* p = reinterpret_cast<const uint4*>(hist + nb - 32 * (lane + 1));
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint4 x = p[q];
      c += x.x + x.y + x.z + x.w;
    }
  } else {
    for (int j = 0; j < per; ++j) {
      const int d = lane * per + j;
      if (d < nb) c += hist[nb - 1 - d];
    }
  }
  const uint32_t incl = wave_inclusive_scan(c);
  const unsigned long long hit = __ballot(incl - c < need && need <= incl);
  if (hit == 0ull) return;                         // need exceeds the histogram's total (callers never ask)
  const int L = __builtin_ctzll(hit);
  const uint32_t run0 = (uint32_t)__shfl((int)(incl - c), L);
  const int d = L * per + lane;
  const uint32_t v = (lane < per && d < nb) ? hist[nb - 1 - d] : 0u;
  const uint32_t incl2 = wave_inclusive_scan(v) + run0;
  if (lane < per && incl2 - v < need && need <= incl2) {
    res->bin = (uint32_t)(nb - 1 - d);
    res->above = incl2 - v;
    res->cnt = v;
  }
}

// Radix passes over register-held keys (PER per thread, bit j of vm set for
// the valid ones) until the boundary prefix is exact or needed whole, or
// pbits reaches max_pbits.  The passes alternate between two histograms,
// h0 and h1 (kBins1 words each): h0 must be clear on entry, h1 is cleared
// during the first pass.  P / pbits / need / cnt carry the state in and out
// (cnt: keys sharing the current prefix; need: how many of them the
// selection takes, <= cnt).
template <int NT, int PER>
__device__ __forceinline__ void reg_radix(const uint32_t (&key)[PER], uint32_t vm, uint32_t* h0, uint32_t* h1,
                                          BinSel* res, uint32_t& P, int& pbits, uint32_t& need, uint32_t& cnt,
                                          int max_pbits = 32) {
  static_assert(PER <= 32, "32-bit validity mask");
  const int wid = threadIdx.x >> 6;
  int cur = 0;
  while (cnt != need && pbits < max_pbits) {       // uniform
    const int bits = 32 - pbits < kBins1Bits ? 32 - pbits : kBins1Bits;
    const int shift = 32 - pbits - bits;
    const uint32_t mask = (1u << bits) - 1u;
    uint32_t* hc = cur ? h1 : h0;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (((vm >> j) & 1u) && key_prefix(key[j], pbits) == P) atomicAdd(&hc[(key[j] >> shift) & mask], 1u);
    lds_barrier();                                 // the histogram is complete
    if (wid == 0) {
      wave_select_bin(hc, 1 << bits, need, res);
    } else {
      uint32_t* hn = cur ? h0 : h1;
      for (int i = threadIdx.x - 64; i < kBins1; i += NT - 64) hn[i] = 0u;
    }
    lds_barrier();                                 // *res is set, the next histogram clear
    const BinSel s = *res;
    P = (P << bits) | s.bin;
    pbits += bits;
    need -= s.above;
    cnt = s.cnt;
    cur ^= 1;
  }
}

}  // namespace dsa
