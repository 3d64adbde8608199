// Lightning indexer on gfx950: the indexer heads of a query row contracted
// with a stream of FP8 keys on the matrix cores, ReLU and head-weighted sum
// fused in registers (ouchyi.pink post on DSA, the DSA paragraph: few heads,
// FP8; tenelement.pl article "DeepSeek V3.2-Exp Cuts Long-Context Costs with
// DeepSeek Sparse Attention (DSA) While Maintaining Benchmark Parity",
// section "Architektura DeepSeek V3.2-Exp: Od MoE do DSA": ReLU logits).
//
//   I[t,s] = k_scale[s] * sum_j (w[t,j] * q_scale[t]) * ReLU(q8[t,j] . k8[s])
//
// Keys stay FP8 (e4m3fn) in HBM and on the load path; each lane widens its
// fragment in registers with v_cvt_scalef32_pk_bf16_fp8 (exact: every e4m3fn
// value is a bf16 value) and the contraction runs on
// v_mfma_f32_16x16x32_bf16.  The FP8 MFMA forms were measured to sum their
// products in a window of about 20 bits below the largest product (error up
// to 1.4e-5 of sum|q_d k_d|), which moves scores near the top-k threshold by
// ~1e-4 relative; the bf16 form accumulates to fp32 rounding.  Decode is
// HBM-bound, so the wider MFMA costs no time there.
//
// MFMA mapping: M = indexer heads (16 per tile), N = 16 keys, K = 32 dims per
// instruction, d_I/32 instructions chained through the accumulator.  Lane l
// holds key (l % 16) and heads 4*(l/16)+i of each tile, so the head sum is
// 4*HT in-lane FMAs plus two cross-lane adds.  The contraction index is split
// over the four 16-lane groups the same way for both operands (group g holds
// bytes [g*d_I/4, (g+1)*d_I/4) of a row; instruction c takes 8 of them),
// which is all a dot product needs.
//
// Two layouts share the kernel:
//   decode  (one query row per sequence): the 4 waves of a workgroup split a
//           chunk of keys; key bytes are streamed once with non-temporal
//           loads; optionally the kernel also builds the first-pass top-k
//           histogram (high 11 bits of the order key) of its row.
//   prefill (many rows per sequence): each wave owns kIdxRowsPerWave rows
//           and walks the whole key chunk, so each key tile feeds
//           HT*d_I/32*kIdxRowsPerWave MFMAs; key chunks past the tile's last
//           position are skipped (causality).
#include "dsa_common.h"
#include "dsa_kernels.h"
#include "idx_math.h"

namespace dsa {

template <int HT, int DI, int R, int RW, bool HIST>
__global__ void __launch_bounds__(256) indexer_kernel(IndexerArgs a) {
  constexpr int KW = 4 / RW;            // waves sharing one row group (they split the keys)
  constexpr bool STREAM = (RW == 1);    // decode: every key byte is read exactly once
  constexpr int U = (R == 1) ? 4 : 2;   // key tiles per pipeline stage
  static_assert(!HIST || (R == 1 && RW == 1), "histogram needs one row per workgroup");
  __shared__ uint32_t hist[HIST ? kBins1 : 1];

  const int b = blockIdx.z;
  const int ytile = blockIdx.x % a.ntiles;
  const int chunk_id = blockIdx.x / a.ntiles;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nl = lane & 15, grp = lane >> 4;
  const int rg = wave / KW, kw = wave % KW;

  const int len = a.g.seq_lens[b];
  int row0, nq;
  if (a.g.q_start) {
    row0 = a.g.q_start[b];
    nq = a.g.q_start[b + 1] - row0;
  } else {
    row0 = b;
    nq = 1;
  }
  const int tile_r0 = ytile * (RW * R);
  if (tile_r0 >= nq) return;
  const int base_pos = len - nq;                      // position of the sequence's first query row
  const int last_r = min(tile_r0 + RW * R, nq) - 1;
  const int kbeg = chunk_id * a.chunk;
  const int kend = min(kbeg + a.chunk, base_pos + last_r + 1);
  if (kbeg >= kend) return;                           // uniform over the workgroup

  if constexpr (HIST) {
    for (int i = threadIdx.x; i < kBins1; i += 256) hist[i] = 0u;
    __syncthreads();
  }

  // ---- this wave's query rows: widened A operands and folded head weights in registers
  Wide<DI> qa[R][HT];
  float wq[R][HT][4];
  int nrow[R];
  int64_t trow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int ri = tile_r0 + rg * R + r;
    const bool ok = ri < nq;
    nrow[r] = ok ? base_pos + ri + 1 : 0;
    const int t = row0 + (ok ? ri : 0);
    trow[r] = t;
    const float qs = a.q_scale ? a.q_scale[t] : 1.0f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 16 + nl;
      Frag<DI> raw;
      if (ok && h < a.H_I)
        load_frag<DI, false>(raw, reinterpret_cast<const char*>(a.q8) + ((int64_t)t * a.H_I + h) * DI, grp);
      else
        zero_frag<DI>(raw);
      qa[r][ht] = widen<DI>(raw);
      const int hw = ht * 16 + grp * 4;
      const float4 w4 = (ok && hw < a.H_I) ? *reinterpret_cast<const float4*>(a.w + (int64_t)t * a.H_I + hw)
                                           : make_float4(0.f, 0.f, 0.f, 0.f);
      wq[r][ht][0] = w4.x * qs;
      wq[r][ht][1] = w4.y * qs;
      wq[r][ht][2] = w4.z * qs;
      wq[r][ht][3] = w4.w * qs;
    }
  }

  // ---- key tiles of 16 keys; this wave takes tiles kw, kw+KW, ...
  const int ntiles = (kend - kbeg + 15) >> 4;
  const int my_tiles = ntiles > kw ? (ntiles - kw + KW - 1) / KW : 0;

  auto load_stage = [&](Frag<DI> (&kt)[U], float (&ks)[U], int m0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (m0 + u < my_tiles) {
        const int s = kbeg + ((kw + KW * (m0 + u)) << 4) + nl;
        const int sl = min(s, kend - 1);
        load_frag<DI, STREAM>(kt[u], token_ptr(a.g, a.kidx, b, sl), grp);
        ks[u] = a.ksc.data ? *reinterpret_cast<const float*>(token_ptr(a.g, a.ksc, b, sl)) : 1.0f;
      }
    }
  };

  auto compute_stage = [&](const Frag<DI> (&kt)[U], const float (&ks)[U], int m0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (m0 + u < my_tiles) {
        const int s0 = kbeg + ((kw + KW * (m0 + u)) << 4);
        const Wide<DI> kb = widen<DI>(kt[u]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (s0 < nrow[r]) {                         // wave-uniform causal skip
            float part = 0.0f;
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
              const v4f acc = mfma_dot<DI>(qa[r][ht], kb);
#pragma unroll
              for (int i = 0; i < 4; ++i) part = fmaf(wq[r][ht][i], relu(acc[i]), part);
            }
            part = group_sum(part);
            const int s = s0 + nl;
            if (grp == 0 && s < nrow[r]) {
              const float sc = part * ks[u];
              a.scores[trow[r] * a.ld + s] = sc;
              if constexpr (HIST) atomicAdd(&hist[score_key(sc) >> (32 - kBins1Bits)], 1u);
            }
          }
        }
      }
    }
  };

  Frag<DI> bufA[U], bufB[U];
  float ksA[U], ksB[U];
  load_stage(bufA, ksA, 0);
  for (int m0 = 0; m0 < my_tiles; m0 += 2 * U) {
    if (m0 + U < my_tiles) load_stage(bufB, ksB, m0 + U);
    compute_stage(bufA, ksA, m0);
    if (m0 + U >= my_tiles) break;
    if (m0 + 2 * U < my_tiles) load_stage(bufA, ksA, m0 + 2 * U);
    compute_stage(bufB, ksB, m0 + U);
  }

  if constexpr (HIST) {
    __syncthreads();
    uint32_t* gh = a.hist + (int64_t)row0 * kBins1;
    for (int i = threadIdx.x; i < kBins1; i += 256) {
      const uint32_t c = hist[i];
      if (c) atomicAdd(gh + i, c);
    }
  }
}

// ---------------------------------------------------------------------------
// Decode indexer with an LDS ring per wave (d_I = 128).
//
// Each wave streams its own 16-key tiles through a ring of kRing slots in
// LDS.  Tiles arrive by global_load_lds DMA with the streaming (nt) hint:
// every 1 KB instruction covers 8 whole keys, so HBM reads are fully
// coalesced, and kRing-1 tiles (about 8 KB per wave) are in flight with no
// registers held for them.  Five slots keep a workgroup at 50 KB of LDS, so
// three workgroups (twelve waves) share a CU; more waves per SIMD hide the
// MFMA/epilogue latency of each tile better than a deeper ring does.
// Inside a slot, the 16-byte chunk c of key n sits at chunk c ^ kswz(n).
// With 128-byte keys, kswz(n) = (n & 7) ^ (n >> 3 & 1) measured free of bank
// conflicts for the operand reads below (16 keys x one chunk per lane group),
// while (n >> 1) & 7 measured about 1.6x slower.
// The DMA is inline asm and its completion is awaited with explicit
// s_waitcnt vmcnt(N): vector-memory operations complete in issue order, so
// "at most N operations outstanding" means everything older has landed; N
// counts the score stores that share the counter.
constexpr int kRing = 5;

__device__ __forceinline__ int kswz(int n) { return (n & 7) ^ ((n >> 3) & 1); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

template <int HT, bool HIST, bool SCALE>
__global__ void __launch_bounds__(256) indexer_decode_ring_kernel(IndexerArgs a) {
  constexpr int DI = 128;
  constexpr int SLOT = 16 * DI + 64;          // key bytes + 16 fp32 scales
  constexpr int PER = SCALE ? 3 : 2;          // DMA instructions per tile
  // The chunk's scores collect in LDS and leave in one coalesced pass after
  // the ring has drained, so no global store shares the vector-memory counter
  // the ring waits on; the histogram is then built in the ring's space.
  __shared__ __attribute__((aligned(16))) float sbuf[kIdxDecodeChunk];
  __shared__ __attribute__((aligned(16))) char ring[4][kRing][SLOT];
  static_assert(!HIST || sizeof(ring) >= kBins1 * sizeof(uint32_t), "histogram fits the ring");

  const int b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nl = lane & 15, grp = lane >> 4;

  const int len = a.g.seq_lens[b];
  const int kbeg = blockIdx.x * a.chunk;
  const int kend = min(kbeg + a.chunk, len);
  if (kbeg >= kend) return;                   // uniform over the workgroup
  // q_scale[b] through the scalar cache: a vector load here would make the
  // compiler wait on the vector-memory counter, which the ring DMA shares
  const float qs = a.q_scale ? *(const __attribute__((address_space(4))) float*)(uintptr_t)(a.q_scale + b) : 1.0f;

  const int ntiles = (kend - kbeg + 15) >> 4;
  const int my_tiles = ntiles > wave ? (ntiles - wave + 3) / 4 : 0;   // tiles wave, wave+4, ...
  char* myring = &ring[wave][0][0];
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)myring;

  // Byte offsets, relative to the tile's first key row, of the two 16-byte
  // chunks this lane moves for a full tile (slot chunk p = 64 i + lane holds
  // chunk p & 7 ^ swizzle of key p >> 3), and of its key scale.  They do not
  // change from tile to tile, so a full tile's DMA needs only a scalar base
  // address.  32-bit offsets need 16 rows to span less than 2 GiB.
  const bool off32 = a.kidx.row_stride < (1 << 26) && (!SCALE || a.ksc.row_stride < (1 << 26));
  const int n0 = lane >> 3, n1 = 8 + (lane >> 3), pc = lane & 7;
  const uint32_t koff0 = (uint32_t)(n0 * a.kidx.row_stride) + 16u * (uint32_t)(pc ^ kswz(n0));
  const uint32_t koff1 = (uint32_t)(n1 * a.kidx.row_stride) + 16u * (uint32_t)(pc ^ kswz(n1));
  const uint32_t soff = SCALE ? (uint32_t)(min(lane, 15) * a.ksc.row_stride) : 0u;

  // A 16-key tile never straddles a page (pages hold a power-of-two >= 16
  // tokens and tiles start at multiples of 16), so its keys are consecutive
  // token rows starting at the row of its first key.  That row is computed
  // from wave-uniform values, so any page-table read is a scalar load and
  // does not disturb the vector-memory counter the ring relies on.
  auto tile_row0 = [&](int s0) -> int64_t {
    const int su = __builtin_amdgcn_readfirstlane(s0);
    if (a.g.block_table) {
      // constant address space: the table is read-only here, so this is an s_load
      const auto* tbl = (const __attribute__((address_space(4))) int32_t*)(uintptr_t)a.g.block_table;
      const int blk = tbl[(int64_t)b * a.g.max_blocks + (su >> a.g.block_shift)];
      return ((int64_t)blk << a.g.block_shift) + (su & ((1 << a.g.block_shift) - 1));
    }
    return (int64_t)b * a.kidx.seq_stride + su;
  };

  auto issue = [&](int m) {                   // DMA of this wave's m-th tile into slot m % kRing
    const int s0 = kbeg + ((wave + 4 * m) << 4);
    const int last = kend - 1 - s0;           // keys past the end re-read the last key
    const int64_t row0 = tile_row0(s0);
    const uint32_t slot = ring_lds + (uint32_t)((m % kRing) * SLOT);
    if (last >= 15 && off32) {                // full tile: scalar base + fixed lane offsets
      const char* kb = a.kidx.data + row0 * a.kidx.row_stride;
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                   :: "s"(slot), "v"(koff0), "s"(kb) : "memory");
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                   :: "s"(slot + 1024u), "v"(koff1), "s"(kb) : "memory");
      if constexpr (SCALE) {
        const char* sb = a.ksc.data + row0 * a.ksc.row_stride;
        if (lane < 16)
          asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2 nt"
                       :: "s"(slot + 16u * DI), "v"(soff), "s"(sb) : "memory");
      }
    } else {                                  // ragged last tile: per-lane 64-bit addresses
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int p = i * 64 + lane;
        const int n = p >> 3;
        const char* src = a.kidx.data + (row0 + min(n, last)) * a.kidx.row_stride + 16 * (pc ^ kswz(n));
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                     :: "s"(slot + i * 1024u), "v"(src) : "memory");
      }
      if constexpr (SCALE) {
        const char* src = a.ksc.data + (row0 + min(lane, last)) * a.ksc.row_stride;
        if (lane < 16)
          asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off nt"
                       :: "s"(slot + 16u * DI), "v"(src) : "memory");
      }
    }
  };

  // The query row arrives through the ring as well: wave w moves indexer
  // heads 16w..16w+15 (laid out and swizzled like a key tile) and their 16
  // head weights into its last slot, then starts its first kRing-1 key tiles
  // before anything waits, so the query and the first tiles are in flight
  // together.  Heads past H_I re-read the last head and are zeroed on use.
  {
    const uint32_t slot = ring_lds + (uint32_t)((kRing - 1) * SLOT);
    const char* qrow = reinterpret_cast<const char*>(a.q8) + (int64_t)b * a.H_I * DI;
    const int qmax = a.H_I * DI - 16;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = i * 64 + lane;
      const int n = p >> 3;
      const char* src = qrow + min((wave * 16 + n) * DI + 16 * (pc ^ kswz(n)), qmax);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                   :: "s"(slot + i * 1024u), "v"(src) : "memory");
    }
    const float* wsrc = a.w + (int64_t)b * a.H_I + min(wave * 16 + lane, a.H_I - 1);
    if (lane < 16)
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                   :: "s"(slot + 16u * DI), "v"(wsrc) : "memory");
  }
  for (int m = 0; m < kRing - 1 && m < my_tiles; ++m) issue(m);
  if (my_tiles >= kRing - 1)
    wait_vmcnt<(kRing - 1) * PER>();          // this wave's query heads have landed
  else
    wait_vmcnt<0>();
  // LDS-only fences: the barrier must not wait for the key tiles in flight
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

  const int rb0 = nl * DI + 16 * ((2 * grp) ^ kswz(nl));
  const int rb1 = nl * DI + 16 * ((2 * grp + 1) ^ kswz(nl));

  // widened A operands and folded head weights in registers
  Wide<DI> qa[HT];
  float wq[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const char* qslot = &ring[ht][kRing - 1][0];
    Frag<DI> raw;
    raw.lo = *reinterpret_cast<const v4i*>(qslot + rb0);
    raw.hi = *reinterpret_cast<const v4i*>(qslot + rb1);
    if (ht * 16 + nl >= a.H_I) zero_frag<DI>(raw);
    qa[ht] = widen<DI>(raw);
    // heads ht*16+4*grp .. +3 (H_I is a multiple of 4)
    const float4 w4 = *reinterpret_cast<const float4*>(qslot + 16 * DI + 16 * grp);
    const bool hv = ht * 16 + grp * 4 < a.H_I;
    wq[ht][0] = hv ? w4.x * qs : 0.0f;
    wq[ht][1] = hv ? w4.y * qs : 0.0f;
    wq[ht][2] = hv ? w4.z * qs : 0.0f;
    wq[ht][3] = hv ? w4.w * qs : 0.0f;
  }
  // every wave has read the query slots before any wave refills its last slot
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

  for (int m = 0; m < my_tiles; ++m) {
    if (m + kRing - 1 < my_tiles) {
      issue(m + kRing - 1);
      wait_vmcnt<(kRing - 1) * PER>();        // only this wave's DMA is in flight
    } else {
      wait_vmcnt<0>();
    }
    const char* slot = myring + (m % kRing) * SLOT;
    Frag<DI> kf;
    kf.lo = *reinterpret_cast<const v4i*>(slot + rb0);
    kf.hi = *reinterpret_cast<const v4i*>(slot + rb1);
    const float ks = SCALE ? *reinterpret_cast<const float*>(slot + 16 * DI + 4 * nl) : 1.0f;
    const Wide<DI> kb = widen<DI>(kf);
    float part = 0.0f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const v4f acc = mfma_dot<DI>(qa[ht], kb);
#pragma unroll
      for (int i = 0; i < 4; ++i) part = fmaf(wq[ht][i], relu(acc[i]), part);
    }
    part = group_sum(part);                   // the four lane groups holding key nl
    if (grp == 0) sbuf[((wave + 4 * m) << 4) + nl] = part * ks;   // keys past kend are never read
  }

  lds_barrier();                              // every wave's scores are in; the ring is drained
  const int nk = kend - kbeg;
  float* srow = a.scores + (int64_t)b * a.ld + kbeg;
  for (int i = threadIdx.x; i < nk; i += 256) srow[i] = sbuf[i];
  if constexpr (HIST) {
    uint32_t* hist = reinterpret_cast<uint32_t*>(&ring[0][0][0]);
    for (int i = threadIdx.x; i < kBins1; i += 256) hist[i] = 0u;
    lds_barrier();
    for (int i = threadIdx.x; i < nk; i += 256) atomicAdd(&hist[score_key(sbuf[i]) >> (32 - kBins1Bits)], 1u);
    lds_barrier();                            // the histogram is complete
    uint32_t* gh = a.hist + (int64_t)b * kBins1;
    for (int i = threadIdx.x; i < kBins1; i += 256) {
      const uint32_t c = hist[i];
      if (c) atomicAdd(gh + i, c);
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill indexer with a workgroup-shared LDS ring (d_I = 128).
//
// A workgroup owns 8 consecutive query rows of one sequence (2 per wave) and
// one chunk of keys.  Keys move through a ring of kPreRing slots of 64 keys,
// filled by DMA that all four waves share (each wave moves a quarter of every
// slot), so each key byte crosses from L2 once per workgroup and feeds 8 rows
// x H_I heads of MFMAs.  One barrier per slot publishes it and retires the
// slot the next DMA overwrites.  Rows compute every key of a full slot, also
// keys past their own position (those entries of the score matrix are
// unspecified), so every wave stores the same number of scores per slot and
// the vector-memory counter the ring waits on stays exact.
//
// FILT (the streaming prefill selection): no score is stored.  Each wave
// keeps, per row, the (key, token) pairs whose order (key desc, token asc)
// reaches the row's threshold in an LDS buffer, one ballot-compacted append
// per 64-key slot, and flushes the buffer as a segment of the row's candidate
// list (see stream.hip).  The reservation atomic of a flush waits for every
// older DMA of the wave, so the ring waits stay correct, only longer, when a
// flush falls inside the loop.  kshift > 0 runs the kernel over a compacted
// sample of every 2^kshift-th token (causal bound p >> kshift).
//
// F8 (filtered pass only): the scores come from
// v_mfma_scale_f32_16x16x128_f8f6f4 on the raw e4m3 bytes (one instruction
// per 16 heads x 16 keys, 3.3x the measured issue rate of the bf16 form) and
// nothing is rescored here.  The FP8 score differs from the exact one (the
// bf16 arithmetic of the other variants) by at most m = kF8ErrRel * 448 * ks
// * sum_h |w_h qs| max_d |q8_hd|: the matrix core's FP8 dot product is within
// kF8ErrRel/2 of max_d |q_d| * max_d |k_d| of the exact one (tests pin it at
// 2^-10), |k8_d| <= 448, ReLU is 1-Lipschitz, and the other half of the
// budget covers the bf16 path's own fp32 rounding.  Every key whose estimate
// plus m reaches the threshold's key is kept with its estimate and m (so
// every pair the exact filter keeps is among them), and
// stream_exactify_kernel settles each row from the bounds estimate +- m.
constexpr int kPreRing = 6;
constexpr int kPreKeys = 64;
constexpr float kF8ErrRel = 0x1p-7f;

// v[g] of four values (selects: an indexed array would go to scratch memory).
__device__ __forceinline__ float sel4(int g, float v0, float v1, float v2, float v3) {
  const float lo = (g & 1) ? v1 : v0;
  const float hi = (g & 1) ? v3 : v2;
  return (g & 2) ? hi : lo;
}

__device__ __forceinline__ v8i frag_v8i(const Frag<128>& f) {
  return v8i{f.lo.x, f.lo.y, f.lo.z, f.lo.w, f.hi.x, f.hi.y, f.hi.z, f.hi.w};
}

template <int HT, bool SCALE, bool FILT, bool F8 = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) indexer_prefill_ring_kernel(IndexerArgs a) {
  static_assert(!F8 || FILT, "the FP8 contraction serves the filtered pass");
  constexpr int DI = 128;
  constexpr int R = 2;                                // rows per wave
  constexpr int SLOT = kPreKeys * DI + kPreKeys * 4;  // keys + scales
  constexpr int PER = SCALE ? 3 : 2;                  // DMA instructions per wave per slot
  constexpr int ST = FILT ? 0 : R * (kPreKeys / 16);  // score stores per wave per slot
  __shared__ __attribute__((aligned(16))) char ring[kPreRing][SLOT];
  // FILT: this wave's candidate buffers, one per row (kStreamLds pairs each)
  __shared__ uint2 cand[FILT ? 4 * R * kStreamLds : 1];

  const int b = blockIdx.z;
  const int ytile = blockIdx.x % a.ntiles;
  const int chunk_id = blockIdx.x / a.ntiles;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nl = lane & 15, grp = lane >> 4;

  const int len = a.g.seq_lens[b];
  const int row0 = a.g.q_start[b];
  const int nq = a.g.q_start[b + 1] - row0;
  const int tile_r0 = ytile * 4 * R;
  if (tile_r0 >= nq) return;
  const int base_pos = len - nq;
  const int last_r = min(tile_r0 + 4 * R, nq) - 1;
  const int kbeg = chunk_id * a.chunk;
  const int kend = min(kbeg + a.chunk, ((base_pos + last_r) >> a.kshift) + 1);
  if (kbeg >= kend) return;                           // uniform over the workgroup
  const int nslots = (kend - kbeg + kPreKeys - 1) / kPreKeys;
  // a partial row tile stores fewer scores per slot: it waits for everything
  const bool exact = tile_r0 + 4 * R <= nq;

  const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&ring[0][0];
  const bool off32 = a.kidx.row_stride < (1 << 26) && (!SCALE || a.ksc.row_stride < (1 << 26));
  // lane offsets of this wave's two DMA instructions (slot keys 8i .. 8i+7,
  // i = 2*wave + {0, 1}): key 8i + (lane >> 3), chunk (lane & 7) ^ swizzle;
  // the swizzle of key n depends on n & 7 = lane >> 3 and on n >> 3 & 1 = i & 1
  const int kn = lane >> 3, pc = lane & 7;
  const uint32_t koff[2] = {(uint32_t)(kn * a.kidx.row_stride) + 16u * (uint32_t)(pc ^ kswz(kn)),
                            (uint32_t)(kn * a.kidx.row_stride) + 16u * (uint32_t)(pc ^ kswz(8 + kn))};
  const uint32_t soff = SCALE ? (uint32_t)(min(lane, 15) * a.ksc.row_stride) : 0u;

  // first token row of 8 keys starting at s0 (8 keys never straddle a page)
  auto row_of = [&](int s0) -> int64_t {
    const int su = __builtin_amdgcn_readfirstlane(s0);
    if (a.g.block_table) {
      const auto* tbl = (const __attribute__((address_space(4))) int32_t*)(uintptr_t)a.g.block_table;
      const int blk = tbl[(int64_t)b * a.g.max_blocks + (su >> a.g.block_shift)];
      return ((int64_t)blk << a.g.block_shift) + (su & ((1 << a.g.block_shift) - 1));
    }
    return (int64_t)b * a.kidx.seq_stride + su;
  };

  auto issue = [&](int m) {
    const uint32_t slot = ring_lds + (uint32_t)((m % kPreRing) * SLOT);
    const int sbase = kbeg + m * kPreKeys;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = 2 * wave + h;                     // 8-key group of the slot
      const int s0 = sbase + 8 * i;
      const int last = kend - 1 - s0;                 // keys past the end re-read the last key
      if (last >= 7 && off32) {
        const char* kb = a.kidx.data + row_of(s0) * a.kidx.row_stride;
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :: "s"(slot + i * 1024u), "v"(koff[h]), "s"(kb) : "memory");
      } else {
        // ragged group: keys past kend re-read key kend-1; a group wholly past
        // kend (last < 0) may start beyond the sequence, so it never looks up
        // its own page and takes the page of key kend-1 instead
        const int64_t r = last >= 0 ? row_of(s0) + min(kn, last) : token_row(a.g, a.kidx, b, kend - 1);
        const char* src = a.kidx.data + r * a.kidx.row_stride + 16 * (pc ^ kswz(8 * (i & 1) + kn));
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                     :: "s"(slot + i * 1024u), "v"(src) : "memory");
      }
    }
    if constexpr (SCALE) {
      const int s0 = sbase + 16 * wave;              // this wave's 16 scales
      const int last = kend - 1 - s0;
      const uint32_t dst = slot + (uint32_t)(kPreKeys * DI + 64 * wave);
      if (last >= 15 && off32) {
        // 16 keys never straddle a page; the page comes from a scalar lookup,
        // which leaves the vector-memory counter of the ring alone
        const int64_t srow = a.g.block_table ? row_of(s0) : (int64_t)b * a.ksc.seq_stride + s0;
        const char* sb = a.ksc.data + srow * a.ksc.row_stride;
        if (lane < 16)
          asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                       :: "s"(dst), "v"(soff), "s"(sb) : "memory");
      } else {
        const int key = s0 + min(lane, max(last, 0));
        const char* src = a.ksc.data + token_row(a.g, a.ksc, b, min(key, kend - 1)) * a.ksc.row_stride;
        if (lane < 16)
          asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                       :: "s"(dst), "v"(src) : "memory");
      }
    }
  };

  // ring prologue first, then this wave's query rows (their loads overlap the
  // prologue; the compiler waits for both before the rows are used)
  for (int m = 0; m < kPreRing - 1 && m < nslots; ++m) issue(m);

  Wide<DI> qa[F8 ? 1 : R][F8 ? 1 : HT];
  Frag<DI> q8[F8 ? R : 1][F8 ? HT : 1];             // F8: the raw query bytes
  float marg[R];                                      // F8: score error bound per unit key scale
  float wq[R][HT][4];
  int64_t trow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int ri = tile_r0 + wave * R + r;
    const bool ok = ri < nq;
    const int t = row0 + (ok ? ri : 0);
    trow[r] = ok ? t : -1;
    const float qs = a.q_scale ? a.q_scale[t] : 1.0f;
    marg[r] = 0.0f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 16 + nl;
      Frag<DI> raw;
      if (h < a.H_I)
        load_frag<DI, false>(raw, reinterpret_cast<const char*>(a.q8) + ((int64_t)t * a.H_I + h) * DI, grp);
      else
        zero_frag<DI>(raw);
      if constexpr (F8) {
        q8[r][ht] = raw;
        // |w_h qs| max_d |q8_hd| of head h, summed over the 16 heads below
        const Wide<DI> wv = widen<DI>(raw);
        float mq = 0.0f;
#pragma unroll
        for (int c = 0; c < DI / 32; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) mq = fmaxf(mq, fabsf((float)wv.c[c][e]));
        mq = fmaxf(mq, __shfl_xor(mq, 16));
        mq = fmaxf(mq, __shfl_xor(mq, 32));
        float c = h < a.H_I ? fabsf(a.w[(int64_t)t * a.H_I + h] * qs) * mq : 0.0f;
        c += __shfl_xor(c, 1);
        c += __shfl_xor(c, 2);
        c += __shfl_xor(c, 4);
        c += __shfl_xor(c, 8);
        marg[r] += c;
      } else {
        qa[r][ht] = widen<DI>(raw);
      }
      const int hw = ht * 16 + grp * 4;
      const float4 w4 = hw < a.H_I ? *reinterpret_cast<const float4*>(a.w + (int64_t)t * a.H_I + hw)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
      wq[r][ht][0] = w4.x * qs;
      wq[r][ht][1] = w4.y * qs;
      wq[r][ht][2] = w4.z * qs;
      wq[r][ht][3] = w4.w * qs;
    }
    // the bound on 448 * max|q8| * max|k8| relative terms, inflated by 2^-10
    // for the rounding of x + margin below
    if constexpr (F8) marg[r] *= kF8ErrRel * 448.0f * (1.0f + 0x1p-10f);
  }
  // FILT: per row its position (-1: no row), threshold, buffered pairs and
  // the number of segments this workgroup has flushed for it (all uniform)
  int rpos[R];
  unsigned long long rthr[R];
  uint32_t ccnt[R], cfl[R];
  if constexpr (FILT) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int ri = tile_r0 + wave * R + r;
      rpos[r] = ri < nq ? base_pos + ri : -1;
      rthr[r] = ri < nq ? a.thr[row0 + ri] : ~0ull;
      ccnt[r] = 0u;
      cfl[r] = 0u;
    }
  }
  uint2* const mycand = &cand[FILT ? wave * R * kStreamLds : 0];
  // Move the buffered pairs of the rows in `which` (bit r) to their lists.
  // Lane r reserves row r's space and segment number with a 64-bit atomic (one
  // instruction, one round trip for both rows), then the pairs and each
  // segment record (chunk, flush number, base, count) are stored.  Pairs past
  // the row's capacity are dropped; the finalize sees the total and
  // recomputes the row.
  static_assert(R == 2, "flush reserves two rows with one atomic");
  auto flush = [&](uint32_t which) {
    const uint32_t act = (which & 1u & (ccnt[0] ? 1u : 0u)) | (which & 2u & (ccnt[1] ? 2u : 0u));
    if (!act) return;
    unsigned long long old = 0ull;
    if (lane < R && ((act >> lane) & 1u)) {
      const int64_t t = lane == 0 ? trow[0] : trow[1];
      const uint32_t c = lane == 0 ? ccnt[0] : ccnt[1];
      old = atomicAdd(&a.rowinfo[t], (1ull << 32) | (unsigned long long)c);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (!((act >> r) & 1u)) continue;
      const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)old, r);
      const uint32_t seg = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(old >> 32), r);
      const uint32_t c = ccnt[r];
      const int64_t t = trow[r];
      const uint2* src = mycand + r * kStreamLds;
      uint2* dst = a.lists + t * a.cap;
      for (uint32_t i = lane; i < c; i += 64)
        if (base + i < (uint32_t)a.cap) dst[base + i] = src[i];
      if (lane == 0 && seg < (uint32_t)kStreamMaxSegs)
        a.segs[t * kStreamMaxSegs + seg] = make_uint2(((uint32_t)chunk_id << 3) | cfl[r], (base << 16) | c);
      ccnt[r] = 0u;
      cfl[r] += 1u;
    }
  };
  __builtin_amdgcn_s_waitcnt(0x0F70);                 // rows and ring prologue are in

  const int rb0 = nl * DI + 16 * ((2 * grp) ^ kswz(nl));
  const int rb1 = nl * DI + 16 * ((2 * grp + 1) ^ kswz(nl));
  for (int m = 0; m < nslots; ++m) {
    const bool more = m + kPreRing - 1 < nslots;
    if (more && exact) {
      // Ops after this wave's slot-m DMA: the DMA of the next kPreRing-2
      // slots and, once the ring is full, the stores of kPreRing-1 slots.
      if (m >= kPreRing - 1)
        wait_vmcnt<(kPreRing - 2) * PER + (kPreRing - 1) * ST>();
      else
        wait_vmcnt<(kPreRing - 2) * PER>();
    } else {
      wait_vmcnt<0>();
    }
    // every wave's part of slot m is in; every wave is done with slot m-1
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (more) issue(m + kPreRing - 1);
    if constexpr (FILT) {
      // room for this slot's pairs (at most kPreKeys per row), so the
      // per-slot append below needs no capacity check
      const uint32_t full = (ccnt[0] > (uint32_t)(kStreamLds - kPreKeys) ? 1u : 0u) |
                            (ccnt[1] > (uint32_t)(kStreamLds - kPreKeys) ? 2u : 0u);
      if (full) flush(full);
    }

    const char* slot = &ring[m % kPreRing][0];
    float fv[FILT ? kPreKeys / 16 : 1][R];              // FILT: scores of key group j, row r
#pragma unroll
    for (int j = 0; j < kPreKeys / 16; ++j) {
      Frag<DI> kf;
      kf.lo = *reinterpret_cast<const v4i*>(slot + j * 16 * DI + rb0);
      kf.hi = *reinterpret_cast<const v4i*>(slot + j * 16 * DI + rb1);
      const float ks = SCALE ? *reinterpret_cast<const float*>(slot + kPreKeys * DI + 4 * (16 * j + nl)) : 1.0f;
      if constexpr (F8) {
        const v8i k8 = frag_v8i(kf);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float part = 0.0f;
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) {
            const v4f acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(frag_v8i(q8[r][ht]), k8,
                                                                              v4f{0.f, 0.f, 0.f, 0.f},
                                                                              0, 0, 0, 127, 0, 127);
#pragma unroll
            for (int i = 0; i < 4; ++i) part = fmaf(wq[r][ht][i], relu(acc[i]), part);
          }
          fv[j][r] = group_sum(part) * ks;            // the FP8 estimate of key 16j + nl
        }
      } else {
        const Wide<DI> kb = widen<DI>(kf);
        const int s = kbeg + m * kPreKeys + 16 * j + nl;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float part = 0.0f;
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) {
            const v4f acc = mfma_dot<DI>(qa[F8 ? 0 : r][F8 ? 0 : ht], kb);
#pragma unroll
            for (int i = 0; i < 4; ++i) part = fmaf(wq[r][ht][i], relu(acc[i]), part);
          }
          part = group_sum(part);
          if constexpr (FILT)
            fv[j][r] = part * ks;                     // every lane holds the score of key 16j + nl
          else if (grp == 0 && s < kend && trow[r] >= 0)
            a.scores[trow[r] * a.ld + s] = part * ks;
        }
      }
    }
    if constexpr (F8) {
      // lane l takes key l of the slot; a key whose FP8 estimate plus its
      // bound reaches the row threshold's key is appended with the estimate's
      // key, its token and its bound rounded up to 14 bits (float bits >> 17)
      // above the token (tokens < 2^18); stream_exactify_kernel turns the
      // row's list into exact keys where they decide the selection
      const int sl = kbeg + m * kPreKeys + lane;
      const float ksl = SCALE ? *reinterpret_cast<const float*>(slot + kPreKeys * DI + 4 * lane) : 1.0f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float xt = sel4(grp, fv[0][r], fv[1][r], fv[2][r], fv[3][r]);
        const float mg = marg[r] * fabsf(ksl);
        const bool maybe = sl <= rpos[r] && score_key(xt + mg) >= (uint32_t)(rthr[r] >> 32);
        const uint32_t menc = (__float_as_uint(mg) + ((1u << 17) - 1u)) >> 17;
        const unsigned long long mm = __ballot(maybe);
        const uint32_t before = __builtin_amdgcn_mbcnt_hi((uint32_t)(mm >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mm, 0u));
        if (maybe) mycand[r * kStreamLds + ccnt[r] + before] = make_uint2(score_key(xt), (uint32_t)sl | (menc << 18));
        ccnt[r] += (uint32_t)__popcll(mm);
      }
    } else if constexpr (FILT) {
      // lane (g, l) takes key 16g + l of the slot, so the 64 lanes hold the
      // slot's keys in token order: one ballot and one append per row keep
      // (key, token) when token <= p and (key, ~token) reaches the threshold
      const int s = kbeg + m * kPreKeys + lane;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float x = grp == 0 ? fv[0][r] : grp == 1 ? fv[1][r] : grp == 2 ? fv[2][r] : fv[3][r];
        const uint32_t key = score_key(x);
        const unsigned long long comp = ((unsigned long long)key << 32) | (uint32_t)~(uint32_t)s;
        const bool keep = s <= rpos[r] && comp >= rthr[r];
        const unsigned long long m64 = __ballot(keep);
        const uint32_t before = __builtin_amdgcn_mbcnt_hi((uint32_t)(m64 >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m64, 0u));
        if (keep) mycand[r * kStreamLds + ccnt[r] + before] = make_uint2(key, (uint32_t)s);
        ccnt[r] += (uint32_t)__popcll(m64);
      }
    }
  }
  if constexpr (FILT) flush(3u);
}

template <int HT, int DI>
static hipError_t launch_ht(const IndexerArgs& a, bool decode_layout, bool with_hist, hipStream_t s) {
  const dim3 grid(a.nchunks * a.ntiles, 1, a.g.num_seqs);
  if (decode_layout && DI == 128) {
    const bool sc = a.ksc.data != nullptr;
    if (with_hist) {
      if (sc) hipLaunchKernelGGL((indexer_decode_ring_kernel<HT, true, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((indexer_decode_ring_kernel<HT, true, false>), grid, dim3(256), 0, s, a);
    } else {
      if (sc) hipLaunchKernelGGL((indexer_decode_ring_kernel<HT, false, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((indexer_decode_ring_kernel<HT, false, false>), grid, dim3(256), 0, s, a);
    }
  } else if (decode_layout) {
    if (with_hist)
      hipLaunchKernelGGL((indexer_kernel<HT, DI, 1, 1, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((indexer_kernel<HT, DI, 1, 1, false>), grid, dim3(256), 0, s, a);
  } else if (DI == 128) {
    if (a.ksc.data) hipLaunchKernelGGL((indexer_prefill_ring_kernel<HT, true, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((indexer_prefill_ring_kernel<HT, false, false>), grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((indexer_kernel<HT, DI, kIdxRowsPerWave, 4, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int DI>
static hipError_t launch_di(const IndexerArgs& a, bool decode_layout, bool with_hist, hipStream_t s) {
  switch ((a.H_I + 15) / 16) {
    case 1: return launch_ht<1, DI>(a, decode_layout, with_hist, s);
    case 2: return launch_ht<2, DI>(a, decode_layout, with_hist, s);
    case 3: return launch_ht<3, DI>(a, decode_layout, with_hist, s);
    case 4: return launch_ht<4, DI>(a, decode_layout, with_hist, s);
    default: return hipErrorInvalidValue;
  }
}

template <int HT>
static hipError_t launch_stream_ht(const IndexerArgs& a, hipStream_t s) {
  const dim3 grid(a.nchunks * a.ntiles, 1, a.g.num_seqs);
  if (a.fp8) {
    if (a.ksc.data) hipLaunchKernelGGL((indexer_prefill_ring_kernel<HT, true, true, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((indexer_prefill_ring_kernel<HT, false, true, true>), grid, dim3(256), 0, s, a);
  } else {
    if (a.ksc.data) hipLaunchKernelGGL((indexer_prefill_ring_kernel<HT, true, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((indexer_prefill_ring_kernel<HT, false, true>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// The prefill layout with the filtered epilogue (d_I = 128): rowinfo must be
// zero and thr set for every row before the launch.
hipError_t launch_indexer_stream(const IndexerArgs& a, hipStream_t stream) {
  switch ((a.H_I + 15) / 16) {
    case 1: return launch_stream_ht<1>(a, stream);
    case 2: return launch_stream_ht<2>(a, stream);
    case 3: return launch_stream_ht<3>(a, stream);
    case 4: return launch_stream_ht<4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_indexer(const IndexerArgs& a, int d_I, bool decode_layout, bool with_hist,
                          hipStream_t stream) {
  if (d_I == 128) return launch_di<128>(a, decode_layout, with_hist, stream);
  if (d_I == 32) return launch_di<32>(a, decode_layout, with_hist, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
