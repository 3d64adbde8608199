// Sparse MQA attention on gfx950: softmax attention of H query heads over
// only the k selected tokens of a row, every head reading the same latent KV
// row (tenelement.pl article "DeepSeek V3.2-Exp Cuts Long-Context Costs with
// DeepSeek Sparse Attention (DSA) While Maintaining Benchmark Parity",
// sections "Architektura DeepSeek V3.2-Exp: Od MoE do DSA" (MQA in decode)
// and "Efektywność Kosztowa" (reuse of the shared KV); degnora.com
// "DeepSeekV3, Farkı Ne?", section "MLA — Multi-Latent Attention").
//
// One workgroup = one query row (all H heads, 16 per wave) and one split of
// its selected slots.  Selected rows are processed kAttnBlock (64) at a time:
//   * gather: global_load_lds_dwordx4 copies each selected row (D bf16)
//     straight from HBM into an LDS tile, no registers involved; tiles are
//     double-buffered so the gather of block i+1 overlaps the math of block i.
//     16-byte chunks of row r are stored at chunk position c ^ ((r>>1)&7), an
//     XOR swizzle that keeps the 16 rows of an MFMA operand in distinct banks.
//   * S^T = K q^T: v_mfma_f32_16x16x32_bf16 with M = 16 selected rows, N = 16
//     heads, K = 32 dims; K comes from the tile (ds_read_b128), q sits in
//     registers.  Lane l ends with head (l%16) and rows 4*(l/16)+i.
//   * online softmax in log2 units with a lazily moved reference max (P <
//     2^8, O rescaled only when a block max jumps past it); P rounded to bf16.
//   * O += P V: M = 16 heads, N = 16 value dims, K = 32 rows.  The S^T
//     accumulator of row tiles 2kb and 2kb+1 is this MFMA's A operand when K
//     slot j of lane group g stands for row 32kb+4g+j (j<4) or 32kb+16+4g+j-4.
//     The matching B operand is read from the same row-major tile with
//     ds_read_b64_tr_b16: lane j of a 16-lane group addresses row R+(j>>2),
//     dims 4*(j&3)..+3, and lane i receives rows R..R+3 of dim i.  So V needs
//     no transposed copy (V = the first D_v dims of the latent row, or a
//     separate cache staged the same way).
// With nsplit > 1 each split writes its normalised partial O (bf16) and lse;
// attn_combine_kernel merges them: out = sum_i exp(lse_i - lse) O_i.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Workgroup id renumbered so that ids dealt to the same XCD (id % 8) form a
// contiguous range; identity when the grid is not a multiple of 8.
__device__ __forceinline__ int xcd_major(int id, int n) {
  return (n & 7) ? id : (id & 7) * (n >> 3) + (id >> 3);
}

// s_waitcnt immediate for "vmcnt(0)" on gfx9-family parts: vmcnt bits [3:0]
// and [15:14] zero, expcnt [6:4] and lgkmcnt [11:8] at their maximum.
constexpr int kWaitVmcnt0 = 0x0F70;

// Issue the gather of one block of kAttnBlock rows (CH chunks each) into `tile`.
// Every wave issues its share of 64-chunk DMA instructions; invalid rows read a
// valid stand-in row (their weight is zero, their values only need be finite).
// The DMA is written as inline asm on purpose: the compiler would otherwise
// make the first LDS read after it wait for it (it cannot tell the two tiles
// apart), which would serialise the double buffering.  Completion is ordered
// explicitly with s_waitcnt vmcnt(0) + a barrier before a tile is read.
template <int CH>
__device__ __forceinline__ void gather_block(char* tile, const char* base, int64_t row_stride,
                                             const uint32_t* rowid, int waves, int wave, int lane) {
  constexpr int RB = kAttnBlock;
  constexpr int NI = RB * CH / 64;                 // DMA instructions per block
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)tile;
  for (int ins = wave; ins < NI; ins += waves) {
    const int p = ins * 64 + lane;                 // chunk position in the tile
    const int r = p / CH, pc = p % CH;
    const int c = pc ^ swz(r);
    const char* src = base + (int64_t)rowid[r] * row_stride + c * 16;
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds0 + ins * 64 * 16);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(m0), "v"(src) : "memory");
  }
}

template <int D, int DV, bool SEPV, int HW>
__global__ void __launch_bounds__(512) attn_kernel(AttnArgs a) {
  // HW head tiles of 16 heads per wave; a workgroup covers H heads
  constexpr int RB = kAttnBlock;
  constexpr int CH = D / 8;                // 16-byte chunks per K row
  constexpr int CHV = SEPV ? DV / 8 : CH;  // chunks per V row
  constexpr int KK = D / 32;               // MFMA K-steps for S
  constexpr int NT = DV / 16;              // output dim tiles
  constexpr int TILE = RB * CH * 16;
  constexpr int VTILE = SEPV ? RB * CHV * 16 : 0;
  constexpr int MAXROWS = kAttnMaxSplit;
  static_assert(D % 32 == 0 && DV % 16 == 0 && DV <= D && CH % 8 == 0 && CHV % 8 == 0, "shape");
  static_assert((RB * CH) % 64 == 0, "tile");
  __shared__ __attribute__((aligned(16))) char ktile[2][TILE];
  __shared__ __attribute__((aligned(16))) char vtile[2][SEPV ? VTILE : 16];
  __shared__ uint32_t rowid[MAXROWS];      // token row of every slot of this split
  __shared__ uint32_t vrowid[SEPV ? MAXROWS : 1];
  __shared__ uint8_t valid[MAXROWS];

  const int waves = blockDim.x >> 6;
  // Workgroups are dealt to the 8 XCDs round-robin by id.  Renumber them so
  // that each XCD gets a contiguous run of (row, split) items: the splits of
  // a row then share one L2, which serves their common q after the first read
  // and keeps the partials near the combine that reads them.
  const int wg = xcd_major(blockIdx.x, gridDim.x);
  const int split = wg % a.nsplit;
  const int t = wg / a.nsplit;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nl = lane & 15, grp = lane >> 4;
  const int h0 = wave * 16 * HW;

  // q fragments (B operand of S^T): head h0+16*ht+nl, dims 32*kk + 8*grp .. +7.
  // Requested first: they depend on nothing, so their latency overlaps the
  // sequence-length and index loads below instead of following them.
  v8bf qf[HW][KK];
#pragma unroll
  for (int ht = 0; ht < HW; ++ht) {
    const int h = h0 + ht * 16 + nl;
    const bool ok = h < a.H;
    const uint16_t* qrow = a.q + ((int64_t)t * a.H + (ok ? h : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const v4i raw = ok ? *reinterpret_cast<const v4i*>(qrow + kk * 32 + grp * 8) : v4i{0, 0, 0, 0};
      qf[ht][kk] = __builtin_bit_cast(v8bf, raw);
    }
  }
  int b, pos;
  row_seq_pos(a.g, t, b, pos);
  const int slot_beg = split * a.per_split;
  const int slot_end = min(a.k, slot_beg + a.per_split);
  const int nslots = slot_end - slot_beg;
  const int nblocks = (nslots + RB - 1) / RB;
  const int32_t* sel = a.idx + (int64_t)t * a.k + slot_beg;

  // token rows of this split's slots; invalid slots borrow token 0 of the sequence
  const uint32_t fallback = (uint32_t)token_row(a.g, a.kv, b, 0);
  const uint32_t vfallback = SEPV ? (uint32_t)token_row(a.g, a.v, b, 0) : 0u;
  for (int i = threadIdx.x; i < nblocks * RB; i += blockDim.x) {
    int s = i < nslots ? sel[i] : -1;
    if (s > pos) s = -1;                   // never attend to the future
    valid[i] = s >= 0;
    rowid[i] = s >= 0 ? (uint32_t)token_row(a.g, a.kv, b, s) : fallback;
    if constexpr (SEPV) vrowid[i] = s >= 0 ? (uint32_t)token_row(a.g, a.v, b, s) : vfallback;
  }

  __syncthreads();

  v4f o[HW][NT];
#pragma unroll
  for (int ht = 0; ht < HW; ++ht)
#pragma unroll
    for (int i = 0; i < NT; ++i) o[ht][i] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run[HW], l_run[HW];   // per head (lane nl of tile ht): running max (log2 units), partial sum
#pragma unroll
  for (int ht = 0; ht < HW; ++ht) {
    m_run[ht] = -INFINITY;
    l_run[ht] = 0.0f;
  }

  // Per-lane LDS operand bases.  The swizzle only permutes chunk bits 0-2 and
  // is the same for every row a lane touches, so each read below is one of
  // these bases plus a compile-time offset.
  //   K fragment (row mt*16+nl, logical chunk 4*kk+grp): bits 0-2 of the chunk
  //   are 4*(kk&1)+grp, the rest is kk>>1 (128 bytes each).
  //   V read (row kb*32+grp*4+(nl>>2) [+16], logical chunk 2*nt+((nl&3)>>1),
  //   +8 bytes for odd nl): bits 0-2 are 2*(nt&3)+((nl&3)>>1), the rest nt>>2.
  int kbase[2], vbase[4];
  {
    const int rk = nl;                                  // + mt*16: same swizzle
    const int yk = swz(rk);
    kbase[0] = (rk * CH + ((0 * 4 + grp) ^ yk)) * 16;
    kbase[1] = (rk * CH + ((1 * 4 + grp) ^ yk)) * 16;
    const int rv = grp * 4 + (nl >> 2);                 // + kb*32 (+16): same swizzle
    const int yv = swz(rv);
#pragma unroll
    for (int u = 0; u < 4; ++u) vbase[u] = (rv * CHV + ((2 * u + ((nl & 3) >> 1)) ^ yv)) * 16 + (nl & 1) * 8;
  }

  auto gather = [&](char* kdst, char* vdst, int blk) {
    gather_block<CH>(kdst, a.kv.data, a.kv.row_stride, rowid + blk * RB, waves, wave, lane);
    if constexpr (SEPV) gather_block<CHV>(vdst, a.v.data, a.v.row_stride, vrowid + blk * RB, waves, wave, lane);
  };

  auto compute = [&](const char* kt, const char* vtv, int blk) {
    const char* vt = SEPV ? vtv : kt;
    const uint8_t* vld = valid + blk * RB;

    // ---- S^T = K q^T: each K fragment read from LDS feeds HW head tiles.
    // One K-step per scheduling region: the scheduler may overlap a step's
    // reads with the previous step's MFMAs but cannot hoist the whole block
    // (which would exhaust registers); the second wave on the SIMD hides the rest.
    v4f s[HW][4];
#pragma unroll
    for (int ht = 0; ht < HW; ++ht)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) s[ht][mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      v8bf kf[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        kf[mt] = *reinterpret_cast<const v8bf*>(kt + kbase[kk & 1] + (kk >> 1) * 128 + mt * 16 * CH * 16);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ht = 0; ht < HW; ++ht)
          s[ht][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mt], qf[ht][kk], s[ht][mt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- online softmax (log2 units), per head tile
    v8bf pf[HW][2];
    float alpha[HW];
#pragma unroll
    for (int ht = 0; ht < HW; ++ht) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = vld[mt * 16 + grp * 4 + i] ? s[ht][mt][i] * a.scale_log2 : -INFINITY;
          s[ht][mt][i] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // Lazy rescaling: the reference max moves only when the block max
      // exceeds it by more than 8 (log2 units), so P stays below 2^8 and the
      // O accumulators are rescaled rarely instead of on most blocks.  While
      // nothing valid has been seen, the reference is -inf and O is zero.
      const float m_old = m_run[ht];
      const bool move = mx > m_old + 8.0f;
      const float m_ref = move ? mx : m_old;
      const float m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;
      alpha[ht] = (move && m_old != -INFINITY) ? __builtin_amdgcn_exp2f(m_old - m_ref) : 1.0f;
      float psum = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(s[ht][mt][i] - m_use);
          psum += p;
          pf[ht][mt >> 1][(mt & 1) * 4 + i] = (__bf16)p;
        }
      }
      l_run[ht] = l_run[ht] * alpha[ht] + psum;
      m_run[ht] = m_ref;
    }

    // rescale O (lane holds heads 4*grp+i of each tile): fetch alpha of those heads
#pragma unroll
    for (int ht = 0; ht < HW; ++ht) {
      if (__any(alpha[ht] != 1.0f)) {
        float ao[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ao[i] = __shfl(alpha[ht], grp * 4 + i);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          o[ht][nt][0] *= ao[0];
          o[ht][nt][1] *= ao[1];
          o[ht][nt][2] *= ao[2];
          o[ht][nt][3] *= ao[3];
        }
      }
    }

    // ---- O += P V, V read transposed from the row-major tile; one read feeds
    // HW head tiles.  One dim tile per scheduling region, like the S loop.
    auto read_v = [&](int nt, int kb) -> v8bf {
      const char* p0 = vt + vbase[nt & 3] + (nt >> 2) * 128 + kb * 32 * CHV * 16;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p0);
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p0 + 16 * CHV * 16));
      return __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      v8bf vf[RB / 32];
#pragma unroll
      for (int kb = 0; kb < RB / 32; ++kb) vf[kb] = read_v(nt, kb);
#pragma unroll
      for (int kb = 0; kb < RB / 32; ++kb)
#pragma unroll
        for (int ht = 0; ht < HW; ++ht)
          o[ht][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[ht][kb], vf[kb], o[ht][nt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (nblocks > 0) gather(ktile[0], vtile[0], 0);
  for (int blk = 0; blk < nblocks; ++blk) {
    const int cur = blk & 1;
    // vmcnt(0) (expcnt/lgkmcnt untouched), as a builtin so the compiler's own
    // wait tracking sees it too
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();   // block blk is in LDS; nobody reads the other buffer any more
    if (blk + 1 < nblocks) gather(ktile[cur ^ 1], vtile[cur ^ 1], blk + 1);
    compute(ktile[cur], vtile[cur], blk);
  }

  // ---- finish: full denominator per head, normalise, write
  uint16_t* obase;
  float* lbase;
  if (a.nsplit == 1) {
    obase = a.out + (int64_t)t * a.H * DV;
    lbase = a.lse ? a.lse + (int64_t)t * a.H : nullptr;
  } else {
    const int64_t base = (int64_t)t * a.nsplit + split;
    obase = a.part_o + base * a.H * DV;
    lbase = a.part_lse + base * a.H;
  }
#pragma unroll
  for (int ht = 0; ht < HW; ++ht) {
    float l_tot = l_run[ht];
    l_tot += __shfl_xor(l_tot, 16);
    l_tot += __shfl_xor(l_tot, 32);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse_h = l_tot > 0.0f ? (m_run[ht] + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    float io[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) io[i] = __shfl(inv, grp * 4 + i);
    const int hb = h0 + ht * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = hb + grp * 4 + i;
      if (h < a.H) {
        uint16_t* orow = obase + (int64_t)h * DV;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) orow[nt * 16 + nl] = bf16_bits(o[ht][nt][i] * io[i]);
      }
    }
    if (lbase && grp == 0 && hb + nl < a.H) lbase[hb + nl] = lse_h;
  }
}

// ---------------------------------------------------------------- 32 heads per wave (H = 128, D = 576)
//
// The production shape runs on v_mfma_f32_32x32x16_bf16, whose measured issue
// rate on this part is 1.76x that of the 16x16x32 form.  A workgroup is four
// waves, one per SIMD, each owning 32 heads: its q fragments (32 heads x 576
// dims, 144 VGPRs) and its output accumulators (32 heads x 512 dims in fp32,
// 256 registers) stay in the wave's 512-entry register file for the whole
// split, so every K or V element read from LDS feeds 32 heads (twice the
// reuse of 16-head waves, half the LDS traffic per FLOP).
//   * tiles of 32 selected rows, gathered by LDS DMA into a 4-slot ring: an
//     iteration reads two tiles (V of tile j, K of tile j+1) while two more
//     are in flight.  Before the first tile each wave stages its q block (32
//     heads x 576 dims, contiguous in HBM) through slot w the same way, with
//     1 KB coalesced DMA instructions, and reads its fragments from there:
//     loading them straight into registers touches 32 rows per instruction
//     and took several microseconds.  The q DMA is issued first; the row's
//     sequence metadata is read by scalar loads meanwhile and the selected
//     ids follow by 4-byte LDS DMA;
//   * S^T = K q^T: A = 32 rows x 16 dims of K (one ds_read_b128 per lane), B =
//     q (registers).  Lane l ends with head l%32 and rows 8(i/4)+4(l/32)+i%4
//     in accumulator i, so a head's softmax is 16 in-lane values and one
//     exchange with lane l^32;
//   * O^T += V^T P^T: A = V^T read transposed from the tile with
//     ds_read_b64_tr_b16 (a 16-lane group reads 4 rows x 16 dims and lane i
//     receives the 4 rows of dim i; two reads give a lane the 8 rows of its
//     K slots), B = P^T straight from the S^T accumulators (K slot j of
//     k-step u is row 16u + 8(j/4) + 4(l/32) + j%4, the same for both
//     operands).  Lane l then holds dims 8(i/4) + 4(l/32) + i%4 of every
//     32-dim tile of head l%32 only: a head's rescale and final 1/l are the
//     lane's own factors, with no exchange;
//   * software pipeline: the softmax of tile j (masking, max, exponentials,
//     bf16 rounding) runs on the VALU between the 36 matrix-core steps of
//     tile j+1's S^T, then P V of tile j follows;
//   * a tile is stored in nine blocks of 8 chunks (128 bytes of each row):
//     16-byte chunk c of row r sits at byte 4096 (c/8) + 128 r +
//     16 ((c%8) ^ f(r)), f(r) = ((r>>1 & 1) << 2) | (r>>2 & 3), so the 16
//     rows of a K read and the 4 rows x 4 chunks of a half-wave's V read land
//     in distinct bank groups.  DMA instruction 4m + w fills block m for rows
//     8w..8w+7: 8 whole 128-byte lines, one per row, and a lane fetches the
//     same row at the same in-block position for every m, so a tile costs one
//     row-id read and one 64-bit address per lane, the block as an immediate
//     offset.
constexpr int kWideRows = 32;       // selected rows per tile
constexpr int kWideSlots = 4;       // tiles in the LDS ring (two read, two in flight)
constexpr int kWideWaves = 4;       // 32 heads each

typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int wswz(int r) {
  const int x = (r >> 1) & 7;
  return ((x & 1) << 2) | (x >> 1);
}

__device__ __forceinline__ v16f mfma32(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Sum (or max) of a value over lanes l and l^32.
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

constexpr int kCombineGroup = 8;      // split partials whose loads a combine thread issues together

__global__ void __launch_bounds__(64 * kWideWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_wide_kernel(AttnArgs a) {
  constexpr int D = 576, DV = 512, CH = D / 8;
  constexpr int TILE = kWideRows * CH * 16;      // 36864 bytes
  constexpr int KK = D / 16;                     // k-steps of S
  constexpr int NT = DV / 32;                    // 32-dim output tiles
  constexpr int NI = kWideRows * CH / 64;        // DMA instructions per tile (36)
  constexpr int NIW = NI / kWideWaves;           // per wave (9)
  constexpr int SPT = kAttnMaxSplit / (64 * kWideWaves);   // slots per thread at most (8)
  static_assert(NI % kWideWaves == 0, "tile split");
  __shared__ __attribute__((aligned(16))) char tiles[kWideSlots][TILE];
  __shared__ uint32_t rowid[kAttnMaxSplit];
  __shared__ uint32_t vmask[kAttnMaxSplit / kWideRows];

  const int wg = xcd_major(blockIdx.x, gridDim.x);
  const int split = wg % a.nsplit;
  const int t = wg / a.nsplit;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n32 = lane & 31, g = lane >> 5;
  const int h0 = wave * 32;

  const uint32_t ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&tiles[0][0];
  // DMA instructions ins0, ins0 + 4, ..., ins0 + 32 of a tile into ring slot
  // `slot`: instruction ins0 + 4m fills slot bytes [1024 (ins0 + 4m), +1024),
  // block m of rows 8 ins0..8 ins0 + 7.  `row` is the source row of this lane
  // (tile row 8 ins0 + l/8; its offset in rows of row_stride bytes from base),
  // the same for all nine.  The instruction's immediate offset (128 m) moves
  // the LDS destination as well as the global address, so M0 is set 128 m
  // below the destination: 1024 ins0 + 3968 m.
  const int drow = lane >> 3;
  auto dma_rows = [&](int slot, const char* base, int64_t row_stride, uint32_t row, int ins0) {
    static_assert(NIW == 9, "nine DMA instructions per wave and tile");
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(ring + (uint32_t)(slot * TILE + ins0 * 1024));
    const char* src = base + (int64_t)row * row_stride + 16 * ((lane & 7) ^ wswz(8 * ins0 + drow));
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
        "s_add_u32 m0, %0, 3968\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:128\n\t"
        "s_add_u32 m0, %0, 7936\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:256\n\t"
        "s_add_u32 m0, %0, 11904\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:384\n\t"
        "s_add_u32 m0, %0, 15872\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:512\n\t"
        "s_add_u32 m0, %0, 19840\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:640\n\t"
        "s_add_u32 m0, %0, 23808\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:768\n\t"
        "s_add_u32 m0, %0, 27776\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:896\n\t"
        "s_add_u32 m0, %0, 31744\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:1024"
        :: "s"(m0), "v"(src) : "memory", "m0", "scc");
  };
  // tile `tile` of the selected rows: the four waves share its DMA instructions
  auto gather = [&](int tile) {
    const uint32_t row = rowid[tile * kWideRows + 8 * wave + drow];
    dma_rows(tile % kWideSlots, a.kv.data, a.kv.row_stride, row, wave);
  };

  // Prologue.  This wave's q block (heads h0..h0+31: 36,864 contiguous
  // bytes, ring slot `wave`) needs only the row, so its DMA goes first; the
  // row's sequence and position are read meanwhile, then the split's selected
  // token ids (and, for paged caches, their block ids) come into rowid[] by
  // LDS DMA.  Vector-memory loads complete in order, so the ids are in once
  // everything is, and no compiler-visible load sits behind the DMA.
  {
    const char* qblock = reinterpret_cast<const char*>(a.q + ((int64_t)t * a.H + h0) * D);
#pragma unroll
    for (int part = 0; part < kWideWaves; ++part)
      dma_rows(wave, qblock, (int64_t)D * 2, (uint32_t)(8 * part + drow), part);
  }
  // The row's sequence and position (as row_seq_pos) through the scalar
  // cache: the tables are read-only here, and scalar loads do not queue
  // behind the DMA on the vector-memory counter.
  int b, pos;
  {
    typedef const __attribute__((address_space(4))) int32_t cint;
    cint* lens = (cint*)(uintptr_t)a.g.seq_lens;
    if (!a.g.q_start) {
      b = t;
      pos = lens[t] - 1;
    } else {
      cint* qst = (cint*)(uintptr_t)a.g.q_start;
      int lo = 0, hi = a.g.num_seqs - 1;            // largest b with q_start[b] <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (qst[mid] <= t) lo = mid; else hi = mid - 1;
      }
      b = lo;
      pos = lens[b] - (qst[b + 1] - qst[b]) + (t - qst[b]);
    }
  }
  const int slot_beg = split * a.per_split;
  const int nslots = min(a.k, slot_beg + a.per_split) - slot_beg;
  const int ntiles = (nslots + kWideRows - 1) / kWideRows;
  const int32_t* sel = a.idx + (int64_t)t * a.k + slot_beg;
  // invalid slots borrow token 0 of the sequence (finite values, zero weight)
  uint32_t fallback;
  if (a.g.block_table) {
    typedef const __attribute__((address_space(4))) int32_t cint;
    const int blk = ((cint*)(uintptr_t)a.g.block_table)[(int64_t)b * a.g.max_blocks];
    fallback = (uint32_t)((int64_t)blk << a.g.block_shift);
  } else {
    fallback = (uint32_t)((int64_t)b * a.kv.seq_stride);
  }
  const uint32_t rid_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&rowid[0];
  // 4-byte LDS DMA of this lane's word for slot i = 256 m + 64 wave + lane into rowid[i]
  auto dma_slot = [&](int m, const void* src) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(rid_lds + 4u * (uint32_t)(64 * kWideWaves * m + 64 * wave));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" :: "s"(m0), "v"(src) : "memory", "m0");
  };
#pragma unroll
  for (int m = 0; m < SPT; ++m) {
    const int i = threadIdx.x + m * 64 * kWideWaves;
    if (i < nslots) dma_slot(m, sel + i);
  }
  int sv[SPT];          // paged: the slots' token ids, kept while their block ids arrive
  if (a.g.block_table) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");      // the id words (and q) are in
#pragma unroll
    for (int m = 0; m < SPT; ++m) {
      const int i = threadIdx.x + m * 64 * kWideWaves;
      int sm = i < nslots ? (int)rowid[i] : -1;
      if (sm > pos) sm = -1;
      sv[m] = sm;
      if (sm >= 0) dma_slot(m, a.g.block_table + (int64_t)b * a.g.max_blocks + (sm >> a.g.block_shift));
    }
  }
  // q and this lane's id (block id) words are in LDS.  Each slot's word was
  // fetched by the lane that now reads and replaces it with the token row;
  // one validity bit per slot.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int m = 0; m < SPT; ++m) {
    const int i = threadIdx.x + m * 64 * kWideWaves;
    if (i < ntiles * kWideRows) {           // whole waves: ntiles * 32 is a multiple of 32
      int sm;
      uint32_t row;
      if (a.g.block_table) {
        sm = sv[m];
        row = sm >= 0 ? (rowid[i] << a.g.block_shift) + (uint32_t)(sm & ((1 << a.g.block_shift) - 1)) : fallback;
      } else {
        sm = i < nslots ? (int)rowid[i] : -1;
        if (sm > pos) sm = -1;
        row = sm >= 0 ? (uint32_t)((int64_t)b * a.kv.seq_stride + sm) : fallback;
      }
      rowid[i] = row;
      const uint64_t bal = __ballot(sm >= 0);
      if ((i & 31) == 0) vmask[i >> 5] = (uint32_t)(bal >> (lane & 32));
    }
  }
  // q fragments (B operand of S^T): head h0 + n32, dims 16kk + 8g .. +7, from
  // this wave's own staging slot (its DMA is complete after vmcnt(0))
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // per-lane LDS operand offsets within a tile.  K (and q): row n32, chunk
  // 2kk + g at byte 4096 (kk/4) + kb[kk%4].  V^T: lane i of 16-lane group G
  // reads row 16u + 8h + 4(G/2) + i/4, chunk 4nt + 2(G&1) + (i/2 & 1), half
  // i&1, at byte 4096 (nt/2) + 2048 u + vb[h][nt&1].
  int kb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) kb[q] = 128 * n32 + 16 * ((2 * q + g) ^ wswz(n32));
  int vb[2][2];
  {
    const int G = lane >> 4, i = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * h + 4 * (G >> 1) + (i >> 2);
      const int y = wswz(row);
#pragma unroll
      for (int np = 0; np < 2; ++np)
        vb[h][np] = 128 * row + 16 * ((4 * np + 2 * (G & 1) + ((i & 3) >> 1)) ^ y) + 8 * (i & 1);
    }
  }
  v8bf qf[KK];
  {
    const char* qs = &tiles[wave][0];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = *reinterpret_cast<const v8bf*>(qs + 4096 * (kk >> 2) + kb[kk & 3]);
  }
  __syncthreads();        // row ids published; every wave holds its q (the slots are free again)

  v16f o[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[nt][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;   // head n32: running max (log2 units) and this lane's partial sum

  // ---- S^T = K q^T of tile jt over 36 k-steps, two accumulator chains in
  // VGPRs (even and odd k-steps; one chain of dependent matrix-core
  // instructions runs at about half the rate).  Written as inline asm so the
  // accumulators stay in VGPRs and the output accumulators keep all 256
  // AGPRs.  Each chain starts from a zero SrcC and accumulates in place
  // (SrcC = VDST, same shape); the last pair is followed by enough wait states
  // (21) for VALU reads of an XDL result, which the compiler does not insert
  // after inline asm.  With one wave per SIMD only the wave's own prefetch
  // hides the LDS latency: K fragments are read four steps ahead through a
  // 6-entry ring.  work(kk) runs after the instruction of step kk: VALU work
  // of the previous tile's softmax, which then overlaps the matrix core.
  v16f sa, sb;
  auto s_tile = [&](int jt, auto&& work) {
    const char* kt = &tiles[jt % kWideSlots][0];
    constexpr int KD = 4, KR = 6;
    v8bf kr[KR];
    auto kread = [&](int kk) -> v8bf { return *reinterpret_cast<const v8bf*>(kt + 4096 * (kk >> 2) + kb[kk & 3]); };
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) kr[kk] = kread(kk);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk + KD < KK) kr[(kk + KD) % KR] = kread(kk + KD);
      const v8bf k0 = kr[kk % KR];
      if (kk < 2) {
        if (kk == 0) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(sa) : "v"(k0), "v"(qf[kk]));
        else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(sb) : "v"(k0), "v"(qf[kk]));
      } else if (kk + 1 < KK) {
        if (kk & 1) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sb) : "v"(k0), "v"(qf[kk]));
        else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sa) : "v"(k0), "v"(qf[kk]));
      } else {
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 4"
                     : "+v"(sb) : "v"(k0), "v"(qf[kk]));
      }
      work(kk);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Software pipeline over the tiles: iteration j takes S^T of tile j (from
  // the accumulators), computes S^T of tile j+1 on the matrix core while the
  // VALU does the online softmax of tile j in its shadow, then O^T += V^T P^T
  // for tile j.  Iteration j reads tiles j (V) and j+1 (K); tiles j+2 and j+3
  // are in flight, and the gather of tile j+3 goes to the slot of tile j-1,
  // which every wave has finished with at the barrier of iteration j.
#pragma unroll
  for (int j0 = 0; j0 < kWideSlots - 1; ++j0)
    if (j0 < ntiles) gather(j0);
  if (ntiles > 0) {
    if (ntiles > 2) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * NIW) : "memory");
    else if (ntiles > 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(NIW) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();        // tile 0 is in LDS
    s_tile(0, [](int) {});
  }
  for (int j = 0; j < ntiles; ++j) {
    // ---- online softmax of tile j in log2 units (lazily moved reference max,
    // P < 2^8), spread over the k-steps of the next tile's S^T
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = sa[i] + sb[i];
    const uint32_t vm = vmask[j] >> (4 * g);      // bit 8(i/4) + i%4: row of accumulator i
    float mx = -INFINITY, m_use = 0.0f, alpha = 1.0f, psum = 0.0f;
    v8bf pa[2];
    auto softmax = [&](int kk) {
      if (kk < 16) {                // scale and mask one value, running max
        const int i = kk;
        x[i] = ((vm >> (8 * (i >> 2) + (i & 3))) & 1u) ? x[i] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[i]);
      } else if (kk == 16) {        // the head's max over both lane halves; move the reference
        mx = xhalf_max(mx);
        const float m_old = m_run;
        const bool move = mx > m_old + 8.0f;
        const float m_ref = move ? mx : m_old;
        m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;
        alpha = (move && m_old != -INFINITY) ? __builtin_amdgcn_exp2f(m_old - m_ref) : 1.0f;
        m_run = m_ref;
      } else if (kk < 33) {         // one probability, rounded to bf16
        const int i = kk - 17;
        const float pr = __builtin_amdgcn_exp2f(x[i] - m_use);
        psum += pr;
        pa[i >> 3][i & 7] = (__bf16)pr;
      } else if (kk == 33) {
        l_run = l_run * alpha + psum;
      }
    };
    if (j + 1 < ntiles) {
      // wait for tile j+1; tile j+2 may stay in flight
      if (j + 2 < ntiles) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(NIW) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();      // tile j+1 is in LDS; every wave is done with tile j-1
      if (j + kWideSlots - 1 < ntiles) gather(j + kWideSlots - 1);
      s_tile(j + 1, softmax);
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) softmax(kk);
    }
    const char* kt = &tiles[j % kWideSlots][0];

    // ---- rescale O^T where the head's reference moved (lane l holds head l%32
    // only, so the factor is the lane's own).  In place in the accumulation
    // registers, by inline asm so the accumulators never leave them; wait
    // states before (XDL result read by VALU) and after (VALU write read as
    // SrcC) are explicit, the compiler does not see inside the asm.
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float tmp;
        asm volatile(
            "s_nop 7\n\ts_nop 7\n\ts_nop 4\n\t"
            "v_accvgpr_read_b32 %16, %0\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %0, %16\n\t"
            "v_accvgpr_read_b32 %16, %1\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %1, %16\n\t"
            "v_accvgpr_read_b32 %16, %2\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %2, %16\n\t"
            "v_accvgpr_read_b32 %16, %3\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %3, %16\n\t"
            "v_accvgpr_read_b32 %16, %4\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %4, %16\n\t"
            "v_accvgpr_read_b32 %16, %5\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %5, %16\n\t"
            "v_accvgpr_read_b32 %16, %6\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %6, %16\n\t"
            "v_accvgpr_read_b32 %16, %7\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %7, %16\n\t"
            "v_accvgpr_read_b32 %16, %8\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %8, %16\n\t"
            "v_accvgpr_read_b32 %16, %9\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %9, %16\n\t"
            "v_accvgpr_read_b32 %16, %10\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %10, %16\n\t"
            "v_accvgpr_read_b32 %16, %11\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %11, %16\n\t"
            "v_accvgpr_read_b32 %16, %12\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %12, %16\n\t"
            "v_accvgpr_read_b32 %16, %13\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %13, %16\n\t"
            "v_accvgpr_read_b32 %16, %14\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %14, %16\n\t"
            "v_accvgpr_read_b32 %16, %15\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %15, %16\n\t"
            "s_nop 2"
            : "+a"(o[nt][0]), "+a"(o[nt][1]), "+a"(o[nt][2]), "+a"(o[nt][3]), "+a"(o[nt][4]), "+a"(o[nt][5]),
              "+a"(o[nt][6]), "+a"(o[nt][7]), "+a"(o[nt][8]), "+a"(o[nt][9]), "+a"(o[nt][10]), "+a"(o[nt][11]),
              "+a"(o[nt][12]), "+a"(o[nt][13]), "+a"(o[nt][14]), "+a"(o[nt][15]), "=&v"(tmp)
            : "v"(alpha));
      }
    }

    // ---- O^T += V^T P^T for tile j, V read transposed from its tile; steps
    // st = 16u + nt, V fragments four steps ahead through a 6-entry ring
    auto vread = [&](int st) -> v8bf {
      const int nt = st & (NT - 1), u = st / NT;
      const char* p0 = kt + 4096 * (nt >> 1) + 2048 * u;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p0 + vb[0][nt & 1]));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p0 + vb[1][nt & 1]));
      return __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int VD = 4, VR = 6;
    v8bf vr[VR];
#pragma unroll
    for (int st = 0; st < VD; ++st) vr[st] = vread(st);
#pragma unroll
    for (int st = 0; st < 2 * NT; ++st) {
      if (st + VD < 2 * NT) vr[(st + VD) % VR] = vread(st + VD);
      o[st & (NT - 1)] = mfma32(vr[st % VR], pa[st / NT], o[st & (NT - 1)]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- finish: denominator of the lane's head, normalise, write.  Lane l
  // holds dims 32nt + 8q + 4g + i (i < 4) of head h0 + l%32; one permlane32
  // swap per pair of q gives each lane 8 consecutive dims (16 bytes).
  const float l_tot = xhalf_sum(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse_h = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  uint16_t* obase;
  float* lbase;
  if (a.nsplit == 1) {
    obase = a.out + (int64_t)t * a.H * DV;
    lbase = a.lse ? a.lse + (int64_t)t * a.H : nullptr;
  } else {
    const int64_t base = (int64_t)t * a.nsplit + split;
    obase = a.part_o + base * a.H * DV;
    lbase = a.part_lse + base * a.H;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      // X: dims of q = 2pp (lane's 4 at 4g), Y: q = 2pp + 1
      const int qa = 2 * pp, qb = 2 * pp + 1;
      uint32_t x0 = (uint32_t)bf16_bits(o[nt][4 * qa] * inv) | ((uint32_t)bf16_bits(o[nt][4 * qa + 1] * inv) << 16);
      uint32_t x1 = (uint32_t)bf16_bits(o[nt][4 * qa + 2] * inv) | ((uint32_t)bf16_bits(o[nt][4 * qa + 3] * inv) << 16);
      uint32_t y0 = (uint32_t)bf16_bits(o[nt][4 * qb] * inv) | ((uint32_t)bf16_bits(o[nt][4 * qb + 1] * inv) << 16);
      uint32_t y1 = (uint32_t)bf16_bits(o[nt][4 * qb + 2] * inv) | ((uint32_t)bf16_bits(o[nt][4 * qb + 3] * inv) << 16);
      // lanes 32-63 of X <-> lanes 0-31 of Y: the low half ends with q = 2pp
      // (its own dims 0-3 in X, the partner's 4-7 in Y), the high half with q = 2pp+1
      const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
      const v4i v = v4i{(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
      // low half: dims 32nt + 16pp + 0..7 of head n32; high half: 32nt + 16pp + 8..15
      *reinterpret_cast<v4i*>(obase + (int64_t)(h0 + n32) * DV + nt * 32 + 16 * pp + 8 * g) = v;
    }
  }
  if (lbase && g == 0) lbase[h0 + n32] = lse_h;
}

// Merge split partials: lse = log sum_i exp(lse_i); out = sum_i exp(lse_i - lse) O_i.
// One thread per 8 consecutive value dims of one head.  The partials are read
// in groups of kCombineGroup splits whose loads are all issued before any is
// used; the weights are taken relative to the largest split lse and the sum
// is normalised once at the end.

__global__ void __launch_bounds__(256) attn_combine_kernel(CombineArgs a) {
  const int per_head = a.D_v / 8;
  // same XCD-major order as the attention workgroups that wrote the partials
  const int64_t item = (int64_t)xcd_major(blockIdx.x, gridDim.x) * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.T * a.H * per_head;
  if (item >= total) return;
  const int d8 = (int)(item % per_head);
  const int64_t th = item / per_head;          // t * H + h
  const int h = (int)(th % a.H);
  const int t = (int)(th / a.H);
  const float* pl = a.part_lse + (int64_t)t * a.nsplit * a.H + h;
  const uint16_t* po = a.part_o + ((int64_t)t * a.nsplit * a.H + h) * a.D_v + d8 * 8;
  const int64_t po_stride = (int64_t)a.H * a.D_v;
  // one pass: each group's lse values and partials are loaded together; the
  // running reference (largest lse so far) rescales the sums when it moves
  float mx = -INFINITY, den = 0.0f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int g = 0; g < a.nsplit; g += kCombineGroup) {
    float wl[kCombineGroup];
    v4i raw[kCombineGroup];
#pragma unroll
    for (int j = 0; j < kCombineGroup; ++j) {
      const bool v = g + j < a.nsplit;
      wl[j] = v ? pl[(int64_t)(g + j) * a.H] : -INFINITY;
      raw[j] = v ? *reinterpret_cast<const v4i*>(po + (g + j) * po_stride) : v4i{0, 0, 0, 0};
    }
    float gm = mx;
#pragma unroll
    for (int j = 0; j < kCombineGroup; ++j) gm = fmaxf(gm, wl[j]);
    if (gm == -INFINITY) continue;                  // nothing valid yet
    const float sc = __expf(mx - gm);               // 0 while mx is -inf
    den *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= sc;
    mx = gm;
#pragma unroll
    for (int j = 0; j < kCombineGroup; ++j) {
      const float wgt = __expf(wl[j] - mx);
      den += wgt;
      const v8bf pv = __builtin_bit_cast(v8bf, raw[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wgt * (float)pv[e];
    }
  }
  float lse = -INFINITY;
  if (mx != -INFINITY) {
    lse = mx + __logf(den);
    const float inv = 1.0f / den;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
  }
  uint32_t pk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pk[j] = (uint32_t)bf16_bits(acc[2 * j]) | ((uint32_t)bf16_bits(acc[2 * j + 1]) << 16);
  *reinterpret_cast<v4i*>(a.out + th * a.D_v + d8 * 8) = v4i{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
  if (a.lse && d8 == 0) a.lse[th] = lse;
}

// The same merge for NS = 2 or 4 splits: a thread merges 8 / NS items (256
// apart, so each of its passes is one coalesced sweep) and issues the loads of
// all of them before it uses any, which keeps eight 16-byte partial loads in
// flight per thread as the general kernel does at eight splits.  The
// arithmetic per item is the general kernel's, in the same order.
template <int NS>
__global__ void __launch_bounds__(256) attn_combine_few_kernel(CombineArgs a) {
  constexpr int IPT = 8 / NS;
  const int per_head = a.D_v / 8;
  const int64_t total = (int64_t)a.T * a.H * per_head;
  const int64_t base = (int64_t)xcd_major(blockIdx.x, gridDim.x) * (256 * IPT) + threadIdx.x;
  const int64_t po_stride = (int64_t)a.H * a.D_v;
  float wl[IPT][NS];
  v4i raw[IPT][NS];
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int64_t item = base + 256 * i;
    const bool ok = item < total;
    const int64_t it = ok ? item : 0;
    const int d8 = (int)(it % per_head);
    const int64_t th = it / per_head;          // t * H + h
    const int h = (int)(th % a.H);
    const int t = (int)(th / a.H);
    const float* pl = a.part_lse + (int64_t)t * NS * a.H + h;
    const uint16_t* po = a.part_o + ((int64_t)t * NS * a.H + h) * a.D_v + d8 * 8;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      wl[i][j] = ok ? pl[(int64_t)j * a.H] : -INFINITY;
      raw[i][j] = ok ? *reinterpret_cast<const v4i*>(po + j * po_stride) : v4i{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int64_t item = base + 256 * i;
    if (item >= total) break;
    float mx = -INFINITY, den = 0.0f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NS; ++j) mx = fmaxf(mx, wl[i][j]);
    float lse = -INFINITY;
    if (mx != -INFINITY) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const float wgt = __expf(wl[i][j] - mx);
        den += wgt;
        const v8bf pv = __builtin_bit_cast(v8bf, raw[i][j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += wgt * (float)pv[e];
      }
      lse = mx + __logf(den);
      const float inv = 1.0f / den;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= inv;
    }
    uint32_t pk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pk[j] = (uint32_t)bf16_bits(acc[2 * j]) | ((uint32_t)bf16_bits(acc[2 * j + 1]) << 16);
    const int d8 = (int)(item % per_head);
    const int64_t th = item / per_head;
    *reinterpret_cast<v4i*>(a.out + th * a.D_v + d8 * 8) = v4i{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
    if (a.lse && d8 == 0) a.lse[th] = lse;
  }
}

hipError_t launch_attn(const AttnArgs& a, int D, int D_v, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)a.g.num_rows * a.nsplit));
  const bool sepv = a.v.data != nullptr;
  if (attn_uses_wide(a.H, D, D_v, sepv, a.per_split)) {
    hipLaunchKernelGGL(attn_wide_kernel, grid, dim3(64 * kWideWaves), 0, stream, a);
  } else if (D == 576 && D_v == 512 && !sepv) {
    const dim3 block(64 * ((a.H + 15) / 16));          // 16 heads per wave
    hipLaunchKernelGGL((attn_kernel<576, 512, false, 1>), grid, block, 0, stream, a);
  } else if (D == 64 && D_v == 64) {
    const dim3 block(64 * ((a.H + 15) / 16));          // 16 heads per wave
    if (sepv) hipLaunchKernelGGL((attn_kernel<64, 64, true, 1>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_kernel<64, 64, false, 1>), grid, block, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const int64_t items = (int64_t)a.T * a.H * (a.D_v / 8);
  if (a.nsplit == 2) {
    hipLaunchKernelGGL(attn_combine_few_kernel<2>, dim3((unsigned)((items + 1023) / 1024)), dim3(256), 0, stream, a);
  } else if (a.nsplit == 4) {
    hipLaunchKernelGGL(attn_combine_few_kernel<4>, dim3((unsigned)((items + 511) / 512)), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

bool attn_uses_wide(int H, int D, int D_v, bool sepv, int per_split) {
  return D == 576 && D_v == 512 && !sepv && H == 32 * kWideWaves && per_split <= kAttnMaxSplit;
}

}  // namespace dsa
