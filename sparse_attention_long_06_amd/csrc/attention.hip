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

// Merge split partials: lse = log sum_i exp(lse_i); out = sum_i exp(lse_i - lse) O_i.
// One thread per 8 consecutive value dims of one head.  The partials are read
// in groups of kCombineGroup splits whose loads are all issued before any is
// used; the weights are taken relative to the largest split lse and the sum
// is normalised once at the end.
constexpr int kCombineGroup = 8;

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

hipError_t launch_attn(const AttnArgs& a, int D, int D_v, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)a.g.num_rows * a.nsplit));
  const bool sepv = a.v.data != nullptr;
  if (D == 576 && D_v == 512 && !sepv) {
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
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
