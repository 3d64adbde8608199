// Lightning-indexer warm-up objective on gfx950, forward and backward
// (tenelement.pl article "DeepSeek V3.2-Exp Cuts Long-Context Costs with
// DeepSeek Sparse Attention (DSA) While Maintaining Benchmark Parity",
// section "Proces Treningu DSA: Od Warm-up do Sparsity": with the main model
// frozen, the indexer is fitted by a KL divergence to the dense attention
// distribution summed over the heads).  For query row t at position p:
//
//   a[s]  = (1/H) sum_h softmax_s(scale * q[t,h] . K[s])      (s <= p)
//   P[s]  = softmax_s(I[t,s])                                  (indexer scores)
//   loss  = sum_s a[s] (log a[s] - log P[s])
//   dI[s] = P[s] - a[s]
//   dw[j] = q_scale sum_s dI[s] k_scale[s] ReLU(z[j,s])         z = q8[j] . k8[s]
//   dq[j] = w[j] sum_s dI[s] k_scale[s] [z[j,s] > 0] k8[s]      (w.r.t. q_scale*q8)
//   dk[s] = sum_t dI_t[s] sum_j w_t[j] q_scale_t [z_t[j,s] > 0] q8_t[j]   (w.r.t. k_scale*k8)
//
// Launch sequence (after the main path's prefill indexer wrote I):
//   warm_attn_kernel<0>  per row and head (two adjacent rows of a sequence per
//                        workgroup), the log2-sum-exp2 of the scaled
//                        dense logits over the row's prefix (S = q K^T; each
//                        lane reduces its keys online, lanes combine at the end);
//   warm_attn_kernel<1>  recomputes the same logits with the same instructions,
//                        sums exp2(x - lse) over heads in-lane and across lane
//                        groups and waves, and turns each key into a, P, the
//                        KL term and dI (written over I); the row's loss is
//                        reduced in a fixed order;
//   warm_dq_kernel       per row: z recomputed on MFMA from widened FP8
//                        (exact products), dw in VALU, dq = C K8 on MFMA with
//                        C = dI k_scale [z > 0] split into bf16 hi + lo parts
//                        (about 2^-17 relative) and K8 read transposed from
//                        the bf16 key tile by ds_read_b64_tr_b16;
//   warm_dk_kernel       per (key tile of 32, chunk of rows): dk partial =
//                        C'^T Q8 with the same hi/lo split, Q8 staged as bf16
//                        and read transposed; warm_dk_reduce_kernel adds the
//                        chunk partials in a fixed order (no float atomics).
//
// MFMA operand layouts (v_mfma_f32_16x16x32_bf16): lane l holds A[l%16][8(l/16)..+7]
// and B[8(l/16)..+7][l%16]; the result D[4(l/16)+i][l%16], i < 4.  When an
// MFMA result feeds the next MFMA as its 32-wide contraction operand, slot j
// of lane group g stands for index 4g+j (j < 4, first 16-tile) or 16+4g+j-4
// (second tile); the other operand is read with that same order.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {
namespace {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ v8bf widen8(int lo, int hi) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ v4f mfma(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Sum over the four 16-lane groups of a wave; every lane gets its column's total.
__device__ __forceinline__ float wsum4(float x) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// hi + lo bf16 split of fp32 values: hi = RNE(x), lo = RNE(x - hi).
__device__ __forceinline__ void split8(const float (&x)[8], v8bf& hi, v8bf& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 h = (__bf16)x[j];
    hi[j] = h;
    lo[j] = (__bf16)(x[j] - (float)h);
  }
}

// ---------------------------------------------------------------- dense pass
// One workgroup per query row, H/16 waves of 16 heads; the row's prefix is
// streamed in 64-key blocks through a double-buffered LDS tile filled by DMA
// (16-byte chunk c of key r at chunk position c ^ ((r >> 1) & 7)).
constexpr int kWD = 576;
constexpr int kWCH = kWD / 8;       // 16-byte chunks per latent row
constexpr int kWKK = kWD / 32;      // MFMA K-steps over the latent row
constexpr int kWRB = 64;            // keys per block
constexpr int kWTile = kWRB * kWCH * 16;

__device__ __forceinline__ int wswz(int r) { return (r >> 1) & 7; }

// Pairs of adjacent query rows of one sequence: pair_start[b] = sum over
// earlier sequences of ceil(nq / 2).  One workgroup, any number of sequences.
__global__ void __launch_bounds__(256) warm_pairs_kernel(WarmArgs a) {
  __shared__ uint32_t tmp[4];
  uint32_t carry = 0;
  for (int b0 = 0; b0 < a.g.num_seqs; b0 += 256) {
    const int bb = b0 + (int)threadIdx.x;
    const uint32_t c = bb < a.g.num_seqs ? (uint32_t)((a.g.q_start[bb + 1] - a.g.q_start[bb] + 1) >> 1) : 0u;
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<256>(c, tmp, tot);
    if (bb < a.g.num_seqs) a.pair_start[bb] = (int)(carry + ex);
    carry += tot;
  }
  if (threadIdx.x == 0) a.pair_start[a.g.num_seqs] = (int)carry;
}

// One workgroup per pair of adjacent query rows of a sequence (the last row of
// a sequence with an odd row count is alone), H/16 waves of 16 heads.  The
// longer row's prefix is streamed in 64-key blocks through a double-buffered
// LDS tile filled by DMA (16-byte chunk c of key r at chunk position
// c ^ ((r >> 1) & 7)); each K fragment read from the tile feeds the MFMAs of
// both rows, and the shorter row masks the one key past its position.
template <int MODE>
__global__ void __launch_bounds__(512) warm_attn_kernel(WarmArgs a) {
  __shared__ __attribute__((aligned(16))) char ktile[2][kWTile];
  __shared__ float hsum[2][8][kWRB];
  __shared__ float red[2][2][8];

  const int waves = blockDim.x >> 6;
  const int npairs = a.pair_start[a.g.num_seqs];
  if ((int)blockIdx.x >= npairs) return;                 // uniform
  const int g = npairs - 1 - (int)blockIdx.x;            // long rows first
  int b;
  {
    int lo = 0, hi = a.g.num_seqs - 1;                   // last sequence with pair_start <= g
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.pair_start[mid] <= g) lo = mid; else hi = mid - 1;
    }
    b = lo;
  }
  const int nq = a.g.q_start[b + 1] - a.g.q_start[b];
  const int i0 = 2 * (g - a.pair_start[b]);
  const int tA = a.g.q_start[b] + i0;
  const bool two = i0 + 1 < nq;                          // uniform
  const int posA = a.g.seq_lens[b] - nq + i0;
  const int n = posA + 1 + (two ? 1 : 0);                // keys of the longer row
  const int tr[2] = {tA, tA + 1};
  const int npos[2] = {posA + 1, posA + 2};              // keys each row sees
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nl = lane & 15, grp = lane >> 4;
  const int nblk = (n + kWRB - 1) / kWRB;
  const int64_t row_base = (int64_t)b * a.kv.seq_stride;

  // q fragments of both rows: head 16*wave + nl, dims 32*kk + 8*grp .. +7
  v8bf qf[2][kWKK];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint16_t* qrow = a.q + ((int64_t)(two ? tr[r] : tA) * a.H + wave * 16 + nl) * kWD;
#pragma unroll
    for (int kk = 0; kk < kWKK; ++kk)
      qf[r][kk] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(qrow + kk * 32 + grp * 8));
  }

  auto issue = [&](int blk) {
    char* tile = ktile[blk & 1];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)tile;
    constexpr int NI = kWRB * kWCH / 64;
    for (int ins = wave; ins < NI; ins += waves) {
      const int p = ins * 64 + lane;
      const int r = p / kWCH, pc = p % kWCH;
      const int s = min(blk * kWRB + r, n - 1);        // keys past the prefix re-read its last key
      const char* src = a.kv.data + (row_base + s) * a.kv.row_stride + (pc ^ wswz(r)) * 16;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds0 + ins * 64 * 16);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" :: "s"(m0), "v"(src) : "memory");
    }
  };

  // LDS bases of this lane's K fragment reads (key 16*mt + nl, logical chunk 4*kk + grp)
  const int yk = wswz(nl);
  const int kb0 = (nl * kWCH + ((0 + grp) ^ yk)) * 16;
  const int kb1 = (nl * kWCH + ((4 + grp) ^ yk)) * 16;

  // MODE 0: per lane and row, heads 16*wave + 4*grp + i over keys 16*mt + nl of
  // every block: online (max, sum) in log2 units, combined across the 16 lanes at the end
  float m_run[2][4], l_run[2][4];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m_run[r][i] = -INFINITY;
      l_run[r][i] = 0.0f;
    }
  // MODE 1: per row, the heads' log2-sum-exp2, the indexer score maximum and
  // log2-sum-exp2 relative to it, and (in wave r, for row r) the KL sum
  float L[2][4];
  float mI[2] = {0.f, 0.f}, lseI2[2] = {0.f, 0.f};
  float kl[2] = {0.f, 0.f};
  const int nrows = two ? 2 : 1;
  if constexpr (MODE == 1) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        L[r][i] = (r == 0 || two) ? a.lse2[(int64_t)tr[r] * a.H + wave * 16 + grp * 4 + i] : 0.0f;
    // softmax of the scores taken relative to their maximum: I - max is exact
    // near the top, so P keeps fp32 relative accuracy however large I is
    for (int r = 0; r < (two ? 2 : 1); ++r) {
      const float* srow = a.scores + (int64_t)tr[r] * a.ld;
      float m = -INFINITY;
      for (int s = threadIdx.x; s < npos[r]; s += blockDim.x) m = fmaxf(m, srow[s]);
      m = wave_max(m);
      if (lane == 0) red[r][0][wave] = m;
      __syncthreads();
      float mm = red[r][0][0];
      for (int w = 1; w < waves; ++w) mm = fmaxf(mm, red[r][0][w]);
      float l = 0.0f;
      for (int s = threadIdx.x; s < npos[r]; s += blockDim.x) l += __builtin_amdgcn_exp2f(__fmul_rn(srow[s] - mm, kLog2e));
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) l += __shfl_xor(l, o);
      if (lane == 0) red[r][1][wave] = l;
      __syncthreads();
      float ll = 0.0f;
      for (int w = 0; w < waves; ++w) ll += red[r][1][w];
      mI[r] = mm;
      lseI2[r] = __builtin_amdgcn_logf(ll);
    }
  }

  issue(0);
  for (int blk = 0; blk < nblk; ++blk) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (blk + 1 < nblk) issue(blk + 1);
    const char* kt = ktile[blk & 1];

    // S = q K^T for both rows, D[head][key]; both passes run this same
    // instruction sequence, so they see bit-identical logits
    v4f s[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) s[r][mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kWKK; ++kk) {
      v8bf kf[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        kf[mt] = *reinterpret_cast<const v8bf*>(kt + ((kk & 1) ? kb1 : kb0) + (kk >> 1) * 128 + mt * 16 * kWCH * 16);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) s[0][mt] = mfma(qf[0][kk], kf[mt], s[0][mt]);
      if (two) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) s[1][mt] = mfma(qf[1][kk], kf[mt], s[1][mt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    if constexpr (MODE == 0) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x[4];
          float mx = -INFINITY;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            const int key = blk * kWRB + mt * 16 + nl;
            x[mt] = key < npos[r] ? __fmul_rn(s[r][mt][i], a.scale_log2) : -INFINITY;
            mx = fmaxf(mx, x[mt]);
          }
          const float m_new = fmaxf(m_run[r][i], mx);
          const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
          float acc = l_run[r][i] * __builtin_amdgcn_exp2f(m_run[r][i] - m_use);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) acc += __builtin_amdgcn_exp2f(x[mt] - m_use);
          l_run[r][i] = acc;
          m_run[r][i] = m_new;
        }
      }
    } else {
      // sum over this wave's 16 heads of exp2(x - lse): in-lane over i, then over lane groups
#pragma unroll
      for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          float e = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) e += __builtin_amdgcn_exp2f(__fmul_rn(s[r][mt][i], a.scale_log2) - L[r][i]);
          e = wsum4(e);
          if (grp == 0) hsum[r][wave][mt * 16 + nl] = e;
        }
      }
      lds_barrier();
      for (int r = wave; r < nrows; r += waves) {       // wave r turns row r's keys into a, P, KL and dI
        const int key = blk * kWRB + lane;
        if (key < npos[r]) {
          float hs = 0.0f;
          for (int w = 0; w < waves; ++w) hs += hsum[r][w][lane];
          float* srow = a.scores + (int64_t)tr[r] * a.ld;
          const float at = hs * a.inv_H;                          // target probability
          const float lp = __fmul_rn(srow[key] - mI[r], kLog2e) - lseI2[r];    // log2 P
          const float pm = __builtin_amdgcn_exp2f(lp);
          srow[key] = pm - at;                                    // dI, written over the score
          if (at > 0.0f) kl[r] += at * (__builtin_amdgcn_logf(at) - lp);
        }
      }
    }
  }

  if constexpr (MODE == 0) {
    // combine the 16 lanes of the group that hold heads 4*grp + i
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = m_run[r][i], l = l_run[r][i];
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const float m2 = __shfl_xor(m, o), l2 = __shfl_xor(l, o);
          const float mm = fmaxf(m, m2);
          const float a1 = (m == -INFINITY) ? 0.0f : l * __builtin_amdgcn_exp2f(m - mm);
          const float a2 = (m2 == -INFINITY) ? 0.0f : l2 * __builtin_amdgcn_exp2f(m2 - mm);
          m = mm;
          l = a1 + a2;
        }
        if (nl == 0 && (r == 0 || two))
          a.lse2[(int64_t)tr[r] * a.H + wave * 16 + grp * 4 + i] = m + __builtin_amdgcn_logf(l);
      }
    }
  } else {
    for (int r = wave; r < nrows; r += waves) {
      float v = kl[r];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
      if (lane == 0) a.loss[tr[r]] = v * kLn2;
    }
  }
}

// ---------------------------------------------------------------- dq, dw
// One workgroup per query row, H_I/16 waves (wave w: indexer heads 16w..16w+15).
// 32-key steps: the key tile is widened to bf16 into LDS (16-byte chunk c of
// key r at chunk position c ^ (r & 7)) together with g = dI * k_scale.
constexpr int kBK = 32;             // keys per backward step
constexpr int kBRow = 256;          // bf16 bytes per key row (d_I = 128)

__device__ __forceinline__ int bswz(int r) { return r & 7; }

__global__ void __launch_bounds__(256) warm_dq_kernel(WarmArgs a) {
  __shared__ __attribute__((aligned(16))) char ktile[kBK * kBRow];
  __shared__ __attribute__((aligned(16))) float gk[kBK];

  const int t = a.g.num_rows - 1 - (int)blockIdx.x;
  const int nthr = blockDim.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nl = lane & 15, grp = lane >> 4;
  int b, pos;
  row_seq_pos(a.g, t, b, pos);
  const int n = pos + 1;
  const int nsteps = (n + kBK - 1) / kBK;
  const int64_t krow0 = (int64_t)b * a.kidx.seq_stride;
  const float* grow = a.scores + (int64_t)t * a.ld;

  // B operand of z^T = K q^T: head 16*wave + nl, dims 32*grp + 8*c .. +7
  v8bf qb[4];
  {
    const v4i* p = reinterpret_cast<const v4i*>(a.q8 + ((int64_t)t * a.H_I + wave * 16 + nl) * 128 + 32 * grp);
    const v4i lo = p[0], hi = p[1];
    qb[0] = widen8(lo.x, lo.y);
    qb[1] = widen8(lo.z, lo.w);
    qb[2] = widen8(hi.x, hi.y);
    qb[3] = widen8(hi.z, hi.w);
  }

  // staging: item i (0..255) = key i >> 3, fp8 bytes 16*(i & 7) .. +15
  v4i raw[2];
  float graw = 0.0f;
  auto fetch = [&](int step) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = threadIdx.x + u * nthr;
      if (i < 256) {
        const int s = min(step * kBK + (i >> 3), n - 1);
        raw[u] = *reinterpret_cast<const v4i*>(a.kidx.data + (krow0 + s) * a.kidx.row_stride + 16 * (i & 7));
      }
    }
    if (threadIdx.x < kBK) {
      const int s = step * kBK + threadIdx.x;
      float g = 0.0f;
      if (s < n) {
        const float ks = a.ksc.data ? *reinterpret_cast<const float*>(a.ksc.data + (krow0 + s) * a.ksc.row_stride) : 1.0f;
        g = grow[s] * ks;
      }
      graw = g;
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = threadIdx.x + u * nthr;
      if (i < 256) {
        const int r = i >> 3, c0 = 2 * (i & 7);
        const v8bf w0 = widen8(raw[u].x, raw[u].y), w1 = widen8(raw[u].z, raw[u].w);
        *reinterpret_cast<v8bf*>(ktile + r * kBRow + ((c0 ^ bswz(r)) << 4)) = w0;
        *reinterpret_cast<v8bf*>(ktile + r * kBRow + (((c0 + 1) ^ bswz(r)) << 4)) = w1;
      }
    }
    if (threadIdx.x < kBK) gk[threadIdx.x] = graw;
  };

  // LDS offsets: A operand of z^T (key 16*mt + nl, logical chunk 4*grp + c) and the
  // transposed reads of dq's B operand (key row R + (nl >> 2) with R = 4*grp or
  // 16 + 4*grp, dims 16*dt + 4*(nl & 3) .. +3: logical chunk 2*dt + ((nl & 3) >> 1), +8 bytes for odd nl).
  int zoff[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int r = mt * 16 + nl;
      zoff[mt][c] = r * kBRow + (((4 * grp + c) ^ bswz(r)) << 4);
    }
  const int rlo = 4 * grp + (nl >> 2), rhi = 16 + 4 * grp + (nl >> 2);

  v4f dq[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) dq[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  float dwacc = 0.0f;

  fetch(0);
  for (int step = 0; step < nsteps; ++step) {
    lds_barrier();                      // the previous step's reads are done
    stage();
    if (step + 1 < nsteps) fetch(step + 1);
    lds_barrier();

    v4f z[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      z[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) z[mt] = mfma(*reinterpret_cast<const v8bf*>(ktile + zoff[mt][c]), qb[c], z[mt]);
    }
    // lane: head 16*wave + nl, keys 16*mt + 4*grp + i
    float cv[8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const float4 g4 = *reinterpret_cast<const float4*>(gk + mt * 16 + 4 * grp);
      const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float zz = z[mt][i];
        cv[mt * 4 + i] = zz > 0.0f ? gg[i] : 0.0f;
        dwacc += zz > 0.0f ? gg[i] * zz : 0.0f;
      }
    }
    v8bf chi, clo;
    split8(cv, chi, clo);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int cpos = 2 * dt + ((nl & 3) >> 1);
      const int boff = (nl & 1) * 8;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4s*)(ktile + rlo * kBRow + ((cpos ^ bswz(rlo)) << 4) + boff));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4s*)(ktile + rhi * kBRow + ((cpos ^ bswz(rhi)) << 4) + boff));
      const v8bf kt = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      dq[dt] = mfma(chi, kt, dq[dt]);
      dq[dt] = mfma(clo, kt, dq[dt]);
    }
  }

  const float qs = a.q_scale ? a.q_scale[t] : 1.0f;
  dwacc = wsum4(dwacc);
  if (a.dw && grp == 0) a.dw[(int64_t)t * a.H_I + wave * 16 + nl] = qs * dwacc;
  if (a.dq) {
    // lane: heads 16*wave + 4*grp + i, dim 16*dt + nl
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = wave * 16 + 4 * grp + i;
      const float wj = a.w[(int64_t)t * a.H_I + j];
      float* dst = a.dq + ((int64_t)t * a.H_I + j) * 128 + nl;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) dst[16 * dt] = wj * dq[dt][i];
    }
  }
}

// ---------------------------------------------------------------- dk
// Workgroup = (key tile of 32, chunk of rows, sequence), 4 waves.  With
// HP = H_I/32 head pairs, a step covers 4/HP rows: wave w takes row w / HP
// of the step and head pair w % HP.  Each step stages the rows' q8 (bf16,
// 16-byte chunk c of head row r at c ^ (r & 7)), their dI over the key tile
// and w * q_scale.
template <int HP>
__global__ void __launch_bounds__(256) warm_dk_kernel(WarmArgs a) {
  constexpr int RPS = 4 / HP;                 // rows per step
  constexpr int HI = 32 * HP;                 // indexer heads
  __shared__ __attribute__((aligned(16))) char qtile[RPS * HI * kBRow];   // 32 KB
  __shared__ __attribute__((aligned(16))) float gt[RPS][kBK];
  __shared__ __attribute__((aligned(16))) float wt[RPS][HI];
  __shared__ __attribute__((aligned(16))) float dkred[kBK * 128];          // 16 KB

  const int tile = blockIdx.x, chunk = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nl = lane & 15, grp = lane >> 4;
  const int s0 = tile * kBK;
  const int len = a.g.seq_lens[b];
  const int r0 = a.g.q_start[b];
  const int nq = a.g.q_start[b + 1] - r0;
  const int base = len - nq;                  // position of the sequence's first query row
  const int ibeg = max(chunk * a.row_chunk, max(s0 - base, 0));
  const int iend = min((chunk + 1) * a.row_chunk, nq);
  float* part = a.dk_part + (((int64_t)chunk * a.g.num_seqs + b) * a.max_len + s0) * 128;
  const int kvalid = min(kBK, a.max_len - s0);    // rows of this tile inside the output

  if (s0 >= len || ibeg >= iend) {
    for (int i = threadIdx.x; i < kvalid * 32; i += 256)
      reinterpret_cast<float4*>(part)[i] = float4{0.f, 0.f, 0.f, 0.f};
    return;
  }

  // B operand of z = Q K^T: key s0 + 16*mt + nl (clamped into the sequence), dims 32*grp + 8*c
  v8bf kb[2][4];
  const int64_t krow0 = (int64_t)b * a.kidx.seq_stride;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int s = min(s0 + mt * 16 + nl, len - 1);
    const v4i* p = reinterpret_cast<const v4i*>(a.kidx.data + (krow0 + s) * a.kidx.row_stride + 32 * grp);
    const v4i lo = p[0], hi = p[1];
    kb[mt][0] = widen8(lo.x, lo.y);
    kb[mt][1] = widen8(lo.z, lo.w);
    kb[mt][2] = widen8(hi.x, hi.y);
    kb[mt][3] = widen8(hi.z, hi.w);
  }

  const int ro = wave / HP, hp = wave % HP;
  // LDS offsets inside the wave's (row, head pair) block of qtile:
  //   A operand of z (head 16*ht + nl of the pair, logical chunk 4*grp + c);
  //   transposed B reads of dk (head rows R + (nl >> 2), R = 4*grp or 16 + 4*grp).
  const int qblk = (ro * HI + hp * 32) * kBRow;
  int aoff[2][4];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int r = ht * 16 + nl;                 // head row inside the pair; swizzle uses the row in qtile
      const int rr = hp * 32 + r;
      aoff[ht][c] = qblk + r * kBRow + (((4 * grp + c) ^ bswz(rr)) << 4);
    }
  const int hlo = 4 * grp + (nl >> 2), hhi = 16 + 4 * grp + (nl >> 2);

  v4f dk[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) dk[mt][dt] = v4f{0.f, 0.f, 0.f, 0.f};

  // The next step's q8 rows, dI over the key tile and w * q_scale are loaded
  // into registers while the current step computes (the loads' latency would
  // otherwise open every step), then widened into LDS at the top of the next.
  constexpr int QI = RPS * HI * 8 / 256;      // 16-byte q8 chunks per thread per step
  static_assert(RPS * HI * 8 == QI * 256 && RPS * kBK <= 256 && RPS * HI <= 256, "staging split");
  v4i qpre[QI];
  float gpre = 0.0f, wpre = 0.0f;
  auto load_step = [&](int i0) {
#pragma unroll
    for (int u = 0; u < QI; ++u) {
      const int it = u * 256 + (int)threadIdx.x;
      const int rr = it / (HI * 8), rem = it % (HI * 8);
      const int h = rem >> 3, c8 = rem & 7;     // head, 16-byte fp8 chunk
      const int i = min(i0 + rr, iend - 1);
      qpre[u] = *reinterpret_cast<const v4i*>(a.q8 + ((int64_t)(r0 + i) * a.H_I + h) * 128 + 16 * c8);
    }
    if ((int)threadIdx.x < RPS * kBK) {
      const int rr = threadIdx.x / kBK, kk = threadIdx.x % kBK;
      const int i = i0 + rr;
      const int s = s0 + kk;
      gpre = (i < iend && s <= base + i) ? a.scores[(int64_t)(r0 + i) * a.ld + s] : 0.0f;
    }
    if ((int)threadIdx.x < RPS * HI) {
      const int rr = threadIdx.x / HI, h = threadIdx.x % HI;
      const int i = min(i0 + rr, iend - 1);
      const float qs = a.q_scale ? a.q_scale[r0 + i] : 1.0f;
      wpre = a.w[(int64_t)(r0 + i) * a.H_I + h] * qs;
    }
  };
  load_step(ibeg);

  for (int i0 = ibeg; i0 < iend; i0 += RPS) {
    lds_barrier();                              // every wave is done with the previous step's tiles
    // stage q8 rows (bf16), dI over the key tile, w * q_scale
#pragma unroll
    for (int u = 0; u < QI; ++u) {
      const int it = u * 256 + (int)threadIdx.x;
      const int rr = it / (HI * 8), rem = it % (HI * 8);
      const int h = rem >> 3, c8 = rem & 7;
      const int row = rr * HI + h;
      char* dst = qtile + row * kBRow;
      const v4i v = qpre[u];
      *reinterpret_cast<v8bf*>(dst + (((2 * c8) ^ bswz(h)) << 4)) = widen8(v.x, v.y);
      *reinterpret_cast<v8bf*>(dst + (((2 * c8 + 1) ^ bswz(h)) << 4)) = widen8(v.z, v.w);
    }
    if ((int)threadIdx.x < RPS * kBK) gt[threadIdx.x / kBK][threadIdx.x % kBK] = gpre;
    if ((int)threadIdx.x < RPS * HI) wt[threadIdx.x / HI][threadIdx.x % HI] = wpre;
    lds_barrier();
    if (i0 + RPS < iend) load_step(i0 + RPS);
    if (i0 + ro >= iend) continue;              // this wave's row is past the chunk (uniform per wave)

    // z[ht][mt]: heads 16*ht + 4*grp + i of the pair, key 16*mt + nl
    v4f z[2][2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        z[ht][mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          z[ht][mt] = mfma(*reinterpret_cast<const v8bf*>(qtile + aoff[ht][c]), kb[mt][c], z[ht][mt]);
      }
    // A operand of dk (key 16*mt + nl, heads 4*grp + j (j < 4) and 16 + 4*grp + j - 4)
    v8bf chi[2], clo[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const float g = gt[ro][mt * 16 + nl];
      float cv[8];
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const float4 w4 = *reinterpret_cast<const float4*>(&wt[ro][hp * 32 + ht * 16 + 4 * grp]);
        const float ww[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) cv[ht * 4 + i] = z[ht][mt][i] > 0.0f ? g * ww[i] : 0.0f;
      }
      split8(cv, chi[mt], clo[mt]);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int cpos = 2 * dt + ((nl & 3) >> 1);
      const int boff = (nl & 1) * 8;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4s*)(qtile + qblk + hlo * kBRow + ((cpos ^ bswz(hp * 32 + hlo)) << 4) + boff));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4s*)(qtile + qblk + hhi * kBRow + ((cpos ^ bswz(hp * 32 + hhi)) << 4) + boff));
      const v8bf qt = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        dk[mt][dt] = mfma(chi[mt], qt, dk[mt][dt]);
        dk[mt][dt] = mfma(clo[mt], qt, dk[mt][dt]);
      }
    }
  }

  // reduce the four waves' partials in wave order; lane holds key 16*mt + 4*grp + i, dim 16*dt + nl
  for (int w = 0; w < 4; ++w) {
    lds_barrier();
    if (wave == w) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float* d = &dkred[(mt * 16 + 4 * grp + i) * 128 + 16 * dt + nl];
            *d = (w == 0 ? 0.0f : *d) + dk[mt][dt][i];
          }
    }
  }
  lds_barrier();
  for (int i = threadIdx.x; i < kvalid * 32; i += 256)
    reinterpret_cast<float4*>(part)[i] = reinterpret_cast<const float4*>(dkred)[i];
}

__global__ void __launch_bounds__(256) warm_dk_reduce_kernel(WarmArgs a) {
  const int64_t per_chunk = (int64_t)a.g.num_seqs * a.max_len * 32;    // float4 per chunk
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= per_chunk) return;
  float4 acc = reinterpret_cast<const float4*>(a.dk_part)[i];
  for (int c = 1; c < a.nchunk; ++c) {
    const float4 v = reinterpret_cast<const float4*>(a.dk_part)[c * per_chunk + i];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  reinterpret_cast<float4*>(a.dk)[i] = acc;
}

}  // namespace

hipError_t launch_warmup(const WarmArgs& a, int stage, hipStream_t s) {
  const int T = a.g.num_rows;
  const dim3 blk_attn(64 * (a.H / 16));
  switch (stage) {
    case 0:
      if (T > 0) {
        hipLaunchKernelGGL(warm_pairs_kernel, dim3(1), dim3(256), 0, s, a);
        hipLaunchKernelGGL(warm_attn_kernel<0>, dim3((T + a.g.num_seqs + 1) / 2), blk_attn, 0, s, a);
      }
      break;
    case 1:
      if (T > 0) hipLaunchKernelGGL(warm_attn_kernel<1>, dim3((T + a.g.num_seqs + 1) / 2), blk_attn, 0, s, a);
      break;
    case 2:
      if (T > 0 && (a.dq || a.dw)) hipLaunchKernelGGL(warm_dq_kernel, dim3(T), dim3(64 * (a.H_I / 16)), 0, s, a);
      break;
    case 3:
      if (a.dk) {
        const dim3 grid((a.max_len + kBK - 1) / kBK, a.nchunk, a.g.num_seqs);
        if (a.H_I == 64) hipLaunchKernelGGL(warm_dk_kernel<2>, grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL(warm_dk_kernel<1>, grid, dim3(256), 0, s, a);
        const int64_t n4 = (int64_t)a.g.num_seqs * a.max_len * 32;
        hipLaunchKernelGGL(warm_dk_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, a);
      }
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dsa
