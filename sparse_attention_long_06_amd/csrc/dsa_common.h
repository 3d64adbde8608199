// Shared device helpers of the DSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// Top-k radix: the first pass bins the high 11 bits of the order key.
constexpr int kBins1Bits = 11;
constexpr int kBins1 = 1 << kBins1Bits;

// Batch geometry as the kernels see it (device pointers, plain values).
struct Geo {
  const int32_t* seq_lens;
  const int32_t* q_start;      // nullptr: one query row per sequence at position len-1
  const int32_t* block_table;  // nullptr: contiguous caches
  int32_t max_blocks;
  int32_t block_shift;         // log2(block_size) when paged
  int32_t num_seqs;
  int32_t num_rows;
};

struct Cache {
  const char* data;
  int64_t row_stride;  // bytes
  int64_t seq_stride;  // rows (contiguous caches)
};

// Token row of logical token s of sequence b.
__device__ __forceinline__ int64_t token_row(const Geo& g, const Cache& c, int b, int s) {
  if (g.block_table) {
    const int blk = g.block_table[(int64_t)b * g.max_blocks + (s >> g.block_shift)];
    return ((int64_t)blk << g.block_shift) + (s & ((1 << g.block_shift) - 1));
  }
  return (int64_t)b * c.seq_stride + s;
}

__device__ __forceinline__ const char* token_ptr(const Geo& g, const Cache& c, int b, int s) {
  return c.data + token_row(g, c, b, s) * c.row_stride;
}

// Sequence and position of query row t.
__device__ __forceinline__ void row_seq_pos(const Geo& g, int t, int& b, int& pos) {
  if (!g.q_start) {
    b = t;
    pos = g.seq_lens[t] - 1;
    return;
  }
  int lo = 0, hi = g.num_seqs - 1;  // largest b with q_start[b] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (g.q_start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  b = lo;
  const int nq = g.q_start[b + 1] - g.q_start[b];
  pos = g.seq_lens[b] - nq + (t - g.q_start[b]);
}

// Order-preserving fp32 -> uint32 map: a larger score gives a larger key and
// -0.0 maps to the key of +0.0, so the two tie.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The score of an order-preserving key (the inverse of score_key).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Exclusive scan of one uint32 per thread over a block of NT threads.
// `tmp` holds NT/64 words of LDS.  Returns the exclusive prefix; `total`
// receives the block total.  Contains two barriers.
// Workgroup barrier that orders LDS only.  __syncthreads() also makes every
// wave wait for its outstanding global stores and atomics; where the barrier
// only publishes LDS data, that wait is pure latency.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves only (no
// LDS traffic): Hillis-Steele inside each 16-lane row by row shifts, then the
// row totals carried across rows by the row_bcast:15 / row_bcast:31 forms.
// A lane whose DPP source falls outside its row, or whose row is masked off,
// adds the `old` operand, 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* tmp, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) tmp[wid] = x;
  lds_barrier();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t s = tmp[w];
    before += (w < wid) ? s : 0u;
    tot += s;
  }
  lds_barrier();
  total = tot;
  return before + x - v;
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(uint16_t, h);
}

}  // namespace dsa
