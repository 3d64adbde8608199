// Attainable-peak probes on gfx950 (declared in include/dsa_probes.h): a
// streaming read through the same DMA-to-LDS path the decode indexer uses,
// and a matrix-core issue loop for the two bf16 MFMA forms of the kernels.
// They are the "microbenchmarked attainable peak" references of the
// measurements; they compute nothing of the method.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa_probes.h"

namespace {

constexpr int kTile = 2048;          // bytes per tile: two 1 KiB DMA instructions
constexpr int kRing = 8;             // LDS slots per wave
constexpr int kChunkTiles = 256;     // tiles per workgroup (512 KiB)

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Workgroup g owns tiles [g*kChunkTiles, ...); wave w takes tiles w, w+4, ...
// and streams them through its kRing-slot ring: kRing-1 tiles in flight, the
// oldest awaited with s_waitcnt vmcnt (operations complete in issue order).
__global__ void __launch_bounds__(256) stream_read_kernel(const char* __restrict__ p, int64_t ntiles,
                                                          uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) char ring[4][kRing][kTile];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t t0 = (int64_t)blockIdx.x * kChunkTiles;
  const int64_t t1 = t0 + kChunkTiles < ntiles ? t0 + kChunkTiles : ntiles;
  const int mine = t1 - t0 > wave ? (int)((t1 - t0 - wave + 3) / 4) : 0;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&ring[wave][0][0];
  const uint32_t off0 = 16u * lane, off1 = 1024u + 16u * lane;
  auto issue = [&](int m) {
    const char* base = p + (t0 + wave + 4 * (int64_t)m) * kTile;
    const uint32_t slot = ring_lds + (uint32_t)((m % kRing) * kTile);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :: "s"(slot), "v"(off0), "s"(base) : "memory");
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :: "s"(slot + 1024u), "v"(off1), "s"(base) : "memory");
  };
  for (int m = 0; m < kRing - 1 && m < mine; ++m) issue(m);
  uint32_t acc = 0;
  for (int m = 0; m < mine; ++m) {
    if (m + kRing - 1 < mine) {
      issue(m + kRing - 1);
      wait_vmcnt<2 * (kRing - 1)>();
    } else {
      wait_vmcnt<0>();
    }
    const uint4 v = *reinterpret_cast<const uint4*>(&ring[wave][m % kRing][16 * lane]);
    acc ^= v.x ^ v.w;
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kMfmaGrid = 2048;      // workgroups of 4 waves: 8 waves per SIMD over 256 CUs

// CH independent accumulator chains per wave, one instruction of each per
// iteration, operands fixed in registers.
template <int FORM>
__global__ void __launch_bounds__(256) mfma_kernel(int iters, float* sink) {
  constexpr int CH = FORM == 0 ? 8 : 4;
  v8bf a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 0.001f + i);
    b[i] = (__bf16)(i * 0.5f);
  }
  float s = 0.0f;
  if constexpr (FORM == 0) {
    v4f c[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) c[j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < CH; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  } else {
    v16f c[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) c[j][i] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < CH; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) s += c[j][i];
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" int64_t dsa_probe_stream_read_sink_words(int64_t bytes) {
  if (bytes <= 0 || bytes % kTile) return -1;
  const int64_t ntiles = bytes / kTile;
  return (ntiles + kChunkTiles - 1) / kChunkTiles * 256;
}

extern "C" int dsa_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int64_t sink_words,
                                     void* stream) {
  if (!buf || !sink || bytes <= 0 || bytes % kTile || ((uintptr_t)buf & 15)) return -1;
  const int64_t need = dsa_probe_stream_read_sink_words(bytes);
  if (sink_words < need) return -1;
  const int64_t ntiles = bytes / kTile;
  const int64_t grid = need / 256;
  if (grid > INT32_MAX) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const char*>(buf), ntiles, sink);
  return (int)hipGetLastError();
}

extern "C" int64_t dsa_probe_mfma_sink_words(void) { return (int64_t)kMfmaGrid * 256; }

extern "C" double dsa_probe_mfma_flops(int form, int iters) {
  if (form == 0) return (double)kMfmaGrid * 4 * iters * 8 * (2.0 * 16 * 16 * 32);
  if (form == 1) return (double)kMfmaGrid * 4 * iters * 4 * (2.0 * 32 * 32 * 16);
  return -1.0;
}

extern "C" int dsa_probe_mfma(int form, int iters, float* sink, int64_t sink_words, void* stream) {
  if (!sink || iters <= 0 || (form != 0 && form != 1) || sink_words < dsa_probe_mfma_sink_words()) return -1;
  if (form == 0)
    hipLaunchKernelGGL(mfma_kernel<0>, dim3(kMfmaGrid), dim3(256), 0, (hipStream_t)stream, iters, sink);
  else
    hipLaunchKernelGGL(mfma_kernel<1>, dim3(kMfmaGrid), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return (int)hipGetLastError();
}
