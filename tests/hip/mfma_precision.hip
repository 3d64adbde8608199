// Test-only probe of matrix-core dot-product accuracy on gfx950 (not part of
// the library).  K = 128 in every variant:
//   variant 0: v_mfma_scale_f32_16x16x128_f8f6f4 on e4m3fn operands,
//   variant 1: four chained v_mfma_f32_16x16x32_fp8_fp8,
//   variant 2: four chained v_mfma_f32_16x16x32_bf16 on the same values
//              widened exactly to bf16 by the host,
//   variant 3: two chained v_mfma_scale_f32_32x32x64_f8f6f4 (32x32 tile).
// Variants 0-2: one 16x16 output tile per workgroup (one wave); lane l
// supplies row/column (l % 16) and contraction slice (l / 16) of each operand,
// the same way for A and B, and output element (4*(l/16)+i, l%16) comes back
// in accumulator register i of lane l.  Variant 3: one 32x32 tile per
// workgroup; lane l supplies row/column (l % 32) and contraction slice (l / 32)
// of each 64-wide step, and output element (8*(i/4) + 4*(l/32) + i%4, l%32)
// comes back in register i.
#include <hip/hip_runtime.h>
#include <stdint.h>
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
extern "C" __global__ void probe(const uint8_t* A8, const uint8_t* B8, const uint16_t* A16, const uint16_t* B16,
                                 float* out, int nblk) {
  const int blk = blockIdx.x;
  if (blk >= nblk) return;
  const int l = threadIdx.x, n = l & 15, g = l >> 4;
  const uint8_t* a8 = A8 + ((size_t)blk * 16 + n) * 128;
  const uint8_t* b8 = B8 + ((size_t)blk * 16 + n) * 128;
  const uint16_t* a16 = A16 + ((size_t)blk * 16 + n) * 128;
  const uint16_t* b16 = B16 + ((size_t)blk * 16 + n) * 128;
  v4f z = {0, 0, 0, 0};
  // variant 0
  {
    const v4i* pa = (const v4i*)(a8 + 32 * g);
    const v4i* pb = (const v4i*)(b8 + 32 * g);
    v4i a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
    v8i A = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    v8i B = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, z, 0, 0, 0, 127, 0, 127);
    for (int i = 0; i < 4; ++i) out[((size_t)0 * nblk + blk) * 256 + (4 * g + i) * 16 + n] = d[i];
  }
  // variant 1
  {
    v4f d = z;
    for (int c = 0; c < 4; ++c) {
      long a = *(const long*)(a8 + 32 * c + 8 * g);
      long b = *(const long*)(b8 + 32 * c + 8 * g);
      d = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, d, 0, 0, 0);
    }
    for (int i = 0; i < 4; ++i) out[((size_t)1 * nblk + blk) * 256 + (4 * g + i) * 16 + n] = d[i];
  }
  // variant 2
  {
    v4f d = z;
    for (int c = 0; c < 4; ++c) {
      v8bf a = __builtin_bit_cast(v8bf, *(const v4i*)(a16 + 32 * c + 8 * g));
      v8bf b = __builtin_bit_cast(v8bf, *(const v4i*)(b16 + 32 * c + 8 * g));
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d, 0, 0, 0);
    }
    for (int i = 0; i < 4; ++i) out[((size_t)2 * nblk + blk) * 256 + (4 * g + i) * 16 + n] = d[i];
  }
}

// variant 3: workgroup blk (one wave) computes the 32x32 tile of rows
// blk*32.. of A against rows blk*32.. of B; out32[blk*1024 + row*32 + col].
extern "C" __global__ void probe32(const uint8_t* A8, const uint8_t* B8, float* out32, int nblk) {
  const int blk = blockIdx.x;
  if (blk >= nblk) return;
  const int l = threadIdx.x, n = l & 31, g = l >> 5;
  const uint8_t* a8 = A8 + ((size_t)blk * 32 + n) * 128;
  const uint8_t* b8 = B8 + ((size_t)blk * 32 + n) * 128;
  v16f d;
  for (int i = 0; i < 16; ++i) d[i] = 0.0f;
  for (int c = 0; c < 2; ++c) {
    const v4i* pa = (const v4i*)(a8 + 64 * c + 32 * g);
    const v4i* pb = (const v4i*)(b8 + 64 * c + 32 * g);
    v4i a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
    v8i A = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    v8i B = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, d, 0, 0, 0, 127, 0, 127);
  }
  for (int i = 0; i < 16; ++i) out32[(size_t)blk * 1024 + (8 * (i / 4) + 4 * g + (i % 4)) * 32 + n] = d[i];
}
