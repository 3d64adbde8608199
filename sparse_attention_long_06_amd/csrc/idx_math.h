// Lane-level pieces of the lightning indexer's contraction on gfx950: FP8
// key/query fragments, their exact widening to bf16, the
// v_mfma_f32_16x16x32_bf16 dot over d_I, the ReLU clamp and the sum over the
// four 16-lane groups of a wave.  Operand layout: lane l holds row (l % 16)
// and bytes [g*d_I/4, (g+1)*d_I/4) of it, g = l / 16.
#pragma once

#include "dsa_common.h"

namespace dsa {

// Raw FP8 fragment of one row held by a lane: d_I/4 bytes.
template <int DI> struct Frag;
template <> struct Frag<128> { v4i lo, hi; };
template <> struct Frag<32> { long v; };

template <int DI, bool NT>
__device__ __forceinline__ void load_frag(Frag<DI>& f, const char* row, int grp) {
  if constexpr (DI == 128) {
    const v4i* p = reinterpret_cast<const v4i*>(row + 32 * grp);
    if constexpr (NT) {
      f.lo = __builtin_nontemporal_load(p);
      f.hi = __builtin_nontemporal_load(p + 1);
    } else {
      f.lo = p[0];
      f.hi = p[1];
    }
  } else {
    const long* p = reinterpret_cast<const long*>(row + 8 * grp);
    if constexpr (NT) f.v = __builtin_nontemporal_load(p); else f.v = *p;
  }
}

template <int DI>
__device__ __forceinline__ void zero_frag(Frag<DI>& f) {
  if constexpr (DI == 128) {
    f.lo = v4i{0, 0, 0, 0};
    f.hi = v4i{0, 0, 0, 0};
  } else {
    f.v = 0;
  }
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Eight e4m3fn bytes (two dwords) -> eight bf16, exactly.
__device__ __forceinline__ v8bf widen8(int lo, int hi) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// bf16 view of a fragment: d_I/32 chunks of 8 values.
template <int DI> struct Wide { v8bf c[DI / 32]; };

template <int DI>
__device__ __forceinline__ Wide<DI> widen(const Frag<DI>& f) {
  Wide<DI> w;
  if constexpr (DI == 128) {
    w.c[0] = widen8(f.lo.x, f.lo.y);
    w.c[1] = widen8(f.lo.z, f.lo.w);
    w.c[2] = widen8(f.hi.x, f.hi.y);
    w.c[3] = widen8(f.hi.z, f.hi.w);
  } else {
    w.c[0] = widen8((int)(f.v & 0xFFFFFFFF), (int)(f.v >> 32));
  }
  return w;
}

template <int DI>
__device__ __forceinline__ v4f mfma_dot(const Wide<DI>& a, const Wide<DI>& b) {
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < DI / 32; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.c[c], b.c[c], acc, 0, 0, 0);
  return acc;
}

// ReLU of a finite MFMA result as a clamp to [0, FLT_MAX]: one v_med3_f32,
// where fmaxf would add a NaN-quieting canonicalize.
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, 3.402823466e38f); }

// Sum over the four 16-lane groups (rows) of a wave: after the row swaps every
// lane holds the total of its column.  Pure VALU (no LDS permute).
__device__ __forceinline__ float group_sum(float part) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(part), __float_as_uint(part), false, false);
  part = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

}  // namespace dsa
