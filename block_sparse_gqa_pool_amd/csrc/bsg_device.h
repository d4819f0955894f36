// Device helpers shared by the gfx950 kernels of the block-sparse GQA library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsg.h"

namespace bsg {

typedef uint16_t bf16_t;  // bf16 storage (bit pattern)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

// Round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ float ld_any(const float* p) { return *p; }
__device__ __forceinline__ float ld_any(const bf16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void st_any(float* p, float v) { *p = v; }
__device__ __forceinline__ void st_any(bf16_t* p, float v) { *p = f32_to_bf16(v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Eight OCP E4M3 codes (little-endian bytes of two words) -> eight bf16 values, unscaled.
// Every E4M3 value is exact in bf16; the hardware conversion (v_cvt_pk_f32_fp8) is exact too.
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(uint2 w) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, true);
  bf16x8_t r;
  r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)b[0]; r[3] = (__bf16)b[1];
  r[4] = (__bf16)c[0]; r[5] = (__bf16)c[1]; r[6] = (__bf16)d[0]; r[7] = (__bf16)d[1];
  return r;
}

// Monotone map float -> uint32 (larger float -> larger key); -0.0 is folded onto +0.0.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 64-bit selection key: score first (higher wins), then block index (lower wins).
__device__ __forceinline__ uint64_t sel_key(float s, int j) {
  return ((uint64_t)order_key(s) << 32) | (uint64_t)(0xffffffffu - (uint32_t)j);
}
__device__ __forceinline__ int sel_key_index(uint64_t key) { return (int)(0xffffffffu - (uint32_t)key); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    T w = __shfl_xor(v, o, 64);
    v = v > w ? v : w;
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over aligned groups of SEG (4, 8 or 16) lanes with DPP lane moves (no LDS traffic);
// every lane of a group receives the group's sum.
template <int SEG>
__device__ __forceinline__ float seg_sum_dpp(float v) {
  static_assert(SEG == 4 || SEG == 8 || SEG == 16, "segment of 4, 8 or 16 lanes");
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  if (SEG >= 8) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // half mirror
  if (SEG >= 16) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // mirror
  return v;
}

}  // namespace bsg
