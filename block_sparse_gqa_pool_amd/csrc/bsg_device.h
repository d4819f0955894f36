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

// Rows of the token-list kernels: (sequence b, query position t) for the window [t0, t0 + CT)
// of the T query positions of every sequence, local row rl = b * CT + (t - t0); positions
// at or past T are absent.  Decode: T = CT = 1, t0 = 0, so rl = b.  Query position t of
// sequence b sits at cache position kv_lens[b] - T + t.
struct RowWindow {
  int T, t0, CT;
  __host__ __device__ int seq(int rl) const { return rl / CT; }
  __host__ __device__ int pos(int rl) const { return t0 + rl % CT; }
};

// Ids read from the caller's tables are clamped into range before they address memory, so a
// bad entry never leads a kernel out of its buffers.  Debug builds (-DBSG_DEBUG) also record
// each clamped id as a bit of a device word (one per source file, the file's kernels being
// compiled apart), which bsg_debug_errors() reads back; release builds only clamp.
enum : unsigned { DBG_PAGE_ID = 1u, DBG_BLOCK_ID = 2u, DBG_TOKEN_ID = 4u };
#ifdef BSG_DEBUG
[[maybe_unused]] static __device__ unsigned int dbg_word;
#endif
__device__ __forceinline__ void dbg_flag(bool bad, unsigned bit) {
#ifdef BSG_DEBUG
  if (bad) atomicOr(&dbg_word, bit);
#else
  (void)bad;
  (void)bit;
#endif
}
// physical page id from a page table: [0, num_pages)
__device__ __forceinline__ int page_id(int p, int num_pages) {
  dbg_flag(p < 0 || p >= num_pages, DBG_PAGE_ID);
  return clampi(p, 0, num_pages - 1);
}
// logical block id from a selection (>= 0 here; -1 padding is handled by the caller): below
// pt_stride
__device__ __forceinline__ int block_id(int j, int pt_stride) {
  dbg_flag(j < 0 || j >= pt_stride, DBG_BLOCK_ID);
  return clampi(j, 0, pt_stride - 1);
}

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

// Ascending bitonic sort of N (a power of two) ints held in registers: every index is a
// compile-time constant once the loops unroll (a rank count over N x N pairs would not
// unroll at N = 64 and would move the array to scratch).
template <int N>
__device__ __forceinline__ void sort_ints_asc(int (&v)[N]) {
#pragma unroll
  for (int k = 2; k <= N; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < N; i++) {
        const int l = i ^ j;
        if (l > i) {
          const int x = v[i], y = v[l];
          const bool up = (i & k) == 0;
          v[i] = up ? min(x, y) : max(x, y);
          v[l] = up ? max(x, y) : min(x, y);
        }
      }
}

// Host side of the debug word of the file that expands this (once, at namespace scope):
// reads it and, with reset, clears it.  Synchronous.
#ifdef BSG_DEBUG
#define BSG_DEBUG_FILE(name)                                                                    \
  __attribute__((visibility("hidden"))) int dbg_fetch_##name(unsigned* out, int reset) {         \
    if (hipMemcpyFromSymbol(out, HIP_SYMBOL(dbg_word), sizeof(unsigned)) != hipSuccess) return -1; \
    const unsigned zero = 0;                                                                     \
    if (reset && hipMemcpyToSymbol(HIP_SYMBOL(dbg_word), &zero, sizeof(unsigned)) != hipSuccess) \
      return -1;                                                                                 \
    return 0;                                                                                    \
  }
#else
#define BSG_DEBUG_FILE(name)
#endif

// Asynchronous copy global -> LDS, 16 bytes per lane: lane l's 16 bytes land at byte
// lds_base + 16 l (gfx950 global_load_lds_dwordx4; the LDS base goes through M0, which the
// compiler reserves and sets before each of its own uses).  Written as inline asm so that the
// compiler does not serialise later LDS reads of other buffers behind it; completion is waited
// for explicitly with vmcnt.  Lanes outside EXEC copy nothing.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base) : "memory");
}

}  // namespace bsg
