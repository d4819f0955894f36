// fp8 KV cache and fp8 block cache (KV-cache quantisation: "Sparse Attention + Linear
// Backbones", section 3, and "Sparse Attention for Long-Context LLMs", section 8; the pages
// fix no format).  Format: OCP E4M3 codes, one power-of-two scale per (page, KV head) tile,
// the smallest 2^e with max|x| <= 448 * 2^e over the tile's valid tokens; codes are x / 2^e
// rounded to nearest even; slots past the sequence length hold code 0.
//
//  * quantize_pages_fp8_kernel: one workgroup per (sequence, block); per KV head the tile is
//    loaded once into registers, its max |x| reduced, and the codes written (8 codes per
//    16-byte load).  HBM-bound: bs * D * 2 bytes read, bs * D bytes written per tile.
//  * block_pool_fp8_kernel: one workgroup per (sequence, complete block); a thread owns 4
//    columns of one head and sums their decoded codes in float32 in token order, scales by
//    scale / bs, and the head's D values are quantised like a KV tile.
#include "bsg_device.h"
#include "bsg_internal.h"

namespace bsg {

// Scale exponent: the smallest e with amax <= 448 * 2^e (0 for amax = 0), clamped to
// [-126, 127].  With amax = 1.m * 2^(X - 127): e = X - 135, plus one when 1.m > 1.75.
__device__ __forceinline__ int fp8_scale_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  if (amax == 0.0f) return 0;
  const int X = (int)(u >> 23);
  if (X == 0) return -126;
  const int e = X - 135 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  return e < -126 ? -126 : (e > 127 ? 127 : e);
}

// E4M3 code of y, |y| <= 448: nearest, ties to even.  At or above 2^-6 the float's top three
// mantissa bits are rounded (the carry may move into the exponent); below, y is a multiple
// of 2^-9 rounded to the nearest even count (8 counts = 2^-6 = code 0x08).
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t s = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x3c800000u) {
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  } else {
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  return s | code;
}

template <int BS, int D>
__global__ __launch_bounds__(256) void quantize_pages_fp8_kernel(const bf16_t* __restrict__ src,
                                                                 const int32_t* __restrict__ page_table,
                                                                 const int32_t* __restrict__ kv_lens,
                                                                 uint8_t* __restrict__ codes, float* __restrict__ scales,
                                                                 int Hkv, int num_pages, int pt_stride) {
  constexpr int CPR = D / 8;                    // 16-byte chunks per row
  constexpr int NCH = BS * CPR / 256;           // chunks per thread
  static_assert(NCH * 256 == BS * CPR, "tile split");
  __shared__ float red[4];
  const int b = blockIdx.y, j = blockIdx.x;
  const int L = kv_lens[b];
  const int nblk = min((L + BS - 1) / BS, pt_stride);
  if (j >= nblk) return;
  const int n = min(BS, L - j * BS);            // valid tokens of the block
  const int p = page_id(page_table[(size_t)b * pt_stride + j], num_pages);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int g = 0; g < Hkv; g++) {
    const size_t tile = ((size_t)p * Hkv + g) * BS * D;
    uint4 x[NCH];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      const int e = c * 256 + tid;
      const int row = e / CPR;
      x[c] = row < n ? *reinterpret_cast<const uint4*>(src + tile + (size_t)e * 8) : make_uint4(0, 0, 0, 0);
      const uint32_t w[4] = {x[c].x, x[c].y, x[c].z, x[c].w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        amax = fmaxf(amax, fabsf(__uint_as_float(w[i] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(w[i] & 0xffff0000u)));
      }
    }
    amax = wave_max(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();                             // red is reused by the next head
    const int ex = fp8_scale_exp(amax);
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      const int e = c * 256 + tid;
      const uint32_t w[4] = {x[c].x, x[c].y, x[c].z, x[c].w};
      uint32_t q[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const uint32_t lo = e4m3_rne(__builtin_ldexpf(__uint_as_float(w[i] << 16), -ex));
        const uint32_t hi = e4m3_rne(__builtin_ldexpf(__uint_as_float(w[i] & 0xffff0000u), -ex));
        q[i >> 1] |= (lo | (hi << 8)) << (16 * (i & 1));
      }
      *reinterpret_cast<uint2*>(codes + tile + (size_t)e * 8) = make_uint2(q[0], q[1]);   // rows >= n: zeros
    }
    if (tid == 0) scales[(size_t)p * Hkv + g] = __builtin_ldexpf(1.0f, ex);
  }
}

template <int BS, int D>
__global__ __launch_bounds__(256) void block_pool_fp8_kernel(const uint8_t* __restrict__ k_codes,
                                                             const float* __restrict__ k_scales,
                                                             const int32_t* __restrict__ page_table,
                                                             const int32_t* __restrict__ kv_lens,
                                                             const int32_t* __restrict__ blk_begin,
                                                             uint8_t* __restrict__ rep_codes,
                                                             float* __restrict__ rep_scales, int Hkv, int num_pages,
                                                             int pt_stride) {
  constexpr int SEG = D / 4;                    // threads per head (4 columns each)
  const int b = blockIdx.y, j = blockIdx.x;
  const int L = kv_lens[b];
  const int nfull = min(L / BS, pt_stride);
  const int begin = blk_begin ? max(blk_begin[b], 0) : 0;
  if (j < begin || j >= nfull) return;
  const int p = page_id(page_table[(size_t)b * pt_stride + j], num_pages);
  const float inv = 1.0f / (float)BS;
  // every pass covers 256 / SEG whole heads, so a head's SEG threads are one aligned lane group
  for (int u0 = 0; u0 < Hkv * SEG; u0 += 256) {
    const int u = u0 + (int)threadIdx.x;
    const bool on = u < Hkv * SEG;
    const int g = on ? u / SEG : 0, d4 = u % SEG;
    const uint8_t* src = k_codes + ((size_t)p * Hkv + g) * BS * D + 4 * d4;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (on) {
#pragma unroll 1
      for (int i0 = 0; i0 < BS; i0 += 8) {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; i++) w[i] = *reinterpret_cast<const uint32_t*>(src + (size_t)(i0 + i) * D);
#pragma unroll
        for (int i = 0; i < 8; i++) {                       // token order
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
          acc[0] = acc[0] + lo[0];
          acc[1] = acc[1] + lo[1];
          acc[2] = acc[2] + hi[0];
          acc[3] = acc[3] + hi[1];
        }
      }
    }
    const float f = (on ? k_scales[(size_t)p * Hkv + g] : 0.0f) * inv;   // a power of two: exact
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      acc[c] = acc[c] * f;
      amax = fmaxf(amax, fabsf(acc[c]));
    }
#pragma unroll
    for (int o = SEG / 2; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    const int ex = fp8_scale_exp(amax);
    uint32_t q = 0u;
#pragma unroll
    for (int c = 0; c < 4; c++) q |= e4m3_rne(__builtin_ldexpf(acc[c], -ex)) << (8 * c);
    if (on) {
      *reinterpret_cast<uint32_t*>(rep_codes + ((size_t)p * Hkv + g) * D + 4 * d4) = q;
      if (d4 == 0) rep_scales[(size_t)p * Hkv + g] = __builtin_ldexpf(1.0f, ex);
    }
  }
}

hipError_t launch_quantize_pages_fp8(const bsg_dims& d, const void* src, const int32_t* page_table,
                                     const int32_t* kv_lens, uint8_t* codes, float* scales, hipStream_t stream) {
  dim3 grid(d.pt_stride, d.batch);
#define BSG_Q8(BB, DD)                                                                                        \
  hipLaunchKernelGGL((quantize_pages_fp8_kernel<BB, DD>), grid, dim3(256), 0, stream, (const bf16_t*)src,      \
                     page_table, kv_lens, codes, scales, d.num_kv_heads, d.num_pages, d.pt_stride)
  if (d.page_size == 64) {
    if (d.head_dim == 128) BSG_Q8(64, 128); else BSG_Q8(64, 64);
  } else {
    if (d.head_dim == 128) BSG_Q8(128, 128); else BSG_Q8(128, 64);
  }
#undef BSG_Q8
  return hipGetLastError();
}

hipError_t launch_block_pool_fp8(const bsg_dims& d, const uint8_t* k_codes, const float* k_scales,
                                 const int32_t* page_table, const int32_t* kv_lens, const int32_t* blk_begin,
                                 uint8_t* rep_codes, float* rep_scales, hipStream_t stream) {
  dim3 grid(d.pt_stride, d.batch);
#define BSG_BP8(BB, DD)                                                                                       \
  hipLaunchKernelGGL((block_pool_fp8_kernel<BB, DD>), grid, dim3(256), 0, stream, k_codes, k_scales,          \
                     page_table, kv_lens, blk_begin, rep_codes, rep_scales, d.num_kv_heads, d.num_pages,      \
                     d.pt_stride)
  if (d.page_size == 64) {
    if (d.head_dim == 128) BSG_BP8(64, 128); else BSG_BP8(64, 64);
  } else {
    if (d.head_dim == 128) BSG_BP8(128, 128); else BSG_BP8(128, 64);
  }
#undef BSG_BP8
  return hipGetLastError();
}

BSG_DEBUG_FILE(fp8_cache)

}  // namespace bsg
