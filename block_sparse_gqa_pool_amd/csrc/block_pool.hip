// Block representatives: mean of each complete page's keys per KV head, written into the
// page-indexed block cache (Ling 2.0 page, "Summarizing the Breakthrough": blocks are
// aggregated at prefill into a cache that shares the KV cache's page indexing).
//
// HBM-bound: every complete (page, head) key tile is read once (bs * D elements) and one
// D-vector is written.  Each thread owns 16 contiguous bytes of one head's row, so a wave
// reads contiguous 256-byte (bf16, D = 128) row segments; the token loop keeps 8 loads in
// flight.  The fp32 sum runs in token order so that the result is bit-reproducible.
#include "bsg_device.h"
#include "bsg_internal.h"

namespace bsg {

template <typename T>
struct Vec16;  // 16 bytes of T
template <>
struct Vec16<bf16_t> {
  static constexpr int N = 8;
  uint4 raw;
  __device__ __forceinline__ float get(int i) const {
    uint32_t w = (&raw.x)[i >> 1];
    return bf16_to_f32((bf16_t)((i & 1) ? (w >> 16) : (w & 0xffffu)));
  }
  __device__ __forceinline__ void set(const float* v) {
    raw.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    raw.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    raw.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
    raw.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
  }
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  float4 raw;
  __device__ __forceinline__ float get(int i) const { return (&raw.x)[i]; }
  __device__ __forceinline__ void set(const float* v) { raw = make_float4(v[0], v[1], v[2], v[3]); }
};

template <typename T, int BS>
__global__ __launch_bounds__(256) void block_pool_kernel(const T* __restrict__ k_cache,
                                                         const int32_t* __restrict__ page_table,
                                                         const int32_t* __restrict__ kv_lens,
                                                         const int32_t* __restrict__ blk_begin,
                                                         T* __restrict__ block_cache, int Hkv, int D,
                                                         int num_pages, int pt_stride, int blocks_per_wg) {
  typedef Vec16<T> V;
  constexpr int N = V::N;
  const int b = blockIdx.y;
  const int L = kv_lens[b];
  const int nfull = min(L / BS, pt_stride);
  const int begin = blk_begin ? max(blk_begin[b], 0) : 0;
  const int j0 = blockIdx.x * blocks_per_wg;
  const int jlo = max(j0, begin), jhi = min(j0 + blocks_per_wg, nfull);
  if (jlo >= jhi) return;
  const int units = Hkv * (D / N);  // 16-byte lanes per page
  const int total = (jhi - jlo) * units;
  const float inv = 1.0f / (float)BS;
  for (int w = threadIdx.x; w < total; w += blockDim.x) {
    const int j = jlo + w / units;
    const int u = w % units;
    const int g = u / (D / N);
    const int d0 = (u % (D / N)) * N;
    const int p = page_id(page_table[(size_t)b * pt_stride + j], num_pages);
    const T* src = k_cache + (((size_t)p * Hkv + g) * BS) * D + d0;
    float acc[N];
#pragma unroll
    for (int e = 0; e < N; e++) acc[e] = 0.0f;
#pragma unroll 1
    for (int i0 = 0; i0 < BS; i0 += 8) {
      V x[8];
#pragma unroll
      for (int i = 0; i < 8; i++) x[i].raw = *reinterpret_cast<const decltype(V::raw)*>(src + (size_t)(i0 + i) * D);
#pragma unroll
      for (int i = 0; i < 8; i++)
#pragma unroll
        for (int e = 0; e < N; e++) acc[e] = acc[e] + x[i].get(e);  // token order
    }
#pragma unroll
    for (int e = 0; e < N; e++) acc[e] = acc[e] * inv;
    V o;
    o.set(acc);
    *reinterpret_cast<decltype(V::raw)*>(block_cache + ((size_t)p * Hkv + g) * D + d0) = o.raw;
  }
}

hipError_t launch_block_pool(const bsg_dims& d, const void* k_cache, const int32_t* page_table,
                             const int32_t* kv_lens, const int32_t* blk_begin, void* block_cache,
                             hipStream_t stream) {
  const long long work = (long long)d.batch * d.pt_stride;
  int bpw = (int)(work / 2048);
  bpw = bpw < 1 ? 1 : (bpw > 8 ? 8 : bpw);
  dim3 grid((d.pt_stride + bpw - 1) / bpw, d.batch);
  dim3 block(256);
#define BSG_BP(T, BS)                                                                                  \
  hipLaunchKernelGGL((block_pool_kernel<T, BS>), grid, block, 0, stream, (const T*)k_cache, page_table, \
                     kv_lens, blk_begin, (T*)block_cache, d.num_kv_heads, d.head_dim, d.num_pages,     \
                     d.pt_stride, bpw)
  if (d.dtype == BSG_BF16) {
    if (d.page_size == 64) BSG_BP(bf16_t, 64); else BSG_BP(bf16_t, 128);
  } else {
    if (d.page_size == 64) BSG_BP(float, 64); else BSG_BP(float, 128);
  }
#undef BSG_BP
  return hipGetLastError();
}

BSG_DEBUG_FILE(block_pool)

}  // namespace bsg
