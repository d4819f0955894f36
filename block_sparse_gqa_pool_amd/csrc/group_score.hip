// Materialised group scores (Ling 2.0 page, "Summarizing the Breakthrough": the heads of a
// GQA group share one block selection; MSA post, second paragraph: blocks are scored per
// GQA group).  score[b, g, t, j] = (sum_h q[b, h, t, :]) . rep[page_table[b, j], g, :]
// for the causal candidates j < own block of t; -inf elsewhere.
//
// One workgroup scores a tile of 16 query tokens against 64 candidate blocks of one
// (sequence, group): the group-summed queries (fp32) and the 64 representatives (fp32)
// are staged in LDS, and each thread produces 4 dot products of length D in fp32.
#include "bsg_device.h"
#include "bsg_internal.h"

namespace bsg {

namespace {
constexpr int GS_TQ = 16;
constexpr int GS_TJ = 64;
}  // namespace

template <typename T>
__global__ __launch_bounds__(256) void group_score_kernel(const T* __restrict__ q, const int32_t* __restrict__ kv_lens,
                                                          const T* __restrict__ block_cache,
                                                          const int32_t* __restrict__ page_table,
                                                          float* __restrict__ scores, int q_len, int score_stride,
                                                          int Hq, int Hkv, int D, int bs, int num_pages,
                                                          int pt_stride) {
  extern __shared__ float gs_smem[];
  const int DP = D + 1;
  float* qs = gs_smem;                 // [GS_TQ][DP]
  float* rs = gs_smem + GS_TQ * DP;    // [GS_TJ][DP]
  const int G = Hq / Hkv;
  const int bg = blockIdx.z;
  const int b = bg / Hkv, g = bg % Hkv;
  const int t0 = blockIdx.x * GS_TQ;
  const int j0 = blockIdx.y * GS_TJ;
  const int L = kv_lens[b];
  const int tid = threadIdx.x;

  // group-summed queries, fp32, heads in order
  for (int e = tid; e < GS_TQ * D; e += 256) {
    const int tt = e / D, dd = e % D;
    const int t = t0 + tt;
    float s = 0.0f;
    if (t < q_len) {
      const T* qp = q + (((size_t)b * Hq + (size_t)g * G) * q_len + t) * D + dd;
      for (int h = 0; h < G; h++) s += ld_any(qp + (size_t)h * q_len * D);
    }
    qs[tt * DP + dd] = s;
  }
  // largest own block in this token tile bounds the candidates worth loading
  const int tlast = min(t0 + GS_TQ, q_len) - 1;
  const int own_max = (L - q_len + tlast) / bs;
  const int jlim = min(min(own_max, pt_stride), j0 + GS_TJ);
  for (int e = tid; e < GS_TJ * D; e += 256) {
    const int jj = e / D, dd = e % D;
    const int j = j0 + jj;
    float v = 0.0f;
    if (j < jlim) {
      const int p = page_id(page_table[(size_t)b * pt_stride + j], num_pages);
      v = ld_any(block_cache + ((size_t)p * Hkv + g) * D + dd);
    }
    rs[jj * DP + dd] = v;
  }
  __syncthreads();

  const int tt = tid / 16;
  const int t = t0 + tt;
  if (t >= q_len) return;
  const int own = (L - q_len + t) / bs;
  const float* qrow = qs + tt * DP;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int jj = (tid % 16) + 16 * r;
    const int j = j0 + jj;
    if (j >= score_stride) continue;
    float acc = -INFINITY;
    if (j < own && j < pt_stride) {
      const float* rrow = rs + jj * DP;
      acc = 0.0f;
      for (int dd = 0; dd < D; dd++) acc = fmaf(qrow[dd], rrow[dd], acc);
    }
    scores[(((size_t)b * Hkv + g) * q_len + t) * score_stride + j] = acc;
  }
}

hipError_t launch_group_score(const bsg_dims& d, const void* q, int q_len, const int32_t* kv_lens,
                              const void* block_cache, const int32_t* page_table, float* scores,
                              int score_stride, hipStream_t stream) {
  dim3 grid((q_len + GS_TQ - 1) / GS_TQ, (score_stride + GS_TJ - 1) / GS_TJ, d.batch * d.num_kv_heads);
  const size_t smem = (size_t)(GS_TQ + GS_TJ) * (d.head_dim + 1) * sizeof(float);
  if (d.dtype == BSG_BF16)
    hipLaunchKernelGGL(group_score_kernel<bf16_t>, grid, dim3(256), smem, stream, (const bf16_t*)q, kv_lens,
                       (const bf16_t*)block_cache, page_table, scores, q_len, score_stride, d.num_q_heads,
                       d.num_kv_heads, d.head_dim, d.page_size, d.num_pages, d.pt_stride);
  else
    hipLaunchKernelGGL(group_score_kernel<float>, grid, dim3(256), smem, stream, (const float*)q, kv_lens,
                       (const float*)block_cache, page_table, scores, q_len, score_stride, d.num_q_heads,
                       d.num_kv_heads, d.head_dim, d.page_size, d.num_pages, d.pt_stride);
  return hipGetLastError();
}

BSG_DEBUG_FILE(group_score)

}  // namespace bsg
