// Causal top-k block selection from materialised scores, exp-free (MSA post, second and
// third paragraphs: top-k per GQA group, ranked on raw logits).
//
// Ranking key: 64 bits = (monotone uint32 image of the fp32 score, ~block index), so that a
// larger key is a larger score or, for equal scores, a lower block index.  All keys of a row
// are distinct, which makes every comparison strict and the result unique.
//
// Two kernels give identical results:
//  * rows_kernel: one thread per row, streaming insertion into a register-resident sorted
//    list (many rows with up to ~a thousand candidates: prefill).
//  * wg_kernel: one workgroup per row (few rows with many candidates: decode).  Each thread
//    takes the maximum of its strided share of candidates; the m-th largest of these maxima
//    (m = top_k - 1) is a threshold that at least m candidates reach and that at most m
//    threads' shares reach, so at most m * share keys survive it.  The survivors are sorted
//    with an LDS bitonic network and the first m are kept.
#include "bsg_device.h"
#include "bsg_internal.h"

namespace bsg {

template <int KCAP>
__global__ __launch_bounds__(256) void topk_rows_kernel(const float* __restrict__ scores, const int32_t* __restrict__ kv_lens,
                                                        int32_t* __restrict__ block_idx, int rows, int Hkv,
                                                        int q_len, int score_stride, int bs, int top_k) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const int b = row / (Hkv * q_len);
  const int t = row % q_len;
  const int own = max(kv_lens[b] - q_len + t, 0) / bs;
  const int ncand = min(own, score_stride);
  const int m = top_k - 1;
  const float* s = scores + (size_t)row * score_stride;
  uint64_t best[KCAP];
#pragma unroll
  for (int i = 0; i < KCAP; i++) best[i] = 0;
  for (int j = 0; j < ncand; j++) {
    uint64_t c = sel_key(s[j], j);
    if (c > best[KCAP - 1]) {
#pragma unroll
      for (int i = 0; i < KCAP; i++) {
        const uint64_t bi = best[i];
        const bool gt = c > bi;
        best[i] = gt ? c : bi;
        c = gt ? bi : c;
      }
    }
  }
  const int cnt = min(m, ncand);
  int32_t* out = block_idx + (size_t)row * top_k;
  if constexpr (KCAP > 32) {
    // ascending by a register sorting network (unused slots hold INT_MAX and sort last)
    int ids[KCAP];
#pragma unroll
    for (int i = 0; i < KCAP; i++) ids[i] = i < cnt ? sel_key_index(best[i]) : 0x7fffffff;
    sort_ints_asc(ids);
#pragma unroll
    for (int i = 0; i < KCAP; i++)
      if (i < cnt) out[i] = ids[i];
  } else {
    // rank of each kept id among the kept ids gives its ascending position
#pragma unroll
    for (int i = 0; i < KCAP; i++) {
      if (i < cnt) {
        const int ji = sel_key_index(best[i]);
        int rank = 0;
#pragma unroll
        for (int i2 = 0; i2 < KCAP; i2++)
          if (i2 < cnt) rank += (sel_key_index(best[i2]) < ji) ? 1 : 0;
        out[rank] = ji;
      }
    }
  }
  out[cnt] = own;
  for (int i = cnt + 1; i < top_k; i++) out[i] = -1;
}

// In-LDS bitonic sort of n (power of two) 64-bit keys, descending.
__device__ __forceinline__ void bitonic_desc(uint64_t* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = a[i], y = a[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) {
            a[i] = y;
            a[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void topk_wg_kernel(const float* __restrict__ scores, const int32_t* __restrict__ kv_lens,
                                                     int32_t* __restrict__ block_idx, int Hkv, int q_len,
                                                     int score_stride, int bs, int top_k, int surv_cap) {
  extern __shared__ uint64_t tk_smem[];
  uint64_t* tmax = tk_smem;            // [NT]
  uint64_t* surv = tk_smem + NT;       // [surv_cap] (power of two)
  __shared__ int n_surv;
  __shared__ int kept[64];
  const int row = blockIdx.x;
  const int b = row / (Hkv * q_len);
  const int t = row % q_len;
  const int own = max(kv_lens[b] - q_len + t, 0) / bs;
  const int ncand = min(own, score_stride);
  const int m = top_k - 1;
  int32_t* out = block_idx + (size_t)row * top_k;
  const int tid = threadIdx.x;
  if (ncand <= m) {  // every candidate is kept (also covers top_k == 1 with no candidate)
    for (int i = tid; i < top_k; i += NT) out[i] = i < ncand ? i : (i == ncand ? own : -1);
    return;
  }
  if (m == 0) {      // only the own block
    for (int i = tid; i < top_k; i += NT) out[i] = i == 0 ? own : -1;
    return;
  }
  const float* s = scores + (size_t)row * score_stride;
  uint64_t mx = 0;
  for (int j = tid; j < ncand; j += NT) {
    const uint64_t c = sel_key(s[j], j);
    mx = c > mx ? c : mx;
  }
  tmax[tid] = mx;
  if (tid == 0) n_surv = 0;
  __syncthreads();
  bitonic_desc(tmax, NT);
  const uint64_t tau = tmax[m - 1];
  for (int j = tid; j < ncand; j += NT) {
    const uint64_t c = sel_key(s[j], j);
    if (c >= tau) {
      const int slot = atomicAdd(&n_surv, 1);
      if (slot < surv_cap) surv[slot] = c;
    }
  }
  __syncthreads();
  const int ns = min(n_surv, surv_cap);
  int n2 = 64;
  while (n2 < ns) n2 <<= 1;
  for (int i = ns + tid; i < n2; i += NT) surv[i] = 0;
  __syncthreads();
  bitonic_desc(surv, n2);
  if (tid < m) kept[tid] = sel_key_index(surv[tid]);
  __syncthreads();
  if (tid < m) {
    const int ji = kept[tid];
    int rank = 0;
    for (int i = 0; i < m; i++) rank += kept[i] < ji ? 1 : 0;
    out[rank] = ji;
  }
  if (tid == 0) out[m] = own;
}

hipError_t launch_topk(const bsg_dims& d, const float* scores, int q_len, int score_stride, const int32_t* kv_lens,
                       int32_t* block_idx, hipStream_t stream) {
  const int rows = d.batch * d.num_kv_heads * q_len;
  const int m = d.top_k - 1;
  if (rows >= 2048 || score_stride <= 256) {
    dim3 grid((rows + 255) / 256);
#define BSG_TR(K)                                                                                          \
  hipLaunchKernelGGL(topk_rows_kernel<K>, grid, dim3(256), 0, stream, scores, kv_lens, block_idx, rows,     \
                     d.num_kv_heads, q_len, score_stride, d.page_size, d.top_k)
    if (m <= 4) BSG_TR(4);
    else if (m <= 8) BSG_TR(8);
    else if (m <= 16) BSG_TR(16);
    else if (m <= 32) BSG_TR(32);
    else BSG_TR(64);
#undef BSG_TR
  } else {
    constexpr int NT = 512;
    const int share = (score_stride + NT - 1) / NT;
    int cap = 64;
    while (cap < m * share) cap <<= 1;
    const size_t smem = (size_t)(NT + cap) * sizeof(uint64_t);
    if (smem > 150 * 1024) return hipErrorInvalidValue;
    {
      hipError_t ea = hipFuncSetAttribute((const void*)topk_wg_kernel<NT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                          (int)smem);
      if (ea != hipSuccess) return ea;
    }
    hipLaunchKernelGGL(topk_wg_kernel<NT>, dim3(rows), dim3(NT), smem, stream, scores, kv_lens, block_idx,
                       d.num_kv_heads, q_len, score_stride, d.page_size, d.top_k, cap);
  }
  return hipGetLastError();
}

}  // namespace bsg
