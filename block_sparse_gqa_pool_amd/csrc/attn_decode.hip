// Decode attention over the selected blocks (Ling 2.0 page, "Summarizing the Breakthrough":
// at decode only the top-k blocks are fetched), split over workgroups with a log-sum-exp
// merge.
//
// Pass 1: workgroup (split s, group g, sequence b) streams its share of the selected pages
// of (b, g) through LDS and keeps, for each of the G query heads of the group, the running
// max m, sum l and unnormalised output o[D].  It writes (m, l, o) to the workspace.
// Pass 2: one workgroup per (b, query head) merges the splits:
//     m* = max m_s,  l* = sum l_s e^(m_s - m*),  out = sum o_s e^(m_s - m*) / l*.
// The work is HBM-bound: each selected (page, head) K and V tile is read exactly once.
#include "bsg_device.h"
#include "bsg_internal.h"

namespace bsg {

namespace {
constexpr int DC_NACC = 8;  // per-thread outputs: G * D <= 256 * DC_NACC
}

template <typename T, int D, int BS>
__global__ __launch_bounds__(256) void attn_decode_split_kernel(
    const T* __restrict__ q, const int32_t* __restrict__ kv_lens, const T* __restrict__ k_cache,
    const T* __restrict__ v_cache, const int32_t* __restrict__ page_table, const int32_t* __restrict__ block_idx,
    float scale, float* __restrict__ ws, int Hq, int Hkv, int top_k, int num_pages, int pt_stride, int nsplit,
    int pps) {
  constexpr int KP = D + 2;   // padded K row (elements) so that row-strided reads spread over banks
  extern __shared__ __attribute__((aligned(16))) unsigned char dc_smem[];
  const int G = Hq / Hkv;
  float* qs = reinterpret_cast<float*>(dc_smem);        // [G][D]
  float* zs = qs + G * D;                                // [G][BS]  scores, then weights
  float* st = zs + G * BS;                               // [G][3]   m, l, alpha
  T* Ks = reinterpret_cast<T*>(st + G * 3 + 1);          // [BS][KP]
  T* Vs = Ks + BS * KP;                                  // [BS][D]

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = kv_lens[b];
  const int pos = L - 1;
  const int32_t* sl = block_idx + ((size_t)b * Hkv + g) * top_k;

  for (int e = tid; e < G * D; e += 256) qs[e] = ld_any(q + ((size_t)b * Hq + g * G) * D + e);
  for (int e = tid; e < G; e += 256) {
    st[3 * e + 0] = -INFINITY;
    st[3 * e + 1] = 0.0f;
    st[3 * e + 2] = 1.0f;
  }
  float acc[DC_NACC];
#pragma unroll
  for (int i = 0; i < DC_NACC; i++) acc[i] = 0.0f;
  __syncthreads();

  const int s0 = split * pps, s1 = min(s0 + pps, top_k);
  for (int si = s0; si < s1; si++) {
    const int j = sl[si];
    if (j < 0) break;
    const int jj = clampi(j, 0, pt_stride - 1);
    const int p = clampi(page_table[(size_t)b * pt_stride + jj], 0, num_pages - 1);
    const int nk = max(0, min(BS, pos - jj * BS + 1));
    const T* kp = k_cache + (((size_t)p * Hkv + g) * BS) * D;
    const T* vp = v_cache + (((size_t)p * Hkv + g) * BS) * D;
    for (int e = tid; e < BS * D; e += 256) {
      const int key = e / D, dd = e % D;
      const bool ok = key < nk;
      Ks[key * KP + dd] = ok ? kp[e] : (T)0;
      Vs[e] = ok ? vp[e] : (T)0;
    }
    __syncthreads();
    for (int e = tid; e < G * BS; e += 256) {
      const int hh = e / BS, key = e % BS;
      float z = -INFINITY;
      if (key < nk) {
        const float* qr = qs + hh * D;
        const T* kr = Ks + key * KP;
        float dot = 0.0f;
#pragma unroll 8
        for (int dd = 0; dd < D; dd++) dot = fmaf(qr[dd], ld_any(kr + dd), dot);
        z = dot * scale;
      }
      zs[e] = z;
    }
    __syncthreads();
    for (int hh = wave; hh < G; hh += 4) {
      float mx = -INFINITY;
      for (int key = lane; key < BS; key += 64) mx = fmaxf(mx, zs[hh * BS + key]);
      mx = wave_max(mx);
      const float m_old = st[3 * hh + 0];
      const float m_new = fmaxf(m_old, mx);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      float sum = 0.0f;
      for (int key = lane; key < BS; key += 64) {
        const float pz = __expf(zs[hh * BS + key] - m_use);
        zs[hh * BS + key] = pz;
        sum += pz;
      }
      sum = wave_sum(sum);
      if (lane == 0) {
        const float a = __expf(m_old - m_use);
        st[3 * hh + 0] = m_new;
        st[3 * hh + 1] = st[3 * hh + 1] * a + sum;
        st[3 * hh + 2] = a;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < DC_NACC; i++) {
      const int e = tid + 256 * i;
      if (e < G * D) {
        const int hh = e / D, dd = e % D;
        float a = acc[i] * st[3 * hh + 2];
        const float* pr = zs + hh * BS;
        for (int key = 0; key < nk; key++) a = fmaf(pr[key], ld_any(Vs + key * D + dd), a);
        acc[i] = a;
      }
    }
    __syncthreads();
  }
  float* wp = ws + (((size_t)b * Hkv + g) * nsplit + split) * G * (D + 2);
#pragma unroll
  for (int i = 0; i < DC_NACC; i++) {
    const int e = tid + 256 * i;
    if (e < G * D) wp[(e / D) * (D + 2) + 2 + (e % D)] = acc[i];
  }
  for (int hh = tid; hh < G; hh += 256) {
    wp[hh * (D + 2) + 0] = st[3 * hh + 0];
    wp[hh * (D + 2) + 1] = st[3 * hh + 1];
  }
}

template <typename T, int D>
__global__ __launch_bounds__(D) void attn_decode_merge_kernel(const float* __restrict__ ws, T* __restrict__ out,
                                                              float* __restrict__ lse, int Hq, int Hkv, int nsplit) {
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh % Hq;
  const int G = Hq / Hkv;
  const int g = h / G, hh = h % G;
  const int d = threadIdx.x;
  const float* base = ws + (((size_t)b * Hkv + g) * nsplit) * G * (D + 2) + (size_t)hh * (D + 2);
  const size_t sstride = (size_t)G * (D + 2);
  float m = -INFINITY;
  for (int s = 0; s < nsplit; s++) m = fmaxf(m, base[s * sstride]);
  float l = 0.0f, o = 0.0f;
  if (m != -INFINITY) {
    for (int s = 0; s < nsplit; s++) {
      const float ms = base[s * sstride];
      if (ms == -INFINITY) continue;
      const float w = __expf(ms - m);
      l += base[s * sstride + 1] * w;
      o += base[s * sstride + 2 + d] * w;
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  st_any(out + ((size_t)b * Hq + h) * D + d, o * inv);
  if (lse && d == 0) lse[(size_t)b * Hq + h] = m + logf(l);
}

int decode_num_splits(const bsg_dims& d) {
  long long units = (long long)d.batch * d.num_kv_heads;
  long long pps = (d.top_k * units + 512) / 1024;
  if (pps < 1) pps = 1;
  if (pps > d.top_k) pps = d.top_k;
  return (int)((d.top_k + pps - 1) / pps);
}

size_t decode_workspace_bytes(const bsg_dims& d) {
  const int G = d.num_q_heads / d.num_kv_heads;
  return (size_t)d.batch * d.num_kv_heads * decode_num_splits(d) * G * (d.head_dim + 2) * sizeof(float);
}

static size_t decode_smem(const bsg_dims& d, size_t elem) {
  const int G = d.num_q_heads / d.num_kv_heads;
  return (size_t)(G * d.head_dim + G * d.page_size + G * 3 + 1) * 4 +
         (size_t)d.page_size * (d.head_dim + 2) * elem + (size_t)d.page_size * d.head_dim * elem;
}

hipError_t launch_attn_decode(const bsg_dims& d, const void* q, const int32_t* kv_lens, const void* k_cache,
                              const void* v_cache, const int32_t* page_table, const int32_t* block_idx,
                              float scale, void* workspace, void* out, float* lse, hipStream_t stream) {
  const int nsplit = decode_num_splits(d);
  const int pps = (d.top_k + nsplit - 1) / nsplit;
  dim3 grid(nsplit, d.num_kv_heads, d.batch);
  float* ws = (float*)workspace;
#define BSG_DS(T, DD, BB)                                                                                       \
  do {                                                                                                          \
    const size_t smem = decode_smem(d, sizeof(T));                                                              \
    auto kfn = attn_decode_split_kernel<T, DD, BB>;                                                             \
    { hipError_t ea_ = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem); if (ea_ != hipSuccess) return ea_; }              \
    hipLaunchKernelGGL(kfn, grid, dim3(256), smem, stream, (const T*)q, kv_lens, (const T*)k_cache,              \
                       (const T*)v_cache, page_table, block_idx, scale, ws, d.num_q_heads, d.num_kv_heads,      \
                       d.top_k, d.num_pages, d.pt_stride, nsplit, pps);                                         \
  } while (0)
#define BSG_DS_D(T)                                                                        \
  do {                                                                                     \
    if (d.head_dim == 128) {                                                               \
      if (d.page_size == 64) BSG_DS(T, 128, 64); else BSG_DS(T, 128, 128);                 \
    } else {                                                                               \
      if (d.page_size == 64) BSG_DS(T, 64, 64); else BSG_DS(T, 64, 128);                   \
    }                                                                                      \
  } while (0)
  if (d.dtype == BSG_BF16) BSG_DS_D(bf16_t); else BSG_DS_D(float);
#undef BSG_DS_D
#undef BSG_DS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 mgrid(d.batch * d.num_q_heads);
  if (d.dtype == BSG_BF16) {
    if (d.head_dim == 128)
      hipLaunchKernelGGL((attn_decode_merge_kernel<bf16_t, 128>), mgrid, dim3(128), 0, stream, ws, (bf16_t*)out, lse,
                         d.num_q_heads, d.num_kv_heads, nsplit);
    else
      hipLaunchKernelGGL((attn_decode_merge_kernel<bf16_t, 64>), mgrid, dim3(64), 0, stream, ws, (bf16_t*)out, lse,
                         d.num_q_heads, d.num_kv_heads, nsplit);
  } else {
    if (d.head_dim == 128)
      hipLaunchKernelGGL((attn_decode_merge_kernel<float, 128>), mgrid, dim3(128), 0, stream, ws, (float*)out, lse,
                         d.num_q_heads, d.num_kv_heads, nsplit);
    else
      hipLaunchKernelGGL((attn_decode_merge_kernel<float, 64>), mgrid, dim3(64), 0, stream, ws, (float*)out, lse,
                         d.num_q_heads, d.num_kv_heads, nsplit);
  }
  return hipGetLastError();
}

}  // namespace bsg
