// Fused prefill scoring + causal top-k selection (no materialised scores).
//
// Scores follow the Ling 2.0 page, "Summarizing the Breakthrough" (one selection per GQA
// group) and the MSA post, second paragraph (blocks scored per group); the selection is
// exp-free (MSA post, third paragraph).
//
// A workgroup (4 waves) takes 128 query tokens of one (sequence, group); each wave owns 32
// tokens.  The group-summed query (fp32) is split into three bf16 terms hi + mid + lo
// (exact to ~2^-24 relative), so that bf16 matrix-core products of the terms with the bf16
// block representatives reproduce the fp32 score to fp32 rounding:
//
//   S^T (32 blocks x 32 tokens) = R (blocks x D) . (hi + mid + lo)^T (D x tokens)
//
// The transposed product gives each lane 16 candidate scores of ONE token per chunk of 32
// blocks (lanes l and l + 32 split a token's candidates), so each lane keeps a sorted
// register list of its best candidates by the 64-bit key (score, then lower index), with a
// threshold test before any insertion.  At the end the two half-lists of a token are merged
// through LDS, the own block is appended and the kept ids are written ascending.
#include "bsg_device.h"
#include "bsg_internal.h"

namespace bsg {

namespace {
constexpr int FS_TOK = 128;   // tokens per workgroup (32 per wave)
constexpr int FS_CH = 32;     // candidate blocks per chunk
constexpr int FS_PAD = 8;     // LDS row padding (bf16 elements)
}  // namespace

__device__ __forceinline__ __bf16 to_bf16_rne(float f) {
  const bf16_t b = f32_to_bf16(f);
  return *reinterpret_cast<const __bf16*>(&b);
}

template <int D, int KCAP>
__global__ __launch_bounds__(256, (KCAP > 32 ? 1 : 2)) void score_topk_fused_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ kv_lens, const bf16_t* __restrict__ block_cache,
    const int32_t* __restrict__ page_table, int32_t* __restrict__ block_idx, int q_len, int Hq, int Hkv, int bs,
    int top_k, int num_pages, int pt_stride) {
  constexpr int NDS = D / 16;
  constexpr int RS = D + FS_PAD;
  __shared__ __attribute__((aligned(16))) bf16_t reps[2][FS_CH * RS];
  extern __shared__ __attribute__((aligned(16))) uint64_t fs_lists[];   // [256][KCAP] merge scratch

  const int G = Hq / Hkv;
  const int g = blockIdx.y, b = blockIdx.z;
  const int t0 = blockIdx.x * FS_TOK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int L = kv_lens[b];
  const int t = t0 + wave * 32 + col;
  const bool row_ok = t < q_len;
  const int own = max(L - q_len + t, 0) / bs;
  const int ncand = row_ok ? min(own, pt_stride) : 0;
  const int tlast = min(t0 + FS_TOK, q_len) - 1;
  const int nc_max = min(max(L - q_len + tlast, 0) / bs, pt_stride);   // candidates of the tile's last token

  // group-summed query, split into three bf16 terms (B operand: k = d, n = token)
  bf16x8_t qh[NDS], qm[NDS], ql[NDS];
  {
    float acc[NDS][8];
#pragma unroll
    for (int ks = 0; ks < NDS; ks++)
#pragma unroll
      for (int i = 0; i < 8; i++) acc[ks][i] = 0.0f;
    if (row_ok) {
      const bf16_t* qp = q + (((size_t)b * Hq + (size_t)g * G) * q_len + t) * D + 8 * half;
      for (int hh = 0; hh < G; hh++) {
        const bf16_t* qr = qp + (size_t)hh * q_len * D;
#pragma unroll
        for (int ks = 0; ks < NDS; ks++) {
          const uint4 v = *reinterpret_cast<const uint4*>(qr + 16 * ks);
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int i = 0; i < 8; i++)
            acc[ks][i] += bf16_to_f32((bf16_t)((i & 1) ? (w4[i >> 1] >> 16) : (w4[i >> 1] & 0xffffu)));
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < NDS; ks++)
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float x = acc[ks][i];
        const __bf16 h = to_bf16_rne(x);
        const float r1 = x - (float)h;
        const __bf16 m = to_bf16_rne(r1);
        const float r2 = r1 - (float)m;
        qh[ks][i] = h;
        qm[ks][i] = m;
        ql[ks][i] = to_bf16_rne(r2);
      }
  }

  uint64_t best[KCAP];
#pragma unroll
  for (int i = 0; i < KCAP; i++) best[i] = 0;

  // chunk loader: 32 representatives x D bf16 into LDS (zeros past the tile's candidates)
  auto load_chunk = [&](int c, int buf) {
    constexpr int CPR = D / 8;  // 16-byte pieces per row
    for (int e = tid; e < FS_CH * CPR; e += 256) {
      const int r = e / CPR, piece = e % CPR;
      const int j = c * FS_CH + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j < nc_max) {
        const int p = clampi(page_table[(size_t)b * pt_stride + j], 0, num_pages - 1);
        v = *reinterpret_cast<const uint4*>(block_cache + ((size_t)p * Hkv + g) * D + 8 * piece);
      }
      *reinterpret_cast<uint4*>(&reps[buf][r * RS + 8 * piece]) = v;
    }
  };

  const int nchunks = (nc_max + FS_CH - 1) / FS_CH;
  if (nchunks > 0) load_chunk(0, 0);
  for (int c = 0; c < nchunks; c++) {
    __syncthreads();                               // chunk c is in LDS; buffer (c+1)&1 is free
    if (c + 1 < nchunks) load_chunk(c + 1, (c + 1) & 1);
    const bf16_t* R = reps[c & 1];
    const int jbase = c * FS_CH;
    if (__ballot(jbase < ncand) != 0) {       // some token of this wave has candidates here
      f32x16_t s;
#pragma unroll
      for (int e = 0; e < 16; e++) s[e] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < NDS; ks++) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(R + col * RS + 16 * ks + 8 * half);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qh[ks], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qm[ks], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ql[ks], s, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int j = jbase + 8 * (e >> 2) + 4 * half + (e & 3);
        if (j < ncand) {
          uint64_t key = sel_key(s[e], j);
          if (key > best[KCAP - 1]) {
#pragma unroll
            for (int i = 0; i < KCAP; i++) {
              const uint64_t bi = best[i];
              const bool gt = key > bi;
              best[i] = gt ? key : bi;
              key = gt ? bi : key;
            }
          }
        }
      }
    }
  }

  // merge the two half-lists of each token, append the own block, write ascending
  uint64_t* mine = fs_lists + (size_t)tid * KCAP;
#pragma unroll
  for (int i = 0; i < KCAP; i++) mine[i] = best[i];
  __syncthreads();
  if (half == 0 && row_ok) {
    const uint64_t* A = mine;
    const uint64_t* Bl = fs_lists + (size_t)(tid + 32) * KCAP;
    const int m = top_k - 1;
    const int cnt = min(m, ncand);
    int ia = 0, ib = 0;
    int32_t* out = block_idx + (((size_t)b * Hkv + g) * q_len + t) * top_k;
    // take the cnt largest keys (all distinct); A and B are sorted descending
    int ids[KCAP];
#pragma unroll
    for (int i = 0; i < KCAP; i++) ids[i] = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < KCAP; i++) {
      if (i < cnt) {
        const uint64_t ka = ia < KCAP ? A[ia] : 0, kb = ib < KCAP ? Bl[ib] : 0;
        const bool ta = ka > kb;
        ids[i] = sel_key_index(ta ? ka : kb);
        ia += ta ? 1 : 0;
        ib += ta ? 0 : 1;
      }
    }
#pragma unroll
    for (int i = 0; i < KCAP; i++) {
      if (i < cnt) {
        int rank = 0;
#pragma unroll
        for (int i2 = 0; i2 < KCAP; i2++) rank += (i2 < cnt && ids[i2] < ids[i]) ? 1 : 0;
        out[rank] = ids[i];
      }
    }
    out[cnt] = own;
    for (int i = cnt + 1; i < top_k; i++) out[i] = -1;
  }
}

bool group_score_topk_fused_supported(const bsg_dims& d, int q_len) {
  return d.dtype == BSG_BF16 && q_len >= 32 && d.top_k <= 65;
}

hipError_t launch_group_score_topk_fused(const bsg_dims& d, const void* q, int q_len, const int32_t* kv_lens,
                                         const void* block_cache, const int32_t* page_table, int32_t* block_idx,
                                         hipStream_t stream) {
  dim3 grid((q_len + FS_TOK - 1) / FS_TOK, d.num_kv_heads, d.batch);
  const int m = d.top_k - 1;
#define BSG_FS(DD, K)                                                                                          \
  do {                                                                                                         \
    const size_t smem = (size_t)256 * (K) * sizeof(uint64_t);                                                  \
    auto kfn = score_topk_fused_kernel<DD, K>;                                                                 \
    hipError_t ea = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem); \
    if (ea != hipSuccess) return ea;                                                                           \
    hipLaunchKernelGGL(kfn, grid, dim3(256), smem, stream, (const bf16_t*)q, kv_lens, (const bf16_t*)block_cache, \
                       page_table, block_idx, q_len, d.num_q_heads, d.num_kv_heads, d.page_size, d.top_k,        \
                       d.num_pages, d.pt_stride);                                                              \
  } while (0)
#define BSG_FS_K(DD)                        \
  do {                                      \
    if (m <= 4) BSG_FS(DD, 4);              \
    else if (m <= 8) BSG_FS(DD, 8);         \
    else if (m <= 16) BSG_FS(DD, 16);       \
    else if (m <= 32) BSG_FS(DD, 32);       \
    else BSG_FS(DD, 64);                    \
  } while (0)
  if (d.head_dim == 128) BSG_FS_K(128); else BSG_FS_K(64);
#undef BSG_FS_K
#undef BSG_FS
  return hipGetLastError();
}

}  // namespace bsg
