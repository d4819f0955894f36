// Exact attention over the selected blocks ("Sparse Attention + Linear Backbones", section
// 5.5: softmax(q.k/sqrt(d)) over the selected keys times their values; "Sparse Attention for
// Long-Context LLMs", section 4.3: the top-k mask removes the other keys, so they are
// skipped rather than masked).  Causal inside the own block.
//
// bf16 path (matrix cores, gfx950 v_mfma_f32_32x32x16_bf16)
// ---------------------------------------------------------
// A workgroup (4 waves) owns 128 query rows = TT tokens x HG heads of one GQA group.  It
// builds the union of its tokens' selected blocks (ascending) and streams those blocks'
// K and V tiles through LDS once; every wave runs the blocks that any of its rows selected
// and skips the others.  Per wave, 32 query rows:
//
//   S^T (keys x rows) = K (keys x D) . Q^T (D x rows)       A = K rows from LDS, B = Q regs
//   O^T (D x rows)   += V^T (D x keys) . P^T (keys x rows)   A = V^T via ds_read_b64_tr_b16,
//                                                           B = P^T straight from S^T regs
//
// Computing the transposed product puts each query row in one lane column, so the
// online-softmax state (max, sum, rescale) is per lane and the probabilities are already in
// the B-operand layout of the second product.  The K rows are fed to the first product in a
// permuted order so that a lane's 8 consecutive accumulator entries belong to 8 consecutive
// keys, which is the k-ordering the second product needs.
//
// fp32 path: one wave per query row, VALU dot products, same online softmax.
#include "bsg_device.h"
#include "bsg_internal.h"

namespace bsg {

namespace {
constexpr int PF_ROWS = 128;   // query rows per workgroup
constexpr int PF_KPAD = 8;     // K row padding (bf16 elements) in LDS
constexpr int PF_VPAD = 16;    // V row padding (bf16 elements) in LDS
constexpr float LOG2E = 1.4426950408889634f;
}  // namespace

typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr;

// Key (row of the K tile) that feeds accumulator row m of a 32-key chunk.
__device__ __forceinline__ int perm_key(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

template <int D, int BS>
__global__ __launch_bounds__(256, 2) void attn_prefill_mfma_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ kv_lens, const bf16_t* __restrict__ k_cache,
    const bf16_t* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ block_idx, float scale, bf16_t* __restrict__ out, float* __restrict__ lse,
    int q_len, int Hq, int Hkv, int HG, int top_k, int num_pages, int pt_stride) {
  constexpr int KS = D + PF_KPAD;  // LDS row strides (elements)
  constexpr int VS = D + PF_VPAD;
  constexpr int NKC = BS / 32;     // 32-key chunks per block
  constexpr int NDS = D / 16;      // k-steps of the first product
  constexpr int NDC = D / 32;      // 32-wide d chunks of the output
  extern __shared__ __attribute__((aligned(16))) unsigned char pf_smem[];
  bf16_t* Ks = reinterpret_cast<bf16_t*>(pf_smem);
  bf16_t* Vs = Ks + BS * KS;
  const int TT = PF_ROWS / HG;
  int32_t* sel = reinterpret_cast<int32_t*>(Vs + BS * VS);   // [TT][top_k]
  const int nbw = (pt_stride + 31) >> 5;
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(sel + TT * top_k);  // [nbw]
  int32_t* ulist = reinterpret_cast<int32_t*>(bitmap + nbw);        // [min(TT*top_k, pt_stride)]
  __shared__ int wsum[8];
  __shared__ int n_union;

  const int G = Hq / Hkv;
  const int slices = G / HG;
  const int g = blockIdx.y / slices;
  const int hs = blockIdx.y % slices;
  const int b = blockIdx.z;
  const int t0 = blockIdx.x * TT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int L = kv_lens[b];
  const int base_pos = L - q_len;

  // ---- selections of the tile's tokens and their union (ascending block ids)
  for (int e = tid; e < TT * top_k; e += 256) {
    const int tt = e / top_k, s = e % top_k;
    const int t = t0 + tt;
    int j = -1;
    if (t < q_len) j = block_idx[(((size_t)b * Hkv + g) * q_len + t) * top_k + s];
    sel[e] = (j >= 0 && j < pt_stride) ? j : (j >= pt_stride ? pt_stride - 1 : -1);
  }
  for (int w = tid; w < nbw; w += 256) bitmap[w] = 0u;
  __syncthreads();
  for (int e = tid; e < TT * top_k; e += 256) {
    const int j = sel[e];
    if (j >= 0) atomicOr(&bitmap[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  {
    // exclusive scan of per-word popcounts; each thread owns a contiguous run of words
    const int per = (nbw + 255) / 256;
    const int w0 = tid * per, w1 = min(w0 + per, nbw);
    int cnt = 0;
    for (int w = w0; w < w1; w++) cnt += __popc(bitmap[w]);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int off = incl - cnt;
    for (int w2 = 0; w2 < wave; w2++) off += wsum[w2];
    if (tid == 255) n_union = off + cnt;
    for (int w = w0; w < w1; w++) {
      uint32_t bits = bitmap[w];
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1;
        ulist[off++] = (w << 5) + bit;
      }
    }
  }
  __syncthreads();
  const int U = n_union;

  // ---- this lane's query row
  const int col = lane & 31;          // row within the wave's 32
  const int half = lane >> 5;
  const int r = wave * 32 + col;
  const int tt = r / HG;
  const int h = g * G + hs * HG + (r % HG);
  const int t = t0 + tt;
  const bool row_ok = t < q_len;
  const int pos = base_pos + t;
  const int own = pos / BS;
  int sp = 0;                          // cursor into this token's ascending selection
  const int32_t* mysel = sel + tt * top_k;

  bf16x8_t qb[NDS];
  {
    const bf16_t* qp = q + (((size_t)b * Hq + h) * q_len + (row_ok ? t : 0)) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < NDS; ks++) {
      uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qp + 16 * ks) : make_uint4(0, 0, 0, 0);
      qb[ks] = *reinterpret_cast<bf16x8_t*>(&v);
    }
  }
  const float c2 = scale * LOG2E;
  float m_i = -INFINITY;  // running max of raw scores
  float l_i = 0.0f;       // this lane's share of the running sum
  f32x16_t o[NDC];
#pragma unroll
  for (int i = 0; i < NDC; i++)
#pragma unroll
    for (int e = 0; e < 16; e++) o[i][e] = 0.0f;

  // LDS read addresses (elements)
  const int kread = perm_key(col) * KS + 8 * half;
  const int qd = lane >> 4, ep = (lane & 15) >> 2, s4 = lane & 3;
  const int vread = (8 * (qd >> 1) + ep) * VS + 16 * (qd & 1) + 4 * s4;

  for (int u = 0; u < U; u++) {
    const int j = ulist[u];
    const int p = clampi(page_table[(size_t)b * pt_stride + j], 0, num_pages - 1);
    const int nvalid = min(BS, L - j * BS);  // tokens of this block that exist
    __syncthreads();                          // previous tiles fully consumed
    {
      const bf16_t* kp = k_cache + (((size_t)p * Hkv + g) * BS) * D;
      const bf16_t* vp = v_cache + (((size_t)p * Hkv + g) * BS) * D;
      constexpr int CH = D / 8;   // 16-byte chunks per row
#pragma unroll
      for (int e0 = 0; e0 < BS * CH; e0 += 256) {
        const int e = e0 + tid;
        const int key = e / CH, c = e % CH;
        uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (key < nvalid) {
          kv = *reinterpret_cast<const uint4*>(kp + (size_t)key * D + 8 * c);
          vv = *reinterpret_cast<const uint4*>(vp + (size_t)key * D + 8 * c);
        }
        *reinterpret_cast<uint4*>(Ks + key * KS + 8 * c) = kv;
        *reinterpret_cast<uint4*>(Vs + key * VS + 8 * c) = vv;
      }
    }
    __syncthreads();
    bool mine = false;
    if (row_ok && sp < top_k && mysel[sp] == j) {
      mine = true;
      sp++;
    }
    if (__ballot(mine) == 0) continue;   // no row of this wave selected block j

    // ---- S^T = K . Q^T
    f32x16_t sacc[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; kc++) {
#pragma unroll
      for (int e = 0; e < 16; e++) sacc[kc][e] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < NDS; ks++) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(Ks + kread + kc * 32 * KS + 16 * ks);
        sacc[kc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], sacc[kc], 0, 0, 0);
      }
    }
    // ---- mask, online softmax
    const int klim = mine ? min(pos - j * BS, BS - 1) : -1;   // last key index allowed
    float mx = -INFINITY;
#pragma unroll
    for (int kc = 0; kc < NKC; kc++)
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int key = kc * 32 + 16 * (e >> 3) + 8 * half + (e & 7);
        const float s = key <= klim ? sacc[kc][e] : -INFINITY;
        sacc[kc][e] = s;
        mx = fmaxf(mx, s);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_i, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = exp2f((m_i - m_use) * c2);
    m_i = m_new;
    const float mc = m_use * c2;
    float rs = 0.0f;
#pragma unroll
    for (int kc = 0; kc < NKC; kc++)
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const float pe = exp2f(fmaf(sacc[kc][e], c2, -mc));
        sacc[kc][e] = pe;
        rs += pe;
      }
    l_i = l_i * alpha + rs;
#pragma unroll
    for (int i = 0; i < NDC; i++)
#pragma unroll
      for (int e = 0; e < 16; e++) o[i][e] *= alpha;

    // ---- O^T += V^T . P^T
#pragma unroll
    for (int st = 0; st < BS / 16; st++) {
      const int kc = st >> 1, hh = st & 1;
      bf16x8_t pb;
#pragma unroll
      for (int i = 0; i < 8; i++) pb[i] = (__bf16)sacc[kc][8 * hh + i];
#pragma unroll
      for (int dc = 0; dc < NDC; dc++) {
        const bf16_t* vbase = Vs + vread + (16 * st) * VS + 32 * dc;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vbase));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vbase + 4 * VS));
        bf16x8_t va;
        *reinterpret_cast<s16x4_t*>(&va) = lo;
        *(reinterpret_cast<s16x4_t*>(&va) + 1) = hi;
        o[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[dc], 0, 0, 0);
      }
    }
  }

  // ---- epilogue
  const float l = l_i + __shfl_xor(l_i, 32, 64);
  if (!row_ok) return;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  bf16_t* op = out + (((size_t)b * Hq + h) * q_len + t) * D;
#pragma unroll
  for (int dc = 0; dc < NDC; dc++)
#pragma unroll
    for (int e4 = 0; e4 < 4; e4++) {
      const int d0 = 32 * dc + 8 * e4 + 4 * half;
      uint2 w;
      w.x = pack_bf16x2(o[dc][4 * e4 + 0] * inv, o[dc][4 * e4 + 1] * inv);
      w.y = pack_bf16x2(o[dc][4 * e4 + 2] * inv, o[dc][4 * e4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + d0) = w;
    }
  if (lse && half == 0) lse[((size_t)b * Hq + h) * q_len + t] = m_i * scale + logf(l);
}

// ---------------------------------------------------------------------------------------
// VALU path (fp32 inputs, or shapes the matrix-core path does not cover): one wave per
// (sequence, head, query), lanes split D, online softmax over the selected keys.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_prefill_valu_kernel(
    const T* __restrict__ q, const int32_t* __restrict__ kv_lens, const T* __restrict__ k_cache,
    const T* __restrict__ v_cache, const int32_t* __restrict__ page_table, const int32_t* __restrict__ block_idx,
    float scale, T* __restrict__ out, float* __restrict__ lse, int q_len, int Hq, int Hkv, int bs, int top_k,
    int num_pages, int pt_stride, long long rows) {
  constexpr int DPL = D / 64;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int t = (int)(row % q_len);
  const int h = (int)((row / q_len) % Hq);
  const int b = (int)(row / ((long long)q_len * Hq));
  const int G = Hq / Hkv;
  const int g = h / G;
  const int L = kv_lens[b];
  const int pos = L - q_len + t;
  const T* qp = q + (((size_t)b * Hq + h) * q_len + t) * D;
  float qv[DPL], acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; i++) {
    qv[i] = (float)ld_any(qp + lane + 64 * i);
    acc[i] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  const int32_t* sl = block_idx + (((size_t)b * Hkv + g) * q_len + t) * top_k;
  for (int s = 0; s < top_k; s++) {
    const int j = sl[s];
    if (j < 0) break;
    const int jj = clampi(j, 0, pt_stride - 1);
    const int p = clampi(page_table[(size_t)b * pt_stride + jj], 0, num_pages - 1);
    const int nk = min(bs, pos - jj * bs + 1);
    const T* kp = k_cache + (((size_t)p * Hkv + g) * bs) * D;
    const T* vp = v_cache + (((size_t)p * Hkv + g) * bs) * D;
    for (int key = 0; key < nk; key++) {
      float dot = 0.0f;
#pragma unroll
      for (int i = 0; i < DPL; i++) dot = fmaf(qv[i], (float)ld_any(kp + (size_t)key * D + lane + 64 * i), dot);
      dot = wave_sum(dot);
      const float z = dot * scale;
      const float mn = fmaxf(m, z);
      const float a = __expf(m - mn);
      const float pz = __expf(z - mn);
      l = l * a + pz;
#pragma unroll
      for (int i = 0; i < DPL; i++) acc[i] = acc[i] * a + pz * (float)ld_any(vp + (size_t)key * D + lane + 64 * i);
      m = mn;
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  T* op = out + (((size_t)b * Hq + h) * q_len + t) * D;
#pragma unroll
  for (int i = 0; i < DPL; i++) st_any(op + lane + 64 * i, acc[i] * inv);
  if (lse && lane == 0) lse[((size_t)b * Hq + h) * q_len + t] = m + logf(l);
}

static int mfma_heads_per_tile(int G) {
  // largest power of two dividing G, capped at 32 (a wave holds 32 rows)
  int hg = 1;
  while (hg < 32 && (G % (hg * 2)) == 0) hg *= 2;
  return hg;
}

static size_t mfma_smem_bytes(const bsg_dims& d, int HG) {
  const int D = d.head_dim, BS = d.page_size;
  const int TT = PF_ROWS / HG;
  const int nbw = (d.pt_stride + 31) / 32;
  const int ucap = TT * d.top_k < d.pt_stride ? TT * d.top_k : d.pt_stride;
  return (size_t)BS * (D + PF_KPAD) * 2 + (size_t)BS * (D + PF_VPAD) * 2 + (size_t)TT * d.top_k * 4 +
         (size_t)nbw * 4 + (size_t)ucap * 4;
}

hipError_t launch_attn_prefill(const bsg_dims& d, const void* q, int q_len, const int32_t* kv_lens,
                               const void* k_cache, const void* v_cache, const int32_t* page_table,
                               const int32_t* block_idx, float scale, void* out, float* lse,
                               hipStream_t stream) {
  const int G = d.num_q_heads / d.num_kv_heads;
  if (d.dtype == BSG_BF16) {
    const int HG = mfma_heads_per_tile(G);
    const size_t smem = mfma_smem_bytes(d, HG);
    if (smem <= 160 * 1024) {
      const int TT = PF_ROWS / HG;
      dim3 grid((q_len + TT - 1) / TT, d.num_kv_heads * (G / HG), d.batch);
#define BSG_PF(DD, BB)                                                                                       \
  do {                                                                                                        \
    auto kfn = attn_prefill_mfma_kernel<DD, BB>;                                                              \
    { hipError_t ea_ = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem); if (ea_ != hipSuccess) return ea_; }            \
    hipLaunchKernelGGL(kfn, grid, dim3(256), smem, stream, (const bf16_t*)q, kv_lens, (const bf16_t*)k_cache, \
                       (const bf16_t*)v_cache, page_table, block_idx, scale, (bf16_t*)out, lse, q_len,         \
                       d.num_q_heads, d.num_kv_heads, HG, d.top_k, d.num_pages, d.pt_stride);                   \
  } while (0)
      if (d.head_dim == 128) {
        if (d.page_size == 64) BSG_PF(128, 64); else BSG_PF(128, 128);
      } else {
        if (d.page_size == 64) BSG_PF(64, 64); else BSG_PF(64, 128);
      }
#undef BSG_PF
      return hipGetLastError();
    }
  }
  const long long rows = (long long)d.batch * d.num_q_heads * q_len;
  dim3 grid((unsigned)((rows + 3) / 4));
#define BSG_PV(T, DD)                                                                                          \
  hipLaunchKernelGGL((attn_prefill_valu_kernel<T, DD>), grid, dim3(256), 0, stream, (const T*)q, kv_lens,       \
                     (const T*)k_cache, (const T*)v_cache, page_table, block_idx, scale, (T*)out, lse, q_len,   \
                     d.num_q_heads, d.num_kv_heads, d.page_size, d.top_k, d.num_pages, d.pt_stride, rows)
  if (d.dtype == BSG_BF16) {
    if (d.head_dim == 128) BSG_PV(bf16_t, 128); else BSG_PV(bf16_t, 64);
  } else {
    if (d.head_dim == 128) BSG_PV(float, 128); else BSG_PV(float, 64);
  }
#undef BSG_PV
  return hipGetLastError();
}

}  // namespace bsg
