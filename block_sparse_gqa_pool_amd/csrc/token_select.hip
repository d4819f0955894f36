// Token-level and two-level selection for decode (q_len = 1).
//
// Token level ("Sparse Attention + Linear Backbones", sections 5.1-5.3 and the pseudocode of
// 5.5: an indexer scores every earlier position and the top-K positions are kept; the
// indexer uses no positional encoding).  The learned indexer is absent, so the index is the
// identity one: score(s) = sum over the group's heads h of q_h . k_s, the block score at
// granularity one.  Two level ("Sparse Attention for Long-Context LLMs", section 8: coarse
// then fine filtering): the candidates are the tokens of the row's selected blocks.
//
//  * token_score_kernel: one workgroup per (64 candidates, 4 groups, sequence).  The
//    group-summed queries are built in LDS; each group's 64 key rows (one page, D bf16 each)
//    are read with 16-byte loads, SEG = D/8 lanes per row, all loads of the workgroup in
//    flight together, and reduced with DPP moves.  Candidates past the query's
//    position (or in an unused block slot) get -inf.  HBM-bound: at token level it reads the
//    whole K cache of the sequence once (the pages' caveat: sparse attention cuts compute,
//    not necessarily memory traffic).
//  * token_topk_kernel: one workgroup of 1024 threads per (sequence, group) selects the top K
//    of the row's candidates exactly, by (score, lower index first).  A three-level radix
//    select on the 32-bit order key (11 + 11 + 10 bits; LDS histograms: the first level, where
//    every candidate falls into a few crowded bins, in 16 copies picked by lane; the later
//    levels, with few keys under the chosen prefix, merge equal bins within a wave before the
//    LDS atomic) finds the K-th key tau; a compaction pass in index
//    order keeps every key above tau and the first K - #above keys equal to tau, and writes
//    the kept tokens ascending (-1 padded).  Rows of at most 4096 candidates (the two-level
//    rows) take token_topk_small_kernel: the same steps with 256 threads holding the keys in
//    registers and one histogram.
#include "bsg_device.h"
#include "bsg_internal.h"

namespace bsg {

namespace {
constexpr int TS_CH = 64;      // candidates per score workgroup
constexpr int TS_HPW = 4;      // KV heads per score workgroup
constexpr int TK_NT = 1024;    // threads of the selection workgroup
constexpr int TK_NW = TK_NT / 64;
constexpr int TK_BINS = 2048;  // radix bins per level (11 bits)
constexpr int TK_UNR = 8;      // row tiles (4 scores per thread each) loaded per batch
constexpr int TK_COPIES = 16;  // level-1 histogram copies (lane % 16): few lanes meet on one entry
constexpr int TKS_NT = 256;    // threads of the short-row selection workgroup
}  // namespace

// Token of candidate c of row (b, g): two level, slot c % BS of block block_idx[c / BS];
// else token c.  -1 if the candidate does not exist.
template <int BS, bool TWO>
__device__ __forceinline__ int cand_token(int c, const int32_t* __restrict__ brow) {
  if constexpr (TWO) {
    const int j = brow[c / BS];
    return j < 0 ? -1 : j * BS + c % BS;
  } else {
    return c;
  }
}

template <int D, int BS, bool TWO>
__global__ __launch_bounds__(256) void token_score_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ kv_lens, const bf16_t* __restrict__ k_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ block_idx, int kblk,
    float* __restrict__ scores, int nc, int Hq, int Hkv, int num_pages, int pt_stride) {
  static_assert(BS % TS_CH == 0, "a chunk lies in one page");
  constexpr int SEG = D / 8;                       // lanes per key row
  constexpr int PPH = TS_CH * SEG;                 // 16-byte pieces per head
  constexpr int NP = TS_HPW * PPH / 256;           // pieces per thread
  __shared__ float qs[TS_HPW][D];
  const int c0 = blockIdx.x * TS_CH, g0 = blockIdx.y * TS_HPW, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int G = Hq / Hkv;
  const int pos = kv_lens[b] - 1;
  // per head of this workgroup: the chunk's first token and key rows (a chunk is 64
  // consecutive tokens of one block; at token level the same block for every head)
  int tok0[TS_HPW];
  const bf16_t* rows[TS_HPW];
#pragma unroll
  for (int hh = 0; hh < TS_HPW; hh++) {
    const int g = g0 + hh;
    const int32_t* brow = TWO ? block_idx + ((size_t)b * Hkv + min(g, Hkv - 1)) * kblk : nullptr;
    const int t0 = g < Hkv ? cand_token<BS, TWO>(c0, brow) : -1;
    const int j = t0 >= 0 ? t0 / BS : -1;
    const bool live = j >= 0 && j < pt_stride && t0 <= pos;
    const int p = live ? clampi(page_table[(size_t)b * pt_stride + j], 0, num_pages - 1) : 0;
    tok0[hh] = live ? t0 : -1;
    rows[hh] = k_cache + (((size_t)p * Hkv + (live ? g : 0)) * BS + (live ? t0 % BS : 0)) * D;
  }
  uint4 raw[NP];
#pragma unroll
  for (int u = 0; u < NP; u++) {
    const int pi = u * 256 + tid;
    const int hh = pi / PPH;
    raw[u] = tok0[hh] >= 0 ? *reinterpret_cast<const uint4*>(rows[hh] + (size_t)(pi % PPH) * 8)
                           : make_uint4(0, 0, 0, 0);
  }
  // group-summed queries (fp32, heads in order), 8 dims per thread from 16-byte loads
  if (tid < TS_HPW * (D / 8)) {
    const int hh = tid / (D / 8), d0 = 8 * (tid % (D / 8)), g = g0 + hh;
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (g < Hkv)
      for (int h = 0; h < G; h++) {
        const uint4 v = *reinterpret_cast<const uint4*>(q + ((size_t)b * Hq + g * G + h) * D + d0);
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
          acc[2 * i] += __uint_as_float(wd[i] << 16);
          acc[2 * i + 1] += __uint_as_float(wd[i] & 0xffff0000u);
        }
      }
#pragma unroll
    for (int i = 0; i < 8; i++) qs[hh][d0 + i] = acc[i];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NP; u++) {
    const int pi = u * 256 + tid;
    const int hh = pi / PPH, r = (pi % PPH) / SEG, w = pi % SEG;
    const float* qv = &qs[hh][w * 8];
    const uint32_t wd[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      s = fmaf(qv[2 * i], __uint_as_float(wd[i] << 16), s);
      s = fmaf(qv[2 * i + 1], __uint_as_float(wd[i] & 0xffff0000u), s);
    }
    s = seg_sum_dpp<SEG>(s);
    const int g = g0 + hh;
    if ((lane % SEG) == 0 && g < Hkv)
      scores[((size_t)b * Hkv + g) * nc + c0 + r] = (tok0[hh] >= 0 && tok0[hh] + r <= pos) ? s : -INFINITY;
  }
}

// Selection key: the order key of a finite score, 0 for a non-candidate (-inf).  Finite
// scores map to keys >= 0x00800000, so 0 sorts below every candidate.
__device__ __forceinline__ uint32_t tk_key(float s) { return s == -INFINITY ? 0u : order_key(s); }

// Add one to hist[bin] for every active lane, merging lanes of the wave that share a bin.
__device__ __forceinline__ void tk_hist_add(uint32_t* hist, int bin, bool active) {
  uint64_t act = __ballot(active);
  while (act) {
    const int leader = __ffsll((unsigned long long)act) - 1;
    const int lb = __shfl(bin, leader, 64);
    const uint64_t same = __ballot(active && bin == lb);
    if ((int)(threadIdx.x & 63) == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(same));
    active = active && bin != lb;
    act &= ~same;
  }
}

// Exclusive prefix sum over the workgroup of NW waves (thread order); returns this thread's
// offset and the total in *tot.  Uses red[NW + 1].
template <int NW>
__device__ __forceinline__ uint32_t tk_scan(uint32_t v, uint32_t* red, uint32_t* tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  uint32_t base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; w++) {
    const uint32_t t = red[w];
    base += w < wave ? t : 0u;
    all += t;
  }
  __syncthreads();
  *tot = all;
  return base + incl - v;
}

template <int BS, bool TWO>
__global__ __launch_bounds__(TK_NT) void token_topk_kernel(const float* __restrict__ scores, int nc, int K,
                                                          const int32_t* __restrict__ block_idx, int kblk,
                                                          int32_t* __restrict__ token_idx, int Hkv) {
  extern __shared__ uint32_t hcopy[];              // level 1: TK_BINS bins x TK_COPIES copies
  __shared__ uint32_t hist[TK_BINS];
  __shared__ uint32_t red[TK_NW + 1];
  __shared__ uint32_t sel_s[3];                    // digit, count above the digit, count in it
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const float* row = scores + ((size_t)b * Hkv + g) * nc;
  const int32_t* brow = TWO ? block_idx + ((size_t)b * Hkv + g) * kblk : nullptr;
  int32_t* orow = token_idx + ((size_t)b * Hkv + g) * K;
  // TK_UNR tiles of the row from cb on, 4 scores per thread per tile, all loads in flight
  // together (-inf past the row; nc is a multiple of 64)
  auto load_batch = [&](int cb, float4* v) {
#pragma unroll
    for (int u = 0; u < TK_UNR; u++) {
      const int c = cb + u * 4 * TK_NT + 4 * tid;
      v[u] = c < nc ? *reinterpret_cast<const float4*>(row + c) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
  };
  // ---- radix select of the K-th largest key (levels of 11, 11 and 10 bits)
  uint32_t prefix = 0, pmask = 0;
  uint32_t above = 0, m_eq = 0;
  bool all = false;                                // fewer than K candidates: keep them all
  for (int lv = 0; lv < 3; lv++) {
    const int shift = lv == 0 ? 21 : (lv == 1 ? 10 : 0);
    const int nbits = lv == 2 ? 10 : 11;
    const uint32_t dmask = (1u << nbits) - 1u;
    if (lv == 0) {
      // every candidate takes part: spread the (few, crowded) top-digit bins over copies
      for (int i = tid; i < TK_BINS * TK_COPIES; i += TK_NT) hcopy[i] = 0u;
      __syncthreads();
      const uint32_t cp = threadIdx.x & (TK_COPIES - 1);
      for (int cb = 0; cb < nc; cb += TK_UNR * 4 * TK_NT) {
        float4 v[TK_UNR];
        load_batch(cb, v);
#pragma unroll
        for (int u = 0; u < TK_UNR; u++) {
          const float vv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const uint32_t key = tk_key(vv[e]);
            if (key != 0u) atomicAdd(&hcopy[((key >> shift) & dmask) * TK_COPIES + cp], 1u);
          }
        }
      }
      __syncthreads();
      for (int i = tid; i < TK_BINS; i += TK_NT) {
        uint32_t t = 0;
#pragma unroll
        for (int k = 0; k < TK_COPIES; k++) t += hcopy[i * TK_COPIES + k];
        hist[i] = t;
      }
      __syncthreads();
    } else {
      // only the keys under the chosen prefix take part: few, and spread over the bins
      for (int i = tid; i < TK_BINS; i += TK_NT) hist[i] = 0u;
      __syncthreads();
      for (int cb = 0; cb < nc; cb += TK_UNR * 4 * TK_NT) {
        float4 v[TK_UNR];
        load_batch(cb, v);
#pragma unroll
        for (int u = 0; u < TK_UNR; u++) {
          const float vv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const uint32_t key = tk_key(vv[e]);
            tk_hist_add(hist, (int)((key >> shift) & dmask), (key & pmask) == prefix);
          }
        }
      }
      __syncthreads();
    }
    // digit holding the (K - above)-th largest remaining key: suffix sums from the top bin
    const uint32_t need = (uint32_t)K - above;
    const int nb = 1 << nbits;
    const int per = nb / TK_NT;                    // 2 (levels 1, 2) or 1 (level 3)
    uint32_t mine = 0;
    for (int k = 0; k < per; k++) mine += hist[nb - 1 - (tid * per + k)];
    uint32_t tot;
    const uint32_t before = tk_scan<TK_NW>(mine, red, &tot);   // keys in higher bins than this thread's
    if (lv == 0 && tot <= (uint32_t)K) {
      all = true;
      break;
    }
    uint32_t run = before;
    for (int k = 0; k < per; k++) {
      const int bin = nb - 1 - (tid * per + k);
      const uint32_t h = hist[bin];
      if (run < need && need <= run + h) {
        sel_s[0] = (uint32_t)bin;
        sel_s[1] = run;
        sel_s[2] = h;
      }
      run += h;
    }
    __syncthreads();
    prefix |= sel_s[0] << shift;
    pmask |= dmask << shift;
    above += sel_s[1];
    m_eq = sel_s[2];
    __syncthreads();
  }
  // ---- compaction in index order: keys above tau, then the first (K - above) keys equal to it
  const uint32_t tau = all ? 1u : prefix;          // all: every candidate (key >= 1)
  const uint32_t take_eq = all ? 0u : (uint32_t)K - above;
  const bool rank_eq = !all && take_eq < m_eq;     // ties at tau split by index
  uint32_t out_base = 0, eq_base = 0;
  for (int cb = 0; cb < nc; cb += TK_UNR * 4 * TK_NT) {
    float4 vb[TK_UNR];
    load_batch(cb, vb);
#pragma unroll
    for (int u = 0; u < TK_UNR; u++) {
      const int c = cb + u * 4 * TK_NT + 4 * tid;
      if (cb + u * 4 * TK_NT >= nc) break;
      const float vv[4] = {vb[u].x, vb[u].y, vb[u].z, vb[u].w};
      uint32_t key[4];
      uint32_t n_eq = 0;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        key[e] = tk_key(vv[e]);
        n_eq += (!all && key[e] == tau) ? 1u : 0u;
      }
      uint32_t eq_off = 0, eq_tot = 0;
      if (rank_eq) eq_off = tk_scan<TK_NW>(n_eq, red, &eq_tot);
      bool keep[4];
      uint32_t n_keep = 0, r = eq_base + eq_off;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const bool gt = all ? key[e] >= tau : key[e] > tau;
        const bool eq = !all && key[e] == tau;
        keep[e] = gt || (eq && (!rank_eq || r < take_eq));
        r += eq ? 1u : 0u;
        n_keep += keep[e] ? 1u : 0u;
      }
      uint32_t ktot;
      uint32_t o = out_base + tk_scan<TK_NW>(n_keep, red, &ktot);
#pragma unroll
      for (int e = 0; e < 4; e++)
        if (keep[e] && o < (uint32_t)K) orow[o++] = cand_token<BS, TWO>(c + e, brow);
      out_base += ktot;
      eq_base += eq_tot;
    }
  }
  for (int i = (int)out_base + tid; i < K; i += TK_NT) orow[i] = -1;
}

// The same selection for short rows (nc <= 256 * PER, e.g. the two-level rows of top_k
// blocks): one workgroup of 256 threads, each holding PER consecutive candidates' keys in
// registers for all three levels and the compaction, with one LDS histogram.
template <int BS, bool TWO, int PER>
__global__ __launch_bounds__(TKS_NT) void token_topk_small_kernel(const float* __restrict__ scores, int nc, int K,
                                                                  const int32_t* __restrict__ block_idx, int kblk,
                                                                  int32_t* __restrict__ token_idx, int Hkv) {
  constexpr int NW = TKS_NT / 64;
  __shared__ uint32_t hist[TK_BINS];
  __shared__ uint32_t red[NW + 1];
  __shared__ uint32_t sel_s[3];
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const float* row = scores + ((size_t)b * Hkv + g) * nc;
  const int32_t* brow = TWO ? block_idx + ((size_t)b * Hkv + g) * kblk : nullptr;
  int32_t* orow = token_idx + ((size_t)b * Hkv + g) * K;
  const int c0 = tid * PER;
  uint32_t key[PER];
#pragma unroll
  for (int u = 0; u < PER / 4; u++) {
    const int c = c0 + 4 * u;
    const float4 v = c < nc ? *reinterpret_cast<const float4*>(row + c)
                            : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    key[4 * u] = tk_key(v.x);
    key[4 * u + 1] = tk_key(v.y);
    key[4 * u + 2] = tk_key(v.z);
    key[4 * u + 3] = tk_key(v.w);
  }
  uint32_t prefix = 0, pmask = 0;
  uint32_t above = 0, m_eq = 0;
  bool all = false;
  for (int lv = 0; lv < 3; lv++) {
    const int shift = lv == 0 ? 21 : (lv == 1 ? 10 : 0);
    const int nbits = lv == 2 ? 10 : 11;
    const uint32_t dmask = (1u << nbits) - 1u;
    for (int i = tid; i < TK_BINS; i += TKS_NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; u++)
      if (key[u] != 0u && (key[u] & pmask) == prefix) atomicAdd(&hist[(key[u] >> shift) & dmask], 1u);
    __syncthreads();
    const uint32_t need = (uint32_t)K - above;
    const int nb = 1 << nbits;
    const int per = nb / TKS_NT;
    uint32_t mine = 0;
    for (int k = 0; k < per; k++) mine += hist[nb - 1 - (tid * per + k)];
    uint32_t tot;
    const uint32_t before = tk_scan<NW>(mine, red, &tot);
    if (lv == 0 && tot <= (uint32_t)K) {
      all = true;
      break;
    }
    uint32_t run = before;
    for (int k = 0; k < per; k++) {
      const int bin = nb - 1 - (tid * per + k);
      const uint32_t h = hist[bin];
      if (run < need && need <= run + h) {
        sel_s[0] = (uint32_t)bin;
        sel_s[1] = run;
        sel_s[2] = h;
      }
      run += h;
    }
    __syncthreads();
    prefix |= sel_s[0] << shift;
    pmask |= dmask << shift;
    above += sel_s[1];
    m_eq = sel_s[2];
    __syncthreads();
  }
  const uint32_t tau = all ? 1u : prefix;
  const uint32_t take_eq = all ? 0u : (uint32_t)K - above;
  const bool rank_eq = !all && take_eq < m_eq;
  uint32_t n_eq = 0;
#pragma unroll
  for (int u = 0; u < PER; u++) n_eq += (!all && key[u] == tau) ? 1u : 0u;
  uint32_t eq_off = 0, eq_tot = 0;
  if (rank_eq) eq_off = tk_scan<NW>(n_eq, red, &eq_tot);
  bool keep[PER];
  uint32_t n_keep = 0, r = eq_off;
#pragma unroll
  for (int u = 0; u < PER; u++) {
    const bool gt = all ? key[u] >= tau : key[u] > tau;
    const bool eq = !all && key[u] == tau;
    keep[u] = gt || (eq && (!rank_eq || r < take_eq));
    r += eq ? 1u : 0u;
    n_keep += keep[u] ? 1u : 0u;
  }
  uint32_t ktot;
  uint32_t o = tk_scan<NW>(n_keep, red, &ktot);
#pragma unroll
  for (int u = 0; u < PER; u++)
    if (keep[u] && o < (uint32_t)K) orow[o++] = cand_token<BS, TWO>(c0 + u, brow);
  for (int i = (int)ktot + tid; i < K; i += TKS_NT) orow[i] = -1;
}

size_t token_topk_workspace_bytes(const bsg_dims& d, bool two_level) {
  const size_t nc = two_level ? (size_t)d.top_k * d.page_size : (size_t)d.pt_stride * d.page_size;
  return (size_t)d.batch * d.num_kv_heads * nc * sizeof(float);
}

hipError_t launch_token_topk(const bsg_dims& d, const void* q, const int32_t* kv_lens, const void* k_cache,
                             const int32_t* page_table, const int32_t* block_idx, int top_k_tokens,
                             int32_t* token_idx, void* workspace, hipStream_t stream) {
  const bool two = block_idx != nullptr;
  const int nc = two ? d.top_k * d.page_size : d.pt_stride * d.page_size;
  float* scores = (float*)workspace;
  dim3 g1(nc / TS_CH, (d.num_kv_heads + TS_HPW - 1) / TS_HPW, d.batch);
#define BSG_TS(DD, BB, TW)                                                                                     \
  hipLaunchKernelGGL((token_score_kernel<DD, BB, TW>), g1, dim3(256), 0, stream, (const bf16_t*)q, kv_lens,     \
                     (const bf16_t*)k_cache, page_table, block_idx, d.top_k, scores, nc, d.num_q_heads,         \
                     d.num_kv_heads, d.num_pages, d.pt_stride)
#define BSG_TS_B(DD, TW)                                    \
  do {                                                      \
    if (d.page_size == 64) BSG_TS(DD, 64, TW);              \
    else BSG_TS(DD, 128, TW);                               \
  } while (0)
  if (d.head_dim == 128) {
    if (two) BSG_TS_B(128, true); else BSG_TS_B(128, false);
  } else {
    if (two) BSG_TS_B(64, true); else BSG_TS_B(64, false);
  }
#undef BSG_TS_B
#undef BSG_TS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(d.num_kv_heads, d.batch);
  if (nc <= TKS_NT * 16) {                         // short rows: keys in registers
#define BSG_TKS(BB, TW, PP)                                                                                    \
  hipLaunchKernelGGL((token_topk_small_kernel<BB, TW, PP>), g2, dim3(TKS_NT), 0, stream, scores, nc, top_k_tokens, \
                     block_idx, d.top_k, token_idx, d.num_kv_heads)
#define BSG_TKS_P(BB, TW)                                    \
  do {                                                       \
    if (nc <= TKS_NT * 8) BSG_TKS(BB, TW, 8);                \
    else BSG_TKS(BB, TW, 16);                                \
  } while (0)
    if (d.page_size == 64) {
      if (two) BSG_TKS_P(64, true); else BSG_TKS_P(64, false);
    } else {
      if (two) BSG_TKS_P(128, true); else BSG_TKS_P(128, false);
    }
#undef BSG_TKS_P
#undef BSG_TKS
    return hipGetLastError();
  }
  const size_t smem = (size_t)TK_BINS * TK_COPIES * sizeof(uint32_t);
#define BSG_TK(BB, TW)                                                                                         \
  do {                                                                                                          \
    auto kfn = token_topk_kernel<BB, TW>;                                                                       \
    hipError_t ea = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem); \
    if (ea != hipSuccess) return ea;                                                                            \
    hipLaunchKernelGGL(kfn, g2, dim3(TK_NT), smem, stream, scores, nc, top_k_tokens, block_idx, d.top_k,        \
                       token_idx, d.num_kv_heads);                                                              \
  } while (0)
  if (d.page_size == 64) {
    if (two) BSG_TK(64, true); else BSG_TK(64, false);
  } else {
    if (two) BSG_TK(128, true); else BSG_TK(128, false);
  }
#undef BSG_TK
  return hipGetLastError();
}

}  // namespace bsg
