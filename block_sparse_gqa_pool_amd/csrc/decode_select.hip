// Decode-time scoring + causal top-k (one query per sequence).  Ling 2.0 page, "Summarizing
// the Breakthrough": at decode the block cache is read and only the top-k blocks are
// fetched; MSA post, second and third paragraphs: top-k per GQA group, without exponentials.
//
// The block cache of every candidate block is read exactly once (the dominant HBM stream of
// a decode step), so scoring is organised for bandwidth:
//
//  A. decode_score_chunk_kernel, grid (chunks of 64 candidate blocks, B), 256 threads.
//     The representatives of all KV heads of a page are contiguous (Hkv*D values), so the
//     workgroup streams whole page rows with 16-byte loads; each 16-byte piece is dotted
//     with the matching slice of the fp32 group-summed query and reduced over the D/8 lanes
//     that hold one (block, group).  The query row and the chunk's page ids are fetched
//     first, with one load each per thread, so that the row loads then go out without a
//     page-table round trip between them, four per thread at a time (more in flight measured
//     slower: the requests congest rather than hide latency).  Then one wave per group ranks the chunk's
//     64 keys (score, lower-index-first; rank = number of larger keys) and writes its best
//     top_k - 1 keys, sorted descending.
//  B. decode_select_kernel, one workgroup per (sequence, group): the exact selection of the
//     fused decode step's prologue (decode_prologue.h: a lower bound from the lists' leading
//     keys, the survivors above it, their ranks), then the kept ids are written ascending,
//     the own block appended and the row padded with -1.
#include "bsg_device.h"
#include "bsg_internal.h"
#include "decode_prologue.h"

namespace bsg {

namespace {
constexpr int DS_CH = 64;    // candidate blocks per workgroup of kernel A
constexpr int DS_NT = 256;
}  // namespace

// F8: the block cache holds OCP E4M3 codes with one scale per (page, head) (16 codes per
// 16-byte piece); the piece sums are then times the representative's scale.
template <int D, bool F8>
__global__ __launch_bounds__(DS_NT) void decode_score_chunk_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ kv_lens, const void* __restrict__ block_cache,
    const float* __restrict__ rep_scales, const int32_t* __restrict__ page_table, uint64_t* __restrict__ lists,
    int Hq, int Hkv, int bs, int m, int num_pages, int pt_stride, int nchunks, uint32_t ppb_magic) {
  extern __shared__ __attribute__((aligned(16))) float ds_smem[];
  float* qs = ds_smem;                   // [Hkv][D]
  float* sc = ds_smem + Hkv * D;         // [Hkv][DS_CH]
  constexpr int VPP = F8 ? 16 : 8;       // values per 16-byte piece
  constexpr int SEG = D / VPP;           // lanes per (block, group)
  constexpr int U = 4;                   // 16-byte loads in flight per thread
  const int b = blockIdx.y, c = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = Hq / Hkv;
  const int j0 = c * DS_CH;
  const int own = max(kv_lens[b] - 1, 0) / bs;
  const int ncand = min(own, pt_stride);
  const int nloc = max(0, min(DS_CH, ncand - j0));   // candidates in this chunk
  const int ppb = Hkv * SEG;                          // 16-byte pieces per block row
  const int total = nloc * ppb;
  const int32_t* ptrow = page_table + (size_t)b * pt_stride + j0;

  // the sequence's query row (Hq x D bf16), 16 bytes per piece, goes out first
  constexpr int QU = 4;
  const int nq16 = Hq * (D / 8);
  const uint4* q16 = reinterpret_cast<const uint4*>(q + (size_t)b * Hq * D);
  uint4 qr[QU];
#pragma unroll
  for (int i = 0; i < QU; i++) {
    const int e = i * DS_NT + tid;
    qr[i] = e < nq16 ? q16[e] : make_uint4(0, 0, 0, 0);
  }
  // the chunk's page ids, one per lane (DS_CH = 64 = wave size): a block row's page is then a
  // lane shuffle, so all row loads below go out without waiting on the page table
  static_assert(DS_CH == 64, "one page id per lane");
  const int pid = lane < nloc ? page_id(ptrow[lane], num_pages) : 0;
  uint4 raw[U];
  float scl[U];                          // F8: the piece's (page, group) scale, segment leaders
  const char* bc = reinterpret_cast<const char*>(block_cache);
  auto issue = [&](int base) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int pi = base + u * DS_NT + tid;
      const int blk = (int)__umulhi((uint32_t)pi, ppb_magic);   // pi / ppb (exact: pi * ppb < 2^32)
      const int p = __shfl(pid, blk & 63, 64);                  // page of this piece's block
      const int w = pi - blk * ppb;
      raw[u] = make_uint4(0, 0, 0, 0);
      if (pi < total)
        raw[u] = *reinterpret_cast<const uint4*>(bc + (size_t)p * Hkv * D * (F8 ? 1 : 2) + (size_t)w * 16);
      if (F8) scl[u] = (pi < total && (lane % SEG) == 0) ? rep_scales[(size_t)p * Hkv + w / SEG] : 0.0f;
    }
  };
  auto consume = [&](int base) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int pi = base + u * DS_NT + tid;
      const int blk = (int)__umulhi((uint32_t)pi, ppb_magic);
      const int w = pi - blk * ppb;
      const float* qv = qs + (size_t)w * VPP;   // (g, d-slice) of this piece
      const uint32_t wd[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
      float s = 0.0f;
      if constexpr (F8) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(wd[i], false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(wd[i], true);
          s = fmaf(qv[4 * i], lo[0], s);
          s = fmaf(qv[4 * i + 1], lo[1], s);
          s = fmaf(qv[4 * i + 2], hi[0], s);
          s = fmaf(qv[4 * i + 3], hi[1], s);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          s = fmaf(qv[2 * i], __uint_as_float(wd[i] << 16), s);
          s = fmaf(qv[2 * i + 1], __uint_as_float(wd[i] & 0xffff0000u), s);
        }
      }
      s = seg_sum_dpp<SEG>(s);
      if (F8) s *= scl[u];
      if (pi < total && (lane % SEG) == 0) sc[(w / SEG) * DS_CH + blk] = s;
    }
  };

  // q is in (the page-id wait above covered it): park it in LDS so that its registers are
  // free before the row loads go out
  uint4* qraw = reinterpret_cast<uint4*>(sc + Hkv * DS_CH + 2 * DS_NT);   // [Hq][D] bf16
#pragma unroll
  for (int i = 0; i < QU; i++) {
    const int e = i * DS_NT + tid;
    if (e < nq16) qraw[e] = qr[i];
  }
  if (total > 0) issue(0);                    // block-cache rows in flight while q is summed
  for (int e = QU * DS_NT + tid; e < nq16; e += DS_NT) qraw[e] = q16[e];   // rows beyond QU pieces
  __syncthreads();
  const bf16_t* qh = reinterpret_cast<const bf16_t*>(qraw);
  for (int e = tid; e < Hkv * D; e += DS_NT) {   // group sums in fp32, heads in order
    const int g = e / D, d = e % D;
    float s = 0.0f;
    for (int h = 0; h < G; h++) s += bf16_to_f32(qh[(size_t)(g * G + h) * D + d]);
    qs[e] = s;
  }
  __syncthreads();
  for (int base = 0; base < total; base += DS_NT * U) {
    if (base > 0) issue(base);
    consume(base);
  }
  __syncthreads();

  // per group: the chunk's best m keys, sorted descending (rank = number of larger keys)
  uint64_t* kbuf = reinterpret_cast<uint64_t*>(sc + Hkv * DS_CH) + wave * 64;
  for (int g = wave; g < Hkv; g += DS_NT / 64) {
    const uint64_t key = lane < nloc ? sel_key(sc[g * DS_CH + lane], j0 + lane) : 0ull;
    kbuf[lane] = key;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // rank = number of larger keys.  Keys of real blocks are distinct and nonzero (they hold
    // the block index), so only the empty slots (key 0, lanes nloc..63) tie; they take their
    // lane as rank, which keeps every rank distinct.
    int rank = 0;
    const ulonglong2* kb2 = reinterpret_cast<const ulonglong2*>(kbuf);
#pragma unroll 8
    for (int i = 0; i < 32; i++) {
      const ulonglong2 o = kb2[i];
      rank += (o.x > key ? 1 : 0) + (o.y > key ? 1 : 0);
    }
    if (key == 0ull) rank = lane;
    uint64_t* dst = lists + (((size_t)b * Hkv + g) * nchunks + c) * m;
    if (rank < m) dst[rank] = key;
    __builtin_amdgcn_wave_barrier();
  }
}

// Selection from the sorted chunk lists.  tau = max over chunks of the chunk's m-th key is
// a lower bound of the global m-th key (that chunk alone holds m keys >= tau), so only keys
// >= tau can be kept; they form a prefix of every list.  Each surviving key counts the keys
// above it in every list prefix (binary search), which gives its global rank; ranks below
// the number to keep are selected.  All keys are distinct, so the ranks are too.
__global__ __launch_bounds__(256) void decode_select_kernel(const uint64_t* __restrict__ lists,
                                                            const int32_t* __restrict__ kv_lens,
                                                            int32_t* __restrict__ block_idx, int Hkv, int bs,
                                                            int top_k, int nchunks, int pt_stride, int lt) {
  extern __shared__ __attribute__((aligned(16))) uint64_t dsel_smem[];
  __shared__ int kept[64];
  __shared__ int counter_s;
  __shared__ uint64_t tau_s;
  const int row = blockIdx.x;
  const int b = row / Hkv;
  const int tid = threadIdx.x;
  const int m = top_k - 1;
  const int own = max(kv_lens[b] - 1, 0) / bs;
  const int cnt = min(m, min(own, pt_stride));
  int32_t* out = block_idx + (size_t)row * top_k;
  if (cnt > 0) {
    decode_select_prologue(lists + (size_t)row * nchunks * m, nchunks, m, lt, cnt, dsel_smem, kept, &counter_s,
                           &tau_s);
    if (tid < cnt) {                                         // ascending
      const int ji = kept[tid];
      int r2 = 0;
      for (int i = 0; i < cnt; i++) r2 += kept[i] < ji ? 1 : 0;
      out[r2] = ji;
    }
  }
  if (tid == 0) out[cnt] = own;
  for (int i = cnt + 1 + tid; i < top_k; i += 256) out[i] = -1;
}

int decode_select_nchunks(const bsg_dims& d) { return (d.pt_stride + DS_CH - 1) / DS_CH; }

size_t decode_select_workspace_bytes(const bsg_dims& d) {
  return (size_t)d.batch * d.num_kv_heads * decode_select_nchunks(d) * (size_t)(d.top_k > 1 ? d.top_k - 1 : 1) *
         sizeof(uint64_t);
}

bool decode_select_supported(const bsg_dims& d, int q_len) {
  const int nchunks = decode_select_nchunks(d);
  const int m = d.top_k - 1;
  return q_len == 1 && d.dtype == BSG_BF16 &&
         decode_prologue_smem_bytes(nchunks, m, decode_prologue_lt(nchunks, m)) <= 150 * 1024;
}

hipError_t launch_decode_score_chunks(const bsg_dims& d, const void* q, const int32_t* kv_lens,
                                     const void* block_cache, const int32_t* page_table, uint64_t* lists,
                                     hipStream_t stream, const float* rep_scales) {
  const int nchunks = decode_select_nchunks(d);
  const int m = d.top_k - 1;
  if (m <= 0) return hipSuccess;
  const bool f8 = rep_scales != nullptr;
  dim3 grid(nchunks, d.batch);
  const size_t smem = (size_t)(d.num_kv_heads * d.head_dim + d.num_kv_heads * DS_CH) * sizeof(float) +
                      (size_t)(DS_NT / 64) * 64 * sizeof(uint64_t) + (size_t)d.num_q_heads * d.head_dim * 2;
  const uint32_t ppb = (uint32_t)d.num_kv_heads * (d.head_dim / (f8 ? 16 : 8));   // pieces per block row
  const uint32_t magic = (uint32_t)((0x100000000ull + ppb - 1) / ppb);             // ceil(2^32 / ppb)
#define BSG_DSC(DD, F)                                                                                          \
  hipLaunchKernelGGL((decode_score_chunk_kernel<DD, F>), grid, dim3(DS_NT), smem, stream, (const bf16_t*)q,      \
                     kv_lens, block_cache, rep_scales, page_table, lists, d.num_q_heads, d.num_kv_heads,         \
                     d.page_size, m, d.num_pages, d.pt_stride, nchunks, magic)
  if (d.head_dim == 128) {
    if (f8) BSG_DSC(128, true); else BSG_DSC(128, false);
  } else {
    if (f8) BSG_DSC(64, true); else BSG_DSC(64, false);
  }
#undef BSG_DSC
  return hipGetLastError();
}

hipError_t launch_decode_select(const bsg_dims& d, const void* q, const int32_t* kv_lens, const void* block_cache,
                                const int32_t* page_table, int32_t* block_idx, void* workspace, hipStream_t stream) {
  if (decode_unit_supported(d))                    // rows of at most 4096 blocks: one kernel
    return launch_decode_unit_select(d, q, kv_lens, block_cache, page_table, block_idx, stream);
  const int nchunks = decode_select_nchunks(d);
  const int m = d.top_k - 1;
  uint64_t* lists = (uint64_t*)workspace;
  hipError_t e = launch_decode_score_chunks(d, q, kv_lens, block_cache, page_table, lists, stream);
  if (e != hipSuccess) return e;
  const int lt = decode_prologue_lt(nchunks, m);
  const size_t smem2 = decode_prologue_smem_bytes(nchunks, m, lt);
  if (smem2 > 64 * 1024) {
    hipError_t ea = hipFuncSetAttribute((const void*)decode_select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                        (int)smem2);
    if (ea != hipSuccess) return ea;
  }
  hipLaunchKernelGGL(decode_select_kernel, dim3(d.batch * d.num_kv_heads), dim3(256), smem2, stream, lists, kv_lens,
                     block_idx, d.num_kv_heads, d.page_size, d.top_k, nchunks, d.pt_stride, lt);
  return hipGetLastError();
}

BSG_DEBUG_FILE(decode_select)

}  // namespace bsg
