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
// blocks (lanes l and l + 32 split a token's candidates).  Each lane keeps its best
// candidates as a descending register list of keys (score, then lower index) held in fp64
// bit patterns, so that a compare-exchange is one fp64 max and one fp64 min.  Per chunk the
// 16 new keys are sorted by a Batcher network and merged into the list bitonically; the
// stages of that work are issued between the matrix-core products of the next chunk.  At
// the end the two half-lists of a token are merged through LDS, the own block is appended
// and the kept ids are written ascending.
#include "bsg_device.h"
#include "bsg_internal.h"

namespace bsg {

namespace {
constexpr int FS_TOK = 128;   // tokens per workgroup (32 per wave)
constexpr int FS_CH = 32;     // candidate blocks per chunk
constexpr int FS_PAD = 8;     // LDS row padding (bf16 elements)
}  // namespace

// Candidate key as an fp64 bit pattern: bits 30..61 hold the score's order key, bits 0..29
// the complement of the block index (lower index wins ties), bits 62..63 are zero.  The
// exponent field's top bit is therefore zero (no inf or NaN), and it is never all zero for a
// finite score (that takes an order key below 2^22, i.e. a negative NaN), so every key is a
// positive normal double or +0 (the empty slot): fp64 max/min order them exactly as the
// 64-bit integers, and a compare-exchange costs two instructions.
__device__ __forceinline__ double fs_key(float s, int j) {
  const uint64_t k = ((uint64_t)order_key(s) << 30) | (uint64_t)(0x3fffffffu - (uint32_t)j);
  return __builtin_bit_cast(double, k);
}
__device__ __forceinline__ int fs_key_index(uint64_t key) { return (int)(0x3fffffffu - (uint32_t)(key & 0x3fffffffu)); }

__device__ __forceinline__ void fs_cas(double& hi, double& lo) {
  const double a = hi, b = lo;
  hi = __builtin_fmax(a, b);
  lo = __builtin_fmin(a, b);
}

// One layer (0..9) of Batcher's odd-even merge sort of 16 keys, descending; the ten layers
// in order hold its 63 compare-exchanges.
__device__ __forceinline__ void fs_sort_layer(double (&k)[16], int L) {
  int layer = 0;
#pragma unroll
  for (int p = 1; p < 16; p <<= 1)
#pragma unroll
    for (int d = p; d >= 1; d >>= 1, layer++)
      if (layer == L)
#pragma unroll
        for (int j = d % p; j + d < 16; j += 2 * d)
#pragma unroll
          for (int i = 0; i < d; i++)
            if (i + j + d < 16 && (i + j) / (2 * p) == (i + j + d) / (2 * p)) fs_cas(k[i + j], k[i + j + d]);
}

// Merging the 16 sorted keys k into best (descending) so that it holds the KCAP largest:
// the tail of best meets k reversed (fs_merge_meet), which leaves a bitonic sequence that
// holds the KCAP largest, and log2(KCAP) bitonic layers (fs_merge_layer) order it again.
template <int KCAP>
__device__ __forceinline__ void fs_merge_meet(double (&best)[KCAP], const double (&k)[16]) {
  constexpr int M = KCAP < 16 ? KCAP : 16;
#pragma unroll
  for (int i = 0; i < M; i++) best[KCAP - M + i] = __builtin_fmax(best[KCAP - M + i], k[M - 1 - i]);
}
template <int KCAP>
__device__ __forceinline__ void fs_merge_layer(double (&best)[KCAP], int L) {
  const int d = KCAP >> (L + 1);
#pragma unroll
  for (int i = 0; i < KCAP; i++)
    if ((i & d) == 0) fs_cas(best[i], best[i + d]);
}

template <int N>
constexpr int fs_log2() { return N <= 1 ? 0 : 1 + fs_log2<N / 2>(); }

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
  const int t0 = (gridDim.x - 1 - blockIdx.x) * FS_TOK;   // later tiles (more candidates) first
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int L = kv_lens[b];
  const int t = t0 + wave * 32 + col;
  const bool row_ok = t < q_len;
  const int own = max(L - q_len + t, 0) / bs;
  const int ncand = row_ok ? min(own, pt_stride) : 0;
  const int tlast = min(t0 + FS_TOK, q_len) - 1;
  const int nc_max = min(max(L - q_len + tlast, 0) / bs, pt_stride);   // candidates of the tile's last token

  // group-summed query, split into three bf16 terms (B operand: k = d, n = token).  With
  // KCAP = 64 the register list of keys takes 128 registers, so the terms wait in LDS (in the
  // region the final merge reuses), each lane reading back only what it wrote.
  constexpr bool QLDS = KCAP > 32;
  bf16x8_t qreg[QLDS ? 1 : 3][QLDS ? 1 : NDS];
  bf16x8_t* qlds = reinterpret_cast<bf16x8_t*>(fs_lists);   // [4 waves][3 terms][NDS][64 lanes]
  auto qterm = [&](int term, int ks) -> bf16x8_t {
    if constexpr (QLDS) return qlds[((wave * 3 + term) * NDS + ks) * 64 + lane];
    else return qreg[term][ks];
  };
  {
    float acc[NDS][8];
#pragma unroll
    for (int ks = 0; ks < NDS; ks++)
#pragma unroll
      for (int i = 0; i < 8; i++) acc[ks][i] = 0.0f;
    if (row_ok) {
      // Four heads' row pieces in flight (a ring of four buffers) while one head is summed.
      // The loads are unconditional (head index clamped; past the last head they re-read it
      // from cache) and heads past the group get weight 0, so the loop body has no branch and
      // the waits before each sum count exactly the loads issued after it.
      constexpr int QR = 4;
      const bf16_t* qp = q + (((size_t)b * Hq + (size_t)g * G) * q_len + t) * D + 8 * half;
      uint4 ring[QR][NDS];
      auto load_head = [&](int hh, uint4* dst) {
        const bf16_t* qr = qp + (size_t)min(hh, G - 1) * q_len * D;
#pragma unroll
        for (int ks = 0; ks < NDS; ks++) dst[ks] = *reinterpret_cast<const uint4*>(qr + 16 * ks);
      };
#pragma unroll
      for (int r = 0; r < QR; r++) load_head(r, ring[r]);
      for (int h0 = 0; h0 < G; h0 += QR) {
#pragma unroll
        for (int r = 0; r < QR; r++) {
          const float wgt = h0 + r < G ? 1.0f : 0.0f;    // a weight, not a branch
#pragma unroll
          for (int ks = 0; ks < NDS; ks++) {
            const uint4 v = ring[r][ks];
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 8; i++)
              acc[ks][i] = __builtin_fmaf(bf16_to_f32((bf16_t)((i & 1) ? (w4[i >> 1] >> 16) : (w4[i >> 1] & 0xffffu))),
                                          wgt, acc[ks][i]);
          }
          load_head(h0 + r + QR, ring[r]);
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < NDS; ks++) {
      bf16x8_t th, tm, tl;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float x = acc[ks][i];
        const __bf16 h = (__bf16)x;                 // v_cvt_pk_bf16_f32, nearest even
        const float r1 = x - (float)h;
        const __bf16 m = (__bf16)r1;
        const float r2 = r1 - (float)m;
        th[i] = h;
        tm[i] = m;
        tl[i] = (__bf16)r2;
      }
      if constexpr (QLDS) {
        qlds[((wave * 3 + 0) * NDS + ks) * 64 + lane] = th;
        qlds[((wave * 3 + 1) * NDS + ks) * 64 + lane] = tm;
        qlds[((wave * 3 + 2) * NDS + ks) * 64 + lane] = tl;
      } else {
        qreg[0][ks] = th;
        qreg[1][ks] = tm;
        qreg[2][ks] = tl;
      }
    }
  }

  double best[KCAP];                                // descending; 0 marks an empty slot
#pragma unroll
  for (int i = 0; i < KCAP; i++) best[i] = 0.0;

  // Chunk c's 32 representatives (zeros past the tile's candidates) travel in three steps,
  // each a chunk ahead of the next: page-table entries (iteration c - 2), rows into
  // registers (iteration c - 1, before that iteration's products), rows into LDS (after
  // them).  The loads are unconditional (indices clamped in range) so that no wait for them
  // is forced before their results are needed; pieces past the candidates are zeroed on
  // the way into LDS.
  constexpr int CPR = D / 8;                       // 16-byte pieces per row
  constexpr int NPC = FS_CH * CPR / 256;           // pieces per thread per chunk
  static_assert(NPC * 256 == FS_CH * CPR, "chunk split");
  auto piece_row = [&](int c, int u) { return c * FS_CH + (u * 256 + tid) / CPR; };
  auto chunk_pt = [&](int c, int* raw) {
#pragma unroll
    for (int u = 0; u < NPC; u++) raw[u] = page_table[(size_t)b * pt_stride + min(piece_row(c, u), nc_max - 1)];
  };
  auto chunk_rows = [&](const int* raw, uint4* v) {
#pragma unroll
    for (int u = 0; u < NPC; u++) {
      const int piece = (u * 256 + tid) % CPR;
      const int pid = page_id(raw[u], num_pages);
      v[u] = *reinterpret_cast<const uint4*>(block_cache + ((size_t)pid * Hkv + g) * D + 8 * piece);
    }
  };
  auto chunk_store = [&](int c, const uint4* v, int buf) {
#pragma unroll
    for (int u = 0; u < NPC; u++) {
      const int e = u * 256 + tid;
      const uint32_t m = piece_row(c, u) < nc_max ? 0xffffffffu : 0u;   // a mask, not a branch
      *reinterpret_cast<uint4*>(&reps[buf][(e / CPR) * RS + 8 * (e % CPR)]) =
          make_uint4(v[u].x & m, v[u].y & m, v[u].z & m, v[u].w & m);
    }
  };

  // scores of chunk c (transposed: lane (col, half) gets 16 candidates of token col)
  auto scores = [&](int c) {
    const bf16_t* R = reps[c & 1];
    f32x16_t sc;
#pragma unroll
    for (int e = 0; e < 16; e++) sc[e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < NDS; ks++) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(R + col * RS + 16 * ks + 8 * half);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qterm(0, ks), sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qterm(1, ks), sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qterm(2, ks), sc, 0, 0, 0);
    }
    return sc;
  };

  // Software pipeline: iteration c runs the products of chunk c + 1 on the matrix cores
  // while the vector units select from chunk c; chunk c + 2 goes into the LDS buffer that
  // chunk c used, and the loads for chunks c + 3 (rows) and c + 4 (page-table entries)
  // are issued.
  const int nchunks = (nc_max + FS_CH - 1) / FS_CH;
  int pt_n[NPC];                                   // page-table entries of a chunk ahead
  uint4 rows_n[NPC];                               // rows of a chunk ahead
#pragma unroll
  for (int c = 0; c < 2; c++)
    if (c < nchunks) {
      chunk_pt(c, pt_n);
      chunk_rows(pt_n, rows_n);
      chunk_store(c, rows_n, c);
    }
  if (2 < nchunks) {
    chunk_pt(2, pt_n);
    chunk_rows(pt_n, rows_n);
  }
  if (3 < nchunks) chunk_pt(3, pt_n);
  __syncthreads();
  f32x16_t s_cur = scores(0);
  // The selection from chunk c runs in stages: 4 of key building (4 keys each), the 10
  // sort layers, the meet and the merge layers.  Stages are spread over the 3 * NDS
  // products of chunk c + 1, each issued right after a product, so that the vector work of
  // this wave covers its own matrix-core latency.
  constexpr int NST = 15 + fs_log2<KCAP>();
  constexpr int NPROD = 3 * NDS;
  for (int c = 0; c < nchunks; c++) {
    const int jbase = c * FS_CH;
    double key[16];
    auto stage = [&](int st) {
      if (st < 4) {
#pragma unroll
        for (int e = 4 * st; e < 4 * st + 4; e++) {
          const int j = jbase + 8 * (e >> 2) + 4 * half + (e & 3);
          const double k = fs_key(s_cur[e], j);
          key[e] = j < ncand ? k : 0.0;
        }
      } else if (st < 14) {
        fs_sort_layer(key, st - 4);
      } else if (st == 14) {
        fs_merge_meet(best, key);
      } else {
        fs_merge_layer(best, st - 15);
      }
    };
    const bf16_t* R = reps[(c + 1) & 1];           // chunk c + 1 (past the last: stale, unused)
    f32x16_t sn;
#pragma unroll
    for (int e = 0; e < 16; e++) sn[e] = 0.0f;
    bf16x8_t a_cur = *reinterpret_cast<const bf16x8_t*>(R + col * RS + 8 * half);
#pragma unroll
    for (int ks = 0; ks < NDS; ks++) {
      const bf16x8_t a_nxt =
          *reinterpret_cast<const bf16x8_t*>(R + col * RS + 16 * (ks + 1 < NDS ? ks + 1 : ks) + 8 * half);
      const bf16x8_t b3[3] = {qterm(0, ks), qterm(1, ks), qterm(2, ks)};
#pragma unroll
      for (int i = 0; i < 3; i++) {
        sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_cur, b3[i], sn, 0, 0, 0);
        const int slot = 3 * ks + i;
#pragma unroll
        for (int x = 0; x < (NST + NPROD - 1) / NPROD; x++) {
          const int st = slot * NST / NPROD + x;
          if (st < (slot + 1) * NST / NPROD) stage(st);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      a_cur = a_nxt;
    }
    // Unconditional (all indices are clamped in range): past the last chunk these move data
    // that is never used, and the loop body stays one block for the scheduler.
    chunk_store(c + 2, rows_n, c & 1);
    chunk_rows(pt_n, rows_n);
    chunk_pt(c + 4, pt_n);
    __syncthreads();                               // chunk c + 2 stored; chunk c + 1 read
    s_cur = sn;
  }

  // merge the two half-lists of each token, append the own block, write ascending (with
  // QLDS this overwrites the query terms: every wave has passed the loop's last barrier, or,
  // with no chunk at all, the barrier below orders it after this wave's own reads)
  if (nchunks == 0) __syncthreads();
  uint64_t* mine = fs_lists + (size_t)tid * KCAP;
#pragma unroll
  for (int i = 0; i < KCAP; i++) mine[i] = __builtin_bit_cast(uint64_t, best[i]);
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
        ids[i] = fs_key_index(ta ? ka : kb);
        ia += ta ? 1 : 0;
        ib += ta ? 0 : 1;
      }
    }
    if constexpr (KCAP > 32) {
      sort_ints_asc(ids);                          // unused slots hold INT_MAX and sort last
#pragma unroll
      for (int i = 0; i < KCAP; i++)
        if (i < cnt) out[i] = ids[i];
    } else {
#pragma unroll
      for (int i = 0; i < KCAP; i++) {
        if (i < cnt) {
          int rank = 0;
#pragma unroll
          for (int i2 = 0; i2 < KCAP; i2++) rank += (i2 < cnt && ids[i2] < ids[i]) ? 1 : 0;
          out[rank] = ids[i];
        }
      }
    }
    out[cnt] = own;
    for (int i = cnt + 1; i < top_k; i++) out[i] = -1;
  }
}

bool group_score_topk_fused_supported(const bsg_dims& d, int q_len) {
  return d.dtype == BSG_BF16 && q_len >= 32 && d.top_k <= 65 && d.pt_stride < (1 << 30) - 1;
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

BSG_DEBUG_FILE(score_topk_fused)

}  // namespace bsg
