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
constexpr int TS_GMAX = 16;    // query heads per KV head the score workgroup takes
constexpr int TK_NT = 1024;    // threads of the selection workgroup
constexpr int TK_NW = TK_NT / 64;
constexpr int TK_BINS = 2048;  // radix bins per level (11 bits)
constexpr int TK_UNR = 8;      // row tiles (4 scores per thread each) loaded per batch
constexpr int TK_COPIES = 16;  // level-1 histogram copies (lane % 16): few lanes meet on one entry
constexpr int TKS_NT = 256;    // threads of the short-row selection workgroup
constexpr int TKM_NT = 1024;   // threads and keys per thread of the register selection of
constexpr int TKM_PER = 32;    //   rows up to 32768 candidates
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

// Candidates a selection reads from a row of nc scores.  Token level: the positions up to
// the query's, rounded up to 64 (the score kernels write -inf past the query's position up to
// there; a row of a prefill tile may hold nothing valid beyond); two level: all block slots.
template <bool TWO>
__device__ __forceinline__ int row_candidates(int nc, int pos) {
  if constexpr (TWO) return nc;
  else return min(nc, (max(pos, 0) + 64) / 64 * 64);
}

template <int D, int BS, bool TWO>
__global__ __launch_bounds__(256) void token_score_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ kv_lens, const bf16_t* __restrict__ k_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ block_idx, int kblk,
    float* __restrict__ scores, int nc, int Hq, int Hkv, int num_pages, int pt_stride, RowWindow rw) {
  static_assert(BS % TS_CH == 0, "a chunk lies in one page");
  constexpr int SEG = D / 8;                       // lanes per key row
  constexpr int PPH = TS_CH * SEG;                 // 16-byte pieces per head
  constexpr int NP = TS_HPW * PPH / 256;           // pieces per thread
  constexpr int QP = TS_HPW * TS_GMAX * (D / 8) / 256;   // query pieces per thread, at most
  __shared__ float qs[TS_HPW][D];
  __shared__ uint4 qraw[TS_HPW * TS_GMAX * (D / 8)];     // the workgroup's query rows, raw bf16
  const int c0 = blockIdx.x * TS_CH, g0 = blockIdx.y * TS_HPW, rl = blockIdx.z;
  const int b = rw.seq(rl), t = rw.pos(rl);
  if (t >= rw.T) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int G = Hq / Hkv;
  const int pos = kv_lens[b] - rw.T + t;
  // token level: a chunk wholly past the query's position lies past what the selection reads
  // (the position rounded up to 64), so it is neither scored nor written
  if (!TWO && c0 > pos) return;
  // the query rows first (one round trip, ahead of the key loads in the in-order load count).
  // The workgroup's TS_HPW groups own the consecutive heads g0 G .. (g0 + TS_HPW) G - 1; piece
  // i is 8 dims of head g0 G + i / (D / 8).  With G > TS_GMAX each summing thread reads its
  // rows itself, below.
  const bool qlds = G <= TS_GMAX;
  const int nq = qlds ? min(TS_HPW * G, Hq - g0 * G) * (D / 8) : 0;
  uint4 qv[QP];
#pragma unroll
  for (int u = 0; u < QP; u++) {
    const int i = u * 256 + tid;
    qv[u] = make_uint4(0, 0, 0, 0);
    if (i < nq)
      qv[u] = *reinterpret_cast<const uint4*>(q + (((size_t)b * Hq + g0 * G + i / (D / 8)) * rw.T + t) * D +
                                              8 * (i % (D / 8)));
  }
  // per head of this workgroup: the chunk's first token and the element offset of its key rows
  // (a chunk is 64 consecutive tokens of one block; at token level the same block for every
  // head); all workgroup-uniform
  int tok0[TS_HPW];
  size_t roff[TS_HPW];
#pragma unroll
  for (int hh = 0; hh < TS_HPW; hh++) {
    const int g = g0 + hh;
    const int32_t* brow = TWO ? block_idx + (((size_t)b * Hkv + min(g, Hkv - 1)) * rw.T + t) * kblk : nullptr;
    const int t0 = g < Hkv ? cand_token<BS, TWO>(c0, brow) : -1;
    const int j = t0 >= 0 ? t0 / BS : -1;
    const bool live = j >= 0 && j < pt_stride && t0 <= pos;
    const int p = live ? page_id(page_table[(size_t)b * pt_stride + j], num_pages) : 0;
    tok0[hh] = __builtin_amdgcn_readfirstlane(live ? t0 : -1);
    roff[hh] = (((size_t)p * Hkv + (live ? g : 0)) * BS + (live ? t0 % BS : 0)) * D / 8;
  }
  // the keys: head hh's 64 rows are PPH consecutive 16-byte pieces, UPH per thread
  constexpr int UPH = NP / TS_HPW;
  const uint4* kc4 = reinterpret_cast<const uint4*>(k_cache);
  uint4 raw[NP];
#pragma unroll
  for (int hh = 0; hh < TS_HPW; hh++) {
#pragma unroll
    for (int v = 0; v < UPH; v++) raw[hh * UPH + v] = make_uint4(0, 0, 0, 0);
    if (tok0[hh] >= 0) {
#pragma unroll
      for (int v = 0; v < UPH; v++) raw[hh * UPH + v] = kc4[roff[hh] + v * 256 + tid];
    }
  }
#pragma unroll
  for (int u = 0; u < QP; u++)
    if (u * 256 + tid < nq) qraw[u * 256 + tid] = qv[u];
  __syncthreads();
  // group-summed queries (fp32, heads in order), 8 dims per thread
  if (tid < TS_HPW * (D / 8)) {
    const int hh = tid / (D / 8), d8 = tid % (D / 8);
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    auto add8 = [&](const uint4 v) {
      const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        acc[2 * i] += __uint_as_float(wd[i] << 16);
        acc[2 * i + 1] += __uint_as_float(wd[i] & 0xffff0000u);
      }
    };
    if (g0 + hh < Hkv) {
      if (qlds) {
        for (int h = 0; h < G; h++) add8(qraw[(hh * G + h) * (D / 8) + d8]);
      } else {
        const uint4* qg = reinterpret_cast<const uint4*>(q);
        for (int h = 0; h < G; h++) add8(qg[(((size_t)b * Hq + (g0 + hh) * G + h) * rw.T + t) * (D / 8) + d8]);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; i++) qs[hh][8 * d8 + i] = acc[i];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NP; u++) {
    const int hh = u / UPH, pp = (u % UPH) * 256 + tid;    // piece pp of head hh's rows
    const int r = pp / SEG, w = pp % SEG;
    const float* qvs = &qs[hh][w * 8];
    const uint32_t wd[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      s = fmaf(qvs[2 * i], __uint_as_float(wd[i] << 16), s);
      s = fmaf(qvs[2 * i + 1], __uint_as_float(wd[i] & 0xffff0000u), s);
    }
    s = seg_sum_dpp<SEG>(s);
    const int g = g0 + hh;
    if ((lane % SEG) == 0 && g < Hkv)
      scores[((size_t)rl * Hkv + g) * nc + c0 + r] = (tok0[hh] >= 0 && tok0[hh] + r <= pos) ? s : -INFINITY;
  }
}

// Token-level scores of prefill rows on the matrix cores.  A workgroup (4 waves) takes 128
// query positions of one (sequence, group), a wave 32 of them, and one range of TG_RANGE
// candidate positions (the tile's candidates end at its last position, so the ranges past
// it have no workgroup's work), walked in chunks of 32 (all in one page): the chunk's 32 key rows go through
// LDS (double-buffered, the next chunk's loads in flight during the products) and
//   S^T (32 candidates x 32 queries) = K (candidates x D) . (hi + mid + lo)^T (D x queries)
// with v_mfma_f32_32x32x16_bf16, where hi + mid + lo are three bf16 terms of the fp32
// group-summed query (exact to ~2^-24 relative, as in the fused block selection), so the
// scores are the fp32 dot products up to accumulation order.  Each lane holds 16 candidates
// of one query; candidates past the query's position are written as -inf, up to the tile's
// last candidate rounded up to 64 (what the selection reads).  A wave's 32 x 32 tile goes
// through LDS and out row by row (eight lanes per 128-byte row), rather than as 16-byte
// pieces of 32 rows per store.
constexpr int TG_RANGE = 2048;                    // candidates per workgroup of token_score_gemm_kernel

// Three waves per SIMD at D = 128 (the three query terms take 96 registers): with the plain
// launch bound the compiler aimed higher and spilled 12 registers to scratch.
template <int D, int BS>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(D == 128 ? 3 : 4, D == 128 ? 3 : 8))) void token_score_gemm_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ kv_lens, const bf16_t* __restrict__ k_cache,
    const int32_t* __restrict__ page_table, float* __restrict__ scores, int nc, int Hq, int Hkv, int num_pages,
    int pt_stride, RowWindow rw) {
  constexpr int NDS = D / 16;                      // k-steps of the product
  constexpr int RS = D + 8;                        // LDS row stride (bf16)
  constexpr int CH = 32;                           // candidates per chunk
  constexpr int CPR = D / 8;                       // 16-byte pieces per key row
  constexpr int NPC = CH * CPR / 256;              // pieces per thread per chunk
  static_assert(NPC * 256 == CH * CPR && BS % CH == 0, "chunk split");
  __shared__ __attribute__((aligned(16))) bf16_t kt[2][CH * RS];
  constexpr int TS = CH + 4;                       // row stride of a wave's staged score tile
  __shared__ __attribute__((aligned(16))) float stile[4][32 * TS];
  const int g = blockIdx.z % Hkv, b = blockIdx.z / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int G = Hq / Hkv;
  const int L = kv_lens[b];
  const int tend = min(rw.T, rw.t0 + rw.CT);
  const int tw0 = rw.t0 + blockIdx.x * 128;
  if (tw0 >= tend) return;
  const int t = tw0 + wave * 32 + col;
  const bool row_ok = t < tend;
  const int pos = L - rw.T + t;
  const int plast = L - rw.T + min(tw0 + 128, tend) - 1;
  const int ncand = min(nc, (max(plast, 0) + 64) / 64 * 64);
  const int cbeg = blockIdx.y * TG_RANGE;               // this workgroup's candidates
  if (cbeg >= ncand) return;
  const int cend = min(ncand, cbeg + TG_RANGE);

  // group-summed query of position t (fp32, heads in order), as three bf16 terms; the
  // B operand of k-step ks holds dims 16 ks + 8 half .. + 7 of query col
  bf16x8_t qh[NDS], qm[NDS], ql[NDS];
  {
    float acc[NDS][8];
#pragma unroll
    for (int ks = 0; ks < NDS; ks++)
#pragma unroll
      for (int i = 0; i < 8; i++) acc[ks][i] = 0.0f;
    if (row_ok) {
      const bf16_t* qp = q + (((size_t)b * Hq + (size_t)g * G) * rw.T + t) * D + 8 * half;
      for (int h = 0; h < G; h++) {
        uint4 v[NDS];
#pragma unroll
        for (int ks = 0; ks < NDS; ks++) v[ks] = *reinterpret_cast<const uint4*>(qp + (size_t)h * rw.T * D + 16 * ks);
#pragma unroll
        for (int ks = 0; ks < NDS; ks++) {
          const uint32_t w4[4] = {v[ks].x, v[ks].y, v[ks].z, v[ks].w};
#pragma unroll
          for (int i = 0; i < 4; i++) {
            acc[ks][2 * i] += __uint_as_float(w4[i] << 16);
            acc[ks][2 * i + 1] += __uint_as_float(w4[i] & 0xffff0000u);
          }
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < NDS; ks++)
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float x = acc[ks][i];
        const __bf16 h = (__bf16)x;
        const float r1 = x - (float)h;
        const __bf16 m = (__bf16)r1;
        qh[ks][i] = h;
        qm[ks][i] = m;
        ql[ks][i] = (__bf16)(r1 - (float)m);
      }
  }

  auto issue = [&](int cc, uint4 (&v)[NPC]) {
    const int s0 = cc * CH;
    const int j = min(s0 / BS, pt_stride - 1);
    const int p = page_id(page_table[(size_t)b * pt_stride + j], num_pages);
    const bf16_t* base = k_cache + (((size_t)p * Hkv + g) * BS + s0 % BS) * D;
#pragma unroll
    for (int u = 0; u < NPC; u++) {
      const int e = u * 256 + tid;
      v[u] = *reinterpret_cast<const uint4*>(base + (size_t)(e / CPR) * D + 8 * (e % CPR));
    }
  };
  auto stash = [&](const uint4 (&v)[NPC], int buf) {
#pragma unroll
    for (int u = 0; u < NPC; u++) {
      const int e = u * 256 + tid;
      *reinterpret_cast<uint4*>(&kt[buf][(e / CPR) * RS + 8 * (e % CPR)]) = v[u];
    }
  };
  const int c0 = cbeg / CH, nch = (cend - cbeg) / CH;   // chunks c0 .. c0 + nch - 1
  uint4 v[NPC];
  issue(c0, v);
  stash(v, 0);
  if (nch > 1) issue(c0 + 1, v);
  __syncthreads();
  for (int cc = 0; cc < nch; cc++) {
    const bf16_t* R = kt[cc & 1];
    f32x16_t sc;
#pragma unroll
    for (int e = 0; e < 16; e++) sc[e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < NDS; ks++) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(R + col * RS + 16 * ks + 8 * half);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qh[ks], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qm[ks], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ql[ks], sc, 0, 0, 0);
    }
    {
      // the wave's 32 x 32 tile (query col, candidates) through LDS, then written row by row:
      // eight lanes cover a row's 32 candidates (128 bytes)
      float* tw = stile[wave];
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        const int cl = 8 * q4 + 4 * half;                   // candidate within the chunk
        const int sa = c0 * CH + cc * CH + cl;               // candidate position
        float4 w;
        w.x = sa <= pos ? sc[4 * q4] : -INFINITY;
        w.y = sa + 1 <= pos ? sc[4 * q4 + 1] : -INFINITY;
        w.z = sa + 2 <= pos ? sc[4 * q4 + 2] : -INFINITY;
        w.w = sa + 3 <= pos ? sc[4 * q4 + 3] : -INFINITY;
        *reinterpret_cast<float4*>(tw + col * TS + cl) = w;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int it = 0; it < 4; it++) {
        const int r = it * 8 + (lane >> 3), c4 = 4 * (lane & 7);
        const int tr = tw0 + wave * 32 + r;
        if (tr < tend) {
          const size_t rlr = (size_t)b * rw.CT + (tr - rw.t0);
          *reinterpret_cast<float4*>(scores + (rlr * Hkv + g) * nc + (size_t)(c0 + cc) * CH + c4) =
              *reinterpret_cast<const float4*>(tw + r * TS + c4);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (cc + 1 < nch) stash(v, (cc + 1) & 1);      // the buffer chunk cc - 1 used
    if (cc + 2 < nch) issue(c0 + cc + 2, v);
    __syncthreads();
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
                                                          int32_t* __restrict__ token_idx, int Hkv,
                                                          const int32_t* __restrict__ kv_lens, RowWindow rw,
                                                          int nparts, int32_t* __restrict__ part_lists) {
  extern __shared__ uint32_t hcopy[];              // level 1: TK_BINS bins x TK_COPIES copies
  __shared__ uint32_t hist[TK_BINS];
  __shared__ uint32_t red[TK_NW + 1];
  __shared__ uint32_t sel_s[3];                    // digit, count above the digit, count in it
  const int g = blockIdx.x, rl = blockIdx.y;
  const int b = rw.seq(rl), t = rw.pos(rl);
  if (t >= rw.T) return;
  const int tid = threadIdx.x;
  const float* row = scores + ((size_t)rl * Hkv + g) * nc;
  const int32_t* brow = TWO ? block_idx + (((size_t)b * Hkv + g) * rw.T + t) * kblk : nullptr;
  int32_t* orow = token_idx + (((size_t)b * Hkv + g) * rw.T + t) * K;
  nc = row_candidates<TWO>(nc, kv_lens[b] - rw.T + t);
  // nparts > 1 (token level): this workgroup selects the top K of part blockIdx.z of the row
  // (a multiple of 64 candidates) into part_lists, absolute candidate ids, for the second stage
  int c_off = 0;
  if (nparts > 1) {
    const int seg = ((nc + nparts - 1) / nparts + 63) / 64 * 64;
    c_off = min((int)blockIdx.z * seg, nc);
    nc = min(nc - c_off, seg);
    row += c_off;
    orow = part_lists + (((size_t)rl * Hkv + g) * nparts + blockIdx.z) * K;
  }
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
  // the kept ids go through LDS (the histogram, free by now) when they fit, so that the row is
  // written with whole-line stores rather than a scatter of 4-byte ones
  const bool staged = K <= TK_BINS;
  int32_t* stage = reinterpret_cast<int32_t*>(hist);
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
        if (keep[e] && o < (uint32_t)K) {
          const int32_t id = cand_token<BS, TWO>(c_off + c + e, brow);
          if (staged) stage[o] = id;
          else orow[o] = id;
          o++;
        }
      out_base += ktot;
      eq_base += eq_tot;
    }
  }
  const int nkept = min((int)out_base, K);
  if (staged) {
    __syncthreads();
    for (int i = tid; i < K; i += TK_NT) orow[i] = i < nkept ? stage[i] : -1;
  } else {
    for (int i = nkept + tid; i < K; i += TK_NT) orow[i] = -1;
  }
}

// The three radix levels and the index-order compaction of a row whose keys sit in registers,
// PER consecutive candidates per thread from c0 = tid * PER (a list's entries when lst is set,
// else candidate positions); the kept ids go to orow, ascending, -1 padded to K.  Every thread
// of the workgroup calls it (it holds barriers).
template <int BS, bool TWO, int PER, int NT>
__device__ __forceinline__ void tk_select_keys(const uint32_t (&key)[PER], int K, int c0,
                                               const int32_t* __restrict__ lst, const int32_t* __restrict__ brow,
                                               int32_t* __restrict__ orow, uint32_t* hist, uint32_t* red,
                                               uint32_t* sel_s) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  uint32_t above = 0, m_eq = 0;
  bool all = false;
  for (int lv = 0; lv < 3; lv++) {
    const int shift = lv == 0 ? 21 : (lv == 1 ? 10 : 0);
    const int nbits = lv == 2 ? 10 : 11;
    const uint32_t dmask = (1u << nbits) - 1u;
    for (int i = tid; i < TK_BINS; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; u++)
      if (key[u] != 0u && (key[u] & pmask) == prefix) atomicAdd(&hist[(key[u] >> shift) & dmask], 1u);
    __syncthreads();
    const uint32_t need = (uint32_t)K - above;
    const int nb = 1 << nbits;
    const int per = nb / NT;
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
  // the kept ids, in candidate order, go through LDS (the histogram, free by now) when they fit,
  // so that the row is written with whole-line stores rather than a scatter of 4-byte ones
  const bool staged = K <= TK_BINS;
  int32_t* stage = reinterpret_cast<int32_t*>(hist);
#pragma unroll
  for (int u = 0; u < PER; u++)
    if (keep[u] && o < (uint32_t)K) {
      const int32_t id = lst ? lst[c0 + u] : cand_token<BS, TWO>(c0 + u, brow);
      if (staged) stage[o] = id;
      else orow[o] = id;
      o++;
    }
  const int nkept = min((int)ktot, K);
  if (staged) {
    __syncthreads();
    for (int i = tid; i < K; i += NT) orow[i] = i < nkept ? stage[i] : -1;
  } else {
    for (int i = nkept + tid; i < K; i += NT) orow[i] = -1;
  }
}

// The same selection for rows of at most NT * PER candidates: one workgroup of NT threads,
// each holding PER consecutive candidates' keys in registers for all three levels and the
// compaction, with one LDS histogram.  Short rows (two-level rows of top_k blocks) take 256
// threads, prefill rows of up to 32768 positions 1024.
template <int BS, bool TWO, int PER, int NT>
__global__ __launch_bounds__(NT) void token_topk_small_kernel(const float* __restrict__ scores, int nc, int K,
                                                                  const int32_t* __restrict__ block_idx, int kblk,
                                                                  int32_t* __restrict__ token_idx, int Hkv,
                                                                  const int32_t* __restrict__ kv_lens, RowWindow rw,
                                                                  int stride, int pt_stride, int full_rows,
                                                                  const int32_t* __restrict__ part_lists) {
  constexpr int NW = NT / 64;
  __shared__ uint32_t hist[TK_BINS];
  __shared__ uint32_t red[NW + 1];
  __shared__ uint32_t sel_s[3];
  const int g = blockIdx.x, rl = blockIdx.y;
  const int b = rw.seq(rl), t = rw.pos(rl);
  if (t >= rw.T) return;
  const int tid = threadIdx.x;
  const float* row = scores + ((size_t)rl * Hkv + g) * stride;
  // two level over full rows (prefill): the candidates' scores sit at their token positions
  // in a row of every position's score (row stride `stride`), gathered through the block list.
  // part_lists (token level, second stage): the candidates are the first stage's kept ids
  // (ascending, -1 padded), their scores gathered from the row.
  const bool gather = TWO && full_rows != 0;
  const int32_t* lst = part_lists ? part_lists + ((size_t)rl * Hkv + g) * nc : nullptr;
  const int pos = kv_lens[b] - rw.T + t;
  const int32_t* brow = TWO ? block_idx + (((size_t)b * Hkv + g) * rw.T + t) * kblk : nullptr;
  int32_t* orow = token_idx + (((size_t)b * Hkv + g) * rw.T + t) * K;
  if (!lst) nc = row_candidates<TWO>(nc, pos);        // a list holds nc entries (-1 padded)
  const int c0 = tid * PER;
  uint32_t key[PER];
#pragma unroll
  for (int u = 0; u < PER / 4; u++) {
    const int c = c0 + 4 * u;
    float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    if (lst) {
      const int4 tk4 = c < nc ? *reinterpret_cast<const int4*>(lst + c) : make_int4(-1, -1, -1, -1);
      v.x = tk4.x >= 0 ? row[tk4.x] : -INFINITY;
      v.y = tk4.y >= 0 ? row[tk4.y] : -INFINITY;
      v.z = tk4.z >= 0 ? row[tk4.z] : -INFINITY;
      v.w = tk4.w >= 0 ? row[tk4.w] : -INFINITY;
    } else if (gather) {                           // 4 consecutive slots: 4 tokens of one block
      const int j = c < nc ? brow[c / BS] : -1;
      const int tk = j >= 0 ? block_id(j, pt_stride) * BS + c % BS : -1;
      if (tk >= 0) {
        v = *reinterpret_cast<const float4*>(row + tk);
        v.x = tk <= pos ? v.x : -INFINITY;           // past the position: not written, not a candidate
        v.y = tk + 1 <= pos ? v.y : -INFINITY;
        v.z = tk + 2 <= pos ? v.z : -INFINITY;
        v.w = tk + 3 <= pos ? v.w : -INFINITY;
      }
    } else if (c < nc) {
      v = *reinterpret_cast<const float4*>(row + c);
    }
    key[4 * u] = tk_key(v.x);
    key[4 * u + 1] = tk_key(v.y);
    key[4 * u + 2] = tk_key(v.z);
    key[4 * u + 3] = tk_key(v.w);
  }
  tk_select_keys<BS, TWO, PER, NT>(key, K, c0, lst, brow, orow, hist, red, sel_s);
}

// Token-level rows of 4097..TKM_NT * TKM_PER candidates (prefill windows, short decode rows):
// the register selection above, but each workgroup walks rows blockIdx.y, + gridDim.y, ... of
// group blockIdx.x, and the next row's scores stream into LDS (global -> LDS copies) while the
// current row is selected, so the row's load latency is not waited for row by row.  Thread t's
// PER consecutive candidates are copied by thread t itself: its u-th 16-byte piece lands at
// slot u * NT + t, so that the reads back are conflict-free, consecutive lanes consecutive slots.
template <int BS>
__global__ __launch_bounds__(TKM_NT) void token_topk_rows_kernel(const float* __restrict__ scores, int nc, int K,
                                                                 int32_t* __restrict__ token_idx, int Hkv,
                                                                 const int32_t* __restrict__ kv_lens, RowWindow rw,
                                                                 int stride, int nrows) {
  constexpr int NT = TKM_NT, PER = TKM_PER, NW = NT / 64, NPC = PER / 4;
  __shared__ uint32_t hist[TK_BINS];
  __shared__ uint32_t red[NW + 1];
  __shared__ uint32_t sel_s[3];
  extern __shared__ __attribute__((aligned(16))) float rowbuf[];   // [NPC][NT] 16-byte pieces
  const int g = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int c0 = tid * PER;
  const uint32_t buf_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)rowbuf;
  // candidates a row's selection reads (0 for a row past the window)
  auto row_nc = [&](int rl) {
    const int b = rw.seq(rl), t = rw.pos(rl);
    if (t >= rw.T) return 0;
    return row_candidates<false>(nc, kv_lens[b] - rw.T + t);
  };
  auto prefetch = [&](int rl) {
    const int n = row_nc(rl);                        // a multiple of 4
    const float* row = scores + ((size_t)rl * Hkv + g) * stride;
#pragma unroll
    for (int u = 0; u < NPC; u++)
      if (c0 + 4 * u < n)
        lds_dma16(row + c0 + 4 * u, __builtin_amdgcn_readfirstlane(buf_base + (uint32_t)(u * NT + wave * 64) * 16u));
  };
  if (blockIdx.y < nrows) prefetch(blockIdx.y);
  for (int rl = blockIdx.y; rl < nrows; rl += gridDim.y) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's copies of the row have landed
    __syncthreads();                                   // and every other wave's
    const int b = rw.seq(rl), t = rw.pos(rl);
    const int n = row_nc(rl);
    uint32_t key[PER];
#pragma unroll
    for (int u = 0; u < NPC; u++) {
      float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (c0 + 4 * u < n) v = *reinterpret_cast<const float4*>(rowbuf + 4 * (u * NT + tid));
      key[4 * u] = tk_key(v.x);
      key[4 * u + 1] = tk_key(v.y);
      key[4 * u + 2] = tk_key(v.z);
      key[4 * u + 3] = tk_key(v.w);
    }
    __syncthreads();                                   // the buffer is free for the next row
    if (rl + (int)gridDim.y < nrows) prefetch(rl + gridDim.y);
    if (t < rw.T) {                                    // workgroup-uniform
      int32_t* orow = token_idx + (((size_t)b * Hkv + g) * rw.T + t) * K;
      tk_select_keys<BS, false, PER, NT>(key, K, c0, nullptr, nullptr, orow, hist, red, sel_s);
    }
  }
}

size_t token_topk_workspace_bytes(const bsg_dims& d, bool two_level) {
  const size_t nc = two_level ? (size_t)d.top_k * d.page_size : (size_t)d.pt_stride * d.page_size;
  // rows longer than the register selection also get room for their parts' lists
  const size_t lists = nc > (size_t)TKM_NT * TKM_PER ? (size_t)TKM_NT * TKM_PER : 0;
  return (size_t)d.batch * d.num_kv_heads * (nc + lists) * sizeof(float);
}

// The register selection (token_topk_small_kernel) of rows of at most TKM_NT * TKM_PER
// candidates: nc candidates per row (a row of scores, a block list over full rows, or the
// parts' lists), 8 / 16 / 32 keys per thread.
static hipError_t token_topk_registers(const bsg_dims& d, bool two, const float* scores, int nc, int K,
                                       const int32_t* block_idx, int32_t* token_idx, const int32_t* kv_lens,
                                       RowWindow rw, int stride, int full_rows, const int32_t* lists, dim3 grid,
                                       hipStream_t stream) {
#define BSG_TKS(BB, TW, PP, NN)                                                                                \
  hipLaunchKernelGGL((token_topk_small_kernel<BB, TW, PP, NN>), grid, dim3(NN), 0, stream, scores, nc, K,       \
                     block_idx, d.top_k, token_idx, d.num_kv_heads, kv_lens, rw, stride, d.pt_stride, full_rows, \
                     lists)
#define BSG_TKS_P(BB, TW)                                    \
  do {                                                       \
    if (nc <= TKS_NT * 8) BSG_TKS(BB, TW, 8, TKS_NT);        \
    else if (nc <= TKS_NT * 16) BSG_TKS(BB, TW, 16, TKS_NT); \
    else BSG_TKS(BB, TW, TKM_PER, TKM_NT);                   \
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

// Parts per long token-level row: doubled while every part still gets a CU (one 128 KiB
// selection workgroup per CU), the parts' lists (P * K ids) fit the register selection and a
// part keeps at least 4 K candidates.
static int token_topk_parts(const bsg_dims& d, int nrows, int nc, int K, bool two) {
  if (two) return 1;
  const long long units = (long long)nrows * d.num_kv_heads;
  int P = 1;
  while (P < 16 && units * P * 2 <= 256 && (long long)P * 2 * K <= TKM_NT * TKM_PER && nc / (P * 2) >= 4 * K) P *= 2;
  return P;
}

// token_topk_rows_kernel over nrows rows: one workgroup per CU (its row buffer takes 128 KiB of
// LDS), the rows of each group dealt round robin to its share of the CUs.
static hipError_t token_topk_rows_persistent(const bsg_dims& d, const float* scores, int nc, int K,
                                             int32_t* token_idx, const int32_t* kv_lens, RowWindow rw, int stride,
                                             int nrows, hipStream_t stream) {
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    ncu = 256;
  int per_group = ncu / d.num_kv_heads;
  if (per_group < 1) per_group = 1;
  if (per_group > nrows) per_group = nrows;
  const size_t smem = (size_t)TKM_NT * TKM_PER * sizeof(float);
  dim3 grid(d.num_kv_heads, per_group);
#define BSG_TKR(BB)                                                                                              \
  do {                                                                                                           \
    auto kfn = token_topk_rows_kernel<BB>;                                                                       \
    hipError_t ea = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem); \
    if (ea != hipSuccess) return ea;                                                                             \
    hipLaunchKernelGGL(kfn, grid, dim3(TKM_NT), smem, stream, scores, nc, K, token_idx, d.num_kv_heads, kv_lens,  \
                       rw, stride, nrows);                                                                       \
  } while (0)
  if (d.page_size == 64) BSG_TKR(64); else BSG_TKR(128);
#undef BSG_TKR
  return hipGetLastError();
}

// Scores of rows rw (B * rw.CT of them) into `scores`, then their exact top-K into token_idx.
// gemm: token level on the matrix cores (prefill tiles of 128 positions); else the per-row
// kernel (decode rows, and two-level rows whose candidates differ from row to row).
static hipError_t token_topk_rows(const bsg_dims& d, const void* q, const int32_t* kv_lens, const void* k_cache,
                                  const int32_t* page_table, const int32_t* block_idx, int top_k_tokens,
                                  int32_t* token_idx, float* scores, RowWindow rw, bool gemm, int32_t* lists,
                                  hipStream_t stream) {
  const bool two = block_idx != nullptr;
  const int nc = two ? d.top_k * d.page_size : d.pt_stride * d.page_size;
  const int nfull = d.pt_stride * d.page_size;
  const int stride = gemm ? nfull : nc;          // gemm: every position's score, two level gathers
  const int nrows = d.batch * rw.CT;
  if (gemm) {
    dim3 g0((rw.CT + 127) / 128, (nfull + TG_RANGE - 1) / TG_RANGE, d.num_kv_heads * d.batch);
#define BSG_TG(DD, BB)                                                                                         \
  hipLaunchKernelGGL((token_score_gemm_kernel<DD, BB>), g0, dim3(256), 0, stream, (const bf16_t*)q, kv_lens,    \
                     (const bf16_t*)k_cache, page_table, scores, nfull, d.num_q_heads, d.num_kv_heads,          \
                     d.num_pages, d.pt_stride, rw)
    if (d.head_dim == 128) {
      if (d.page_size == 64) BSG_TG(128, 64); else BSG_TG(128, 128);
    } else {
      if (d.page_size == 64) BSG_TG(64, 64); else BSG_TG(64, 128);
    }
#undef BSG_TG
  } else {
    dim3 g1(nc / TS_CH, (d.num_kv_heads + TS_HPW - 1) / TS_HPW, nrows);
#define BSG_TS(DD, BB, TW)                                                                                     \
  hipLaunchKernelGGL((token_score_kernel<DD, BB, TW>), g1, dim3(256), 0, stream, (const bf16_t*)q, kv_lens,     \
                     (const bf16_t*)k_cache, page_table, block_idx, d.top_k, scores, nc, d.num_q_heads,         \
                     d.num_kv_heads, d.num_pages, d.pt_stride, rw)
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
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(d.num_kv_heads, nrows);
  if (!two && nc > TKS_NT * 16 && nc <= TKM_NT * TKM_PER)   // token-level rows for the 1024-thread form
    return token_topk_rows_persistent(d, scores, nc, top_k_tokens, token_idx, kv_lens, rw, stride, nrows, stream);
  if (nc <= TKM_NT * TKM_PER)                      // rows whose keys fit in registers
    return token_topk_registers(d, two, scores, nc, top_k_tokens, block_idx, token_idx, kv_lens, rw, stride,
                                gemm ? 1 : 0, nullptr, g2, stream);
  // long rows: with few rows, each row's parts are selected by workgroups of their own and the
  // register selection then takes the top K of the parts' lists (the global top K lies in
  // their union, and the lists are in candidate order, so ties resolve as in one pass)
  const int P = lists ? token_topk_parts(d, nrows, nc, top_k_tokens, two) : 1;
  const size_t smem = (size_t)TK_BINS * TK_COPIES * sizeof(uint32_t);
  dim3 g3(d.num_kv_heads, nrows, P);
#define BSG_TK(BB, TW)                                                                                         \
  do {                                                                                                          \
    auto kfn = token_topk_kernel<BB, TW>;                                                                       \
    hipError_t ea = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem); \
    if (ea != hipSuccess) return ea;                                                                            \
    hipLaunchKernelGGL(kfn, g3, dim3(TK_NT), smem, stream, scores, nc, top_k_tokens, block_idx, d.top_k,        \
                       token_idx, d.num_kv_heads, kv_lens, rw, P, lists);                                       \
  } while (0)
  if (d.page_size == 64) {
    if (two) BSG_TK(64, true); else BSG_TK(64, false);
  } else {
    if (two) BSG_TK(128, true); else BSG_TK(128, false);
  }
#undef BSG_TK
  e = hipGetLastError();
  if (e != hipSuccess || P == 1) return e;
  return token_topk_registers(d, two, scores, P * top_k_tokens, top_k_tokens, block_idx, token_idx, kv_lens, rw,
                              stride, 0, lists, g2, stream);
}

hipError_t launch_token_topk(const bsg_dims& d, const void* q, const int32_t* kv_lens, const void* k_cache,
                             const int32_t* page_table, const int32_t* block_idx, int top_k_tokens,
                             int32_t* token_idx, void* workspace, hipStream_t stream) {
  const size_t nc = block_idx ? (size_t)d.top_k * d.page_size : (size_t)d.pt_stride * d.page_size;
  int32_t* lists = nc > (size_t)TKM_NT * TKM_PER
                       ? reinterpret_cast<int32_t*>((float*)workspace + (size_t)d.batch * d.num_kv_heads * nc)
                       : nullptr;
  return token_topk_rows(d, q, kv_lens, k_cache, page_table, block_idx, top_k_tokens, token_idx, (float*)workspace,
                         RowWindow{1, 0, 1}, false, lists, stream);
}

// Prefill: the q_len positions go through in windows of CT rows per sequence, so that the
// scores of one window (B * CT * Hkv rows of nc floats) stay within TOKEN_PREFILL_WS bytes.
static constexpr size_t TOKEN_PREFILL_WS = (size_t)1 << 30;

static int token_prefill_window(const bsg_dims& d, int q_len) {
  const size_t nc = (size_t)d.pt_stride * d.page_size;
  const size_t per_pos = (size_t)d.batch * d.num_kv_heads * nc * sizeof(float);
  long long ct = (long long)(TOKEN_PREFILL_WS / per_pos);
  if (ct >= 128) ct = ct / 128 * 128;                  // whole tiles of the matrix-core kernel
  if (ct < 1) ct = 1;
  return (int)(ct < q_len ? ct : q_len);
}

size_t token_topk_prefill_workspace_bytes(const bsg_dims& d, int q_len, bool two_level) {
  (void)two_level;                                 // both forms score full rows
  const size_t nc = (size_t)d.pt_stride * d.page_size;
  return (size_t)d.batch * token_prefill_window(d, q_len) * d.num_kv_heads * nc * sizeof(float);
}

hipError_t launch_token_topk_prefill(const bsg_dims& d, const void* q, int q_len, const int32_t* kv_lens,
                                     const void* k_cache, const int32_t* page_table, const int32_t* block_idx,
                                     int top_k_tokens, int32_t* token_idx, void* workspace, hipStream_t stream) {
  const int ct = token_prefill_window(d, q_len);
  for (int t0 = 0; t0 < q_len; t0 += ct) {
    hipError_t e = token_topk_rows(d, q, kv_lens, k_cache, page_table, block_idx, top_k_tokens, token_idx,
                                   (float*)workspace, RowWindow{q_len, t0, ct}, true, nullptr, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

BSG_DEBUG_FILE(token_select)

}  // namespace bsg
