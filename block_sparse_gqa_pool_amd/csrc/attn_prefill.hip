// Exact attention over the selected blocks ("Sparse Attention + Linear Backbones", section
// 5.5: softmax(q.k/sqrt(d)) over the selected keys times their values; "Sparse Attention for
// Long-Context LLMs", section 4.3: the top-k mask removes the other keys, so they are
// skipped rather than masked).  Causal inside the own block.
//
// bf16 path (matrix cores, gfx950 v_mfma_f32_32x32x16_bf16)
// ---------------------------------------------------------
// A workgroup (8 waves) owns 256 query rows = TT tokens x HG heads of one GQA group.  It
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
constexpr int PF_WAVES = 8;                 // waves per workgroup
constexpr int PF_ROWS = 32 * PF_WAVES;      // query rows per workgroup (32 per wave)
constexpr int PF_SUB = 64;                  // keys per staged sub-block
constexpr int PF_MAX_STAGES = 4;            // depth of the LDS ring of K/V sub-blocks
constexpr int PF_KW = 4;                    // K operand reads in flight ahead of the score product
// The ring's copies are issued by waves 0-3 only.  The matrix core serves the older wave of a
// SIMD first, so waves 4-7 are the last to reach each barrier; taking the copy issue off them
// shortens every wait (128K prompt 10.69-10.76 -> 10.50 ms; copies on waves 4-7: 10.80 ms).
constexpr int PF_CW = 4;                    // waves that issue the ring's copies
constexpr int PF_CW0 = 0;                   // the first of them
constexpr float LOG2E = 1.4426950408889634f;
}  // namespace

typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr;

// Key (row of the K tile) that feeds accumulator row m of a 32-key chunk.
__device__ __forceinline__ int perm_key(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

// K and V tiles sit in LDS unpadded, D bf16 per row; the 16-byte chunk c of row r is stored
// at chunk position c ^ swz(r).  With this permutation the 16 rows read by one ds_read_b128
// group of the first product, and the 4 rows x 64 bytes read by one half-wave transposing
// read of the second, fall into distinct banks.
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// Wait until at most N of this wave's global->LDS copies are outstanding and all its LDS
// accesses are done, then workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_copies_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------------------------------
// Data movement and scheduling:
//  * the union's blocks are streamed in 64-key sub-blocks through a ring of nst LDS stages
//    (K and V tile each), copied by waves 0-3 straight from global memory into LDS (no
//    register staging) into stages every wave released at an earlier barrier: with 4 stages
//    the sub-blocks go in pairs, one barrier per pair and the next pair in flight while one is
//    computed; with fewer, one barrier per sub-block and up to nst-1 sub-blocks in flight;
//  * a workgroup is 8 waves (256 query rows = 32 tokens x 8 heads for G = 8): the selections
//    of neighbouring tokens overlap, so the union grows much slower than the row count and
//    the K/V bytes fetched per query row drop with the tile size;
//  * a wave skips every sub-block that none of its rows attends to; rows of the wave that did
//    not select the block get weight 0 through an infinite offset, and the causal mask is
//    applied only when the block is some row's own block;
//  * each row keeps a lazy reference maximum: the output and sum are only rescaled when a
//    sub-block would push a lane's sum of weights past 2^64 (or on the row's first block);
//  * workgroups are mapped to tiles XCD by XCD: the dispatcher deals workgroups to the 8
//    XCDs round robin, so the ids are remapped to give each XCD contiguous ranges of tiles
//    (whose selections overlap, in its own L2) in pairs, one early and one late in position:
//    later positions have more causal blocks to select from and cost more, so pairing them
//    evens out the XCDs' work; the later range and, within a range, the last tiles go first,
//    so the cheap tiles fill the end of the launch (three forms, below).
//  * the output rows leave through LDS: each lane's 8-byte pieces of its row are staged over
//    the ring, then 16 lanes write a 256-byte row (instead of sixteen bytes of 32 rows per
//    store).
template <int D, int BS, bool PAIRS>
__global__ __launch_bounds__(64 * PF_WAVES, 1) void attn_prefill_mfma_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ kv_lens, const bf16_t* __restrict__ k_cache,
    const bf16_t* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ block_idx, float scale, bf16_t* __restrict__ out, float* __restrict__ lse,
    int q_len, int Hq, int Hkv, int HG, int top_k, int num_pages, int pt_stride, int n_tt, int nst, gate_args ga) {
  constexpr int NT = 64 * PF_WAVES;
  constexpr int SUB = PF_SUB;
  constexpr int NSUB = BS / SUB;
  constexpr int NDS = D / 16;
  constexpr int NDC = D / 32;
  constexpr int CPR = D / 8;                       // 16-byte chunks per row
  constexpr int TILE = SUB * D * 2;                // bytes of one K (or V) sub-block tile
  constexpr int STG = 2 * TILE;                    // bytes of one ring stage
  constexpr int NCP = TILE / 1024 / PF_CW;         // 1 KiB copies per copying wave per tile
  static_assert(NCP >= 1 && NCP * 1024 * PF_CW == TILE, "tile split");
  extern __shared__ __attribute__((aligned(16))) unsigned char pf_smem[];
  const int TT = PF_ROWS / HG;
  int32_t* sel = reinterpret_cast<int32_t*>(pf_smem + nst * STG);   // [TT][top_k]
  const int nbw = (pt_stride + 31) >> 5;
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(sel + TT * top_k);
  int32_t* ulist = reinterpret_cast<int32_t*>(bitmap + nbw);          // union, ascending
  const int ucap = min(TT * top_k, pt_stride);
  int32_t* upage = ulist + ucap;                                       // its physical pages
  __shared__ int wsum[PF_WAVES];
  __shared__ int n_union;

  // ---- XCD-aware tile (the workgroup id mod 8 is its XCD).  The tiles (head-major, positions
  // ascending) are cut into equal contiguous parts and XCD x takes parts x and 15 - x of every
  // 16: one earlier and one later range, so that the XCDs get equal work although a tile's union
  // grows with its position, and each range stays contiguous for the XCD's L2.  The part with
  // the later positions goes first and each part runs last position first (costliest first).
  const int G = Hq / Hkv;
  const int slices = G / HG;
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  int logical;
  const int NR = nwg / n_tt;                         // (sequence, group, head slice) ranges
  if (NR % 8 == 0 && n_tt % 16 == 0 && n_tt / 16 >= 32) {
    // Each range is cut into 16 parts of P tiles.  In round k (of 8 per eight ranges, run
    // k = 7 down to 0) XCD x takes parts 15 - k, then k, of range 8c + (x + k) mod 8: every XCD
    // sees every position pair and every range once, whatever the ranges' cost profiles, and
    // at any time the XCDs work on eight different ranges (different strides of the caches).
    const int P = n_tt / 16;
    const int rnd = slot / (2 * P), s2 = slot % (2 * P);
    const int c = rnd >> 3, k = 7 - (rnd & 7);
    const int rest8 = 8 * c + ((xcd + k) & 7);
    const int part = s2 < P ? 15 - k : k;
    const int within = s2 < P ? s2 : s2 - P;
    logical = rest8 * n_tt + part * P + (P - 1 - within);
  } else if (nwg % 16 == 0) {
    // R rounds of 16 equal parts; in round k XCD x takes parts 16k + x and 16k + 15 - x.  One
    // round while a part is at least half of one (sequence, group)'s tiles: the two parts of an
    // XCD are then an early and a late range.  With shorter parts a pair can be two middle
    // ranges, which cost more (a tile's union grows with its position and then saturates), so
    // the parts are made finer (down to 32 tiles), every round covering other positions.
    int R = 1;
    if (2 * (nwg / 16) < n_tt)
      while (R < 8 && nwg % (32 * R) == 0 && nwg / (32 * R) >= 32) R *= 2;
    const int P = nwg / (16 * R);
    const int k = slot / (2 * P), s2 = slot % (2 * P);
    const int pa = 16 * k + xcd, pb = 16 * k + 15 - xcd;
    const int oa = (int)(((long long)pa * P) % n_tt), ob = (int)(((long long)pb * P) % n_tt);
    const int first = ob > oa ? pb : pa, second = ob > oa ? pa : pb;
    logical = s2 < P ? first * P + (P - 1 - s2) : second * P + (2 * P - 1 - s2);
  } else {                                         // a contiguous run per XCD
    const int qd8 = nwg >> 3, rd8 = nwg & 7;
    logical = xcd * qd8 + min(xcd, rd8) + slot;
    logical = (logical / n_tt) * n_tt + (n_tt - 1 - logical % n_tt);
  }
  const int tile = logical % n_tt;
  const int rest = logical / n_tt;
  const int gs = rest % (Hkv * slices);
  const int b = rest / (Hkv * slices);
  const int g = gs / slices, hs = gs % slices;
  const int t0 = tile * TT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int L = kv_lens[b];
  const int base_pos = L - q_len;

  // ---- the tile's selections and their union (ascending block ids)
  for (int e = tid; e < TT * top_k; e += NT) {
    const int tt = e / top_k, s = e % top_k;
    const int t = t0 + tt;
    int j = -1;
    if (t < q_len) j = block_idx[(((size_t)b * Hkv + g) * q_len + t) * top_k + s];
    sel[e] = j >= 0 ? block_id(j, pt_stride) : -1;
  }
  for (int w = tid; w < nbw; w += NT) bitmap[w] = 0u;
  __syncthreads();
  for (int e = tid; e < TT * top_k; e += NT) {
    const int j = sel[e];
    if (j >= 0) atomicOr(&bitmap[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  {
    const int per = (nbw + NT - 1) / NT;
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
    if (tid == NT - 1) n_union = off + cnt;
    for (int w = w0; w < w1; w++) {
      uint32_t bits = bitmap[w];
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1;
        const int j = (w << 5) + bit;
        ulist[off] = j;
        off++;
      }
    }
  }
  __syncthreads();
  const int U = n_union;
  // the union's physical pages: one page-table lookup per thread, all in flight together
  for (int u = tid; u < U; u += NT) upage[u] = page_id(page_table[(size_t)b * pt_stride + ulist[u]], num_pages);
  __syncthreads();

  // ---- this lane's query row
  const int col = lane & 31;
  const int half = lane >> 5;
  const int r = wave * 32 + col;
  const int tt = r / HG;
  const int h = g * G + hs * HG + (r % HG);
  const int t = t0 + tt;
  const bool row_ok = t < q_len;
  const int pos = base_pos + t;
  const int own = row_ok ? pos / BS : -1;
  int sp = 0;
  const int32_t* mysel = sel + tt * top_k;

  bf16x8_t qb[NDS];
  {
    const bf16_t* qp = q + (((size_t)b * Hq + h) * q_len + (row_ok ? t : 0)) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < NDS; ks++) {
      uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qp + 16 * ks) : make_uint4(0, 0, 0, 0);
      qb[ks] = *reinterpret_cast<bf16x8_t*>(&v);
    }
    // Consume the loads here: the compiler then waits for them before the loop instead of
    // at the first use inside it, where its wait would also drain the ring's copies.
#pragma unroll
    for (int ks = 0; ks < NDS; ks++) asm volatile("" ::"v"(qb[ks]));
  }
  const float c2 = scale * LOG2E;
  float m_i = -INFINITY;
  float l_i = 0.0f;
  f32x16_t o[NDC];
#pragma unroll
  for (int i = 0; i < NDC; i++)
#pragma unroll
    for (int e = 0; e < 16; e++) o[i][e] = 0.0f;

  // LDS byte offsets of this lane's operand reads inside a stage
  int koff[NDS];                 // first product: K row perm_key(col) (+32 per kc), chunk 2 ks + half
  {
    const int kr = perm_key(col);
#pragma unroll
    for (int ks = 0; ks < NDS; ks++) koff[ks] = kr * (D * 2) + (((2 * ks + half) ^ tile_swz<D>(kr)) << 4);
  }
  int voff[NDC][2];              // second product: V rows 16 st + 8 (qd>>1) + ep (+4), 8 bytes
  {
    const int qd = lane >> 4, ep = (lane & 15) >> 2, s4 = lane & 3;
#pragma unroll
    for (int dc = 0; dc < NDC; dc++)
#pragma unroll
      for (int hi = 0; hi < 2; hi++) {
        const int vr = 8 * (qd >> 1) + ep + 4 * hi;
        const int ch = 4 * dc + 2 * (qd & 1) + (s4 >> 1);
        voff[dc][hi] = TILE + vr * (D * 2) + ((ch ^ tile_swz<D>(vr)) << 4) + 8 * (s4 & 1);
      }
  }
  // this lane's share of the copies of one stage: tile row and element offset per copy
  int crow[NCP], coff[NCP];
#pragma unroll
  for (int c = 0; c < NCP; c++) {
    const int e = (wave - PF_CW0 + PF_CW * c) * 64 + lane;   // 16-byte slot of the tile
    crow[c] = e / CPR;
    coff[c] = crow[c] * D + ((e % CPR) ^ tile_swz<D>(crow[c])) * 8;
  }
  const uint32_t smem_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)pf_smem;
  const bool copier = wave >= PF_CW0 && wave < PF_CW0 + PF_CW;
  const uint32_t wave_slot = __builtin_amdgcn_readfirstlane((wave - PF_CW0) * 1024);
  const bf16_t* kbase = k_cache + (size_t)g * BS * D;   // + page * Hkv * BS * D
  const bf16_t* vbase = v_cache + (size_t)g * BS * D;
  // this wave's share of the copies of sub-block ic (block cj in page cp) into LDS stage c_stage
  int ic = 0, c_stage = 0;
  auto copy_sub = [&](int cj, int cp) {
    const int h2 = ic % NSUB;
    const int nvb = min(BS, L - cj * BS);                // valid keys of the block (>= 1)
    const size_t poff = (size_t)cp * Hkv * BS * D + (size_t)h2 * SUB * D;
    const bf16_t* kp = kbase + poff;
    const bf16_t* vp = vbase + poff;
    const uint32_t sb = smem_base + (uint32_t)(c_stage * STG) + wave_slot;
    if (nvb >= (h2 + 1) * SUB) {                         // every key of the sub-block is valid
#pragma unroll
      for (int c = 0; c < NCP; c++) {
        lds_dma16(kp + coff[c], sb + c * PF_CW * 1024);
        lds_dma16(vp + coff[c], sb + c * PF_CW * 1024 + TILE);
      }
    } else {
      // slots past the valid keys copy key 0 instead: finite data, masked out of the scores
#pragma unroll
      for (int c = 0; c < NCP; c++) {
        const int eo = h2 * SUB + crow[c] < nvb ? coff[c] : coff[c] - (h2 * SUB + crow[c]) * D;
        lds_dma16(kp + eo, sb + c * PF_CW * 1024);
        lds_dma16(vp + eo, sb + c * PF_CW * 1024 + TILE);
      }
    }
  };
  // the next sub-block's copies (waves 0-3), and every wave's count of issued sub-blocks
  auto issue = [&](int cj, int cp) {
    if (copier) copy_sub(cj, cp);
    ic++;
    c_stage = c_stage + 1 == nst ? 0 : c_stage + 1;
  };

  const int NS = U * NSUB;
  // With a ring of 4 stages the sub-blocks go in pairs: one barrier per pair, the pair's copies
  // issued during the pair before, after its first sub-block (into the stages of the pair
  // before that, released at that pair's barrier).  With fewer stages (large tables leave less LDS), one barrier per
  // sub-block, the copies of sub-block i+nst-1 issued at the end of iteration i.  Pairs halve
  // the barriers and even out the waves' work per barrier: when the waves attend to different
  // sub-blocks (32K prompt: ~2-3 of 8 waves per block), a barrier waits for the busiest SIMD.
  while (ic < (PAIRS ? 2 : nst - 1) && ic < NS) {
    const int u = ic / NSUB;
    issue(copier ? __builtin_amdgcn_readfirstlane(ulist[u]) : 0, copier ? __builtin_amdgcn_readfirstlane(upage[u]) : 0);
  }
  // the block schedule is read one block ahead, so that no LDS latency sits between the
  // barrier and the first product: jn = next union block, selc = this row's next selection
  int jn = U > 0 ? ulist[0] : 0;
  int selc = row_ok ? mysel[0] : -1;
  int j = 0;
  bool mine = false;
  int r_stage = 0;                                      // stage of sub-block i
  constexpr int PER = PAIRS ? 2 : 1;                   // sub-blocks per barrier
  for (int i0 = 0; i0 < NS; i0 += PER) {
    int cj = 0, cp = 0;
    if constexpr (PAIRS) {
      // pair i0/2 has landed (nothing younger is in flight)
      wait_copies_barrier<0>();
    } else {
      const int i = i0;
      // stage i has landed once at most min(nst-2, NS-1-i) younger stages are outstanding
      const int ahead = min(nst - 2, NS - 1 - i);
      if (ahead >= 2) wait_copies_barrier<4 * NCP>();
      else if (ahead == 1) wait_copies_barrier<2 * NCP>();
      else wait_copies_barrier<0>();
      // schedule entry of this iteration's copy, read now and used at the end
      if (copier && ic < NS) {
        cj = ulist[ic / NSUB];
        cp = upage[ic / NSUB];
      }
    }
#pragma unroll 1
  for (int i = i0; i < i0 + PER && i < NS; i++) {
    const int h2 = i % NSUB;
    if (h2 == 0) {
      j = __builtin_amdgcn_readfirstlane(jn);
      const int u = i / NSUB;
      if (u + 1 < U) jn = ulist[u + 1];
      mine = row_ok && selc == j;
      if (mine) {
        sp++;
        selc = sp < top_k ? mysel[sp] : -1;
      }
    }
    const int kfirst = j * BS + h2 * SUB;               // position of the sub-block's first key
    const bool act = mine && kfirst <= pos;             // the row attends to this sub-block
    if (__ballot(act) != 0) {
      const unsigned char* sbp = pf_smem + r_stage * STG;
      f32x16_t sacc[2];
      const f32x16_t zero16 = {};
      {
        // Score product: the two 32-key chains interleaved (k-step outer), every K operand
        // read PF_KW products ahead of its use, so that no product waits on a read issued
        // just before it (the chains' accumulation order is unchanged).
        constexpr int NK = 2 * NDS;
        bf16x8_t kbuf[PF_KW];
#pragma unroll
        for (int n = 0; n < PF_KW; n++)
          kbuf[n] = *reinterpret_cast<const bf16x8_t*>(sbp + koff[n >> 1] + (n & 1) * 32 * D * 2);
#pragma unroll
        for (int n = 0; n < NK; n++) {
          const int ks = n >> 1, kc = n & 1;
          const bf16x8_t a = kbuf[n % PF_KW];
          sacc[kc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], ks == 0 ? zero16 : sacc[kc], 0, 0, 0);
          if (n + PF_KW < NK)
            kbuf[n % PF_KW] =
                *reinterpret_cast<const bf16x8_t*>(sbp + koff[(n + PF_KW) >> 1] + ((n + PF_KW) & 1) * 32 * D * 2);
        }
        // schedule: PF_KW reads, then alternately one product and one read, then the rest
#pragma unroll
        for (int n = 0; n < PF_KW; n++) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
#pragma unroll
        for (int n = 0; n < NK - PF_KW; n++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int n = 0; n < PF_KW; n++) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      if (__ballot(act && j == own) != 0) {             // causal mask inside the own block
        const int klim = j == own ? pos - kfirst : SUB - 1;
#pragma unroll
        for (int kc = 0; kc < 2; kc++)
#pragma unroll
          for (int e = 0; e < 16; e++) {
            const int key = kc * 32 + 16 * (e >> 3) + 8 * half + (e & 7);
            sacc[kc][e] = key <= klim ? sacc[kc][e] : -INFINITY;
          }
      }
      // Probabilities against the row's reference maximum m_i, which only moves when the
      // sum would leave a safe range: softmax does not depend on the subtracted constant,
      // so the weights only need to stay finite (the sum <= 2^64).  Rows that do not
      // attend get probability 0 through an infinite offset.  A row seen for the first
      // time (m_i = -inf) gets an infinite sum and so also takes the exact update.
      bf16x8_t pb[SUB / 16];
      float rs = 0.0f;
      auto probs = [&]() {
        const float mc = act ? m_i * c2 : INFINITY;
        rs = 0.0f;
#pragma unroll
        for (int st = 0; st < SUB / 16; st++) {
          const int kc = st >> 1, hh = st & 1;
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const float pe = __builtin_amdgcn_exp2f(fmaf(sacc[kc][8 * hh + e], c2, -mc));
            pb[st][e] = (__bf16)pe;
            rs += pe;
          }
        }
      };
      probs();
      const bool bad = !(rs <= 0x1p64f);
      if (__ballot(bad) != 0) {                          // rare: move the reference maximum
        float mx = -INFINITY;
#pragma unroll
        for (int kc = 0; kc < 2; kc++)
#pragma unroll
          for (int e = 0; e < 16; e++) mx = fmaxf(mx, sacc[kc][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // both halves of a row must move together: every lane reads its partner's flag (a
        // cross-lane read inside a short-circuit would run only in the lanes that are not bad,
        // and their partners, the bad lanes, would be inactive sources)
        const int partner_bad = __shfl_xor((int)bad, 32, 64);
        const bool bad_row = bad || partner_bad != 0;
        const float m_new = (act && bad_row) ? fmaxf(m_i, mx) : m_i;
        const float alpha = m_new == m_i ? 1.0f : __builtin_amdgcn_exp2f((m_i - m_new) * c2);
        l_i *= alpha;
#pragma unroll
        for (int i2 = 0; i2 < NDC; i2++)
#pragma unroll
          for (int e = 0; e < 16; e++) o[i2][e] *= alpha;
        m_i = m_new;
        probs();
      }
      l_i += rs;
#pragma unroll
      for (int st = 0; st < SUB / 16; st++) {
#pragma unroll
        for (int dc = 0; dc < NDC; dc++) {
          const unsigned char* vb = sbp + st * 16 * D * 2;
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vb + voff[dc][0]));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vb + voff[dc][1]));
          bf16x8_t va;
          *reinterpret_cast<s16x4_t*>(&va) = lo;
          *(reinterpret_cast<s16x4_t*>(&va) + 1) = hi;
          o[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[st], o[dc], 0, 0, 0);
        }
      }
    }
    // next copy, into the stage everyone finished with before this iteration's barrier
    if (!PAIRS && ic < NS) issue(__builtin_amdgcn_readfirstlane(cj), __builtin_amdgcn_readfirstlane(cp));
    if (PAIRS && i == i0) {
#pragma unroll 1
      for (int c2 = 0; c2 < 2; c2++) {
        if (ic < NS) {
          const int u = ic / NSUB;
          issue(copier ? __builtin_amdgcn_readfirstlane(ulist[u]) : 0, copier ? __builtin_amdgcn_readfirstlane(upage[u]) : 0);
        }
      }
    }
    r_stage = r_stage + 1 == nst ? 0 : r_stage + 1;
  }
  }

  const float l = l_i + __shfl_xor(l_i, 32, 64);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const size_t row = ((size_t)b * Hq + h) * q_len + t;
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  // the workgroup's 256 output rows go through LDS (the ring is free once every wave has left
  // the loop) and out row by row, 16 lanes per 256-byte row
  constexpr int OS = D + 8;                        // LDS row stride (bf16)
  bf16_t* ot = reinterpret_cast<bf16_t*>(pf_smem);
  __syncthreads();
#pragma unroll
  for (int dc = 0; dc < NDC; dc++)
#pragma unroll
    for (int e4 = 0; e4 < 4; e4++) {
      const int d0 = 32 * dc + 8 * e4 + 4 * half;
      float a[4];
#pragma unroll
      for (int x = 0; x < 4; x++) a[x] = o[dc][4 * e4 + x] * inv;
      if (ga.g && row_ok) {                            // out = g A + (1 - g) x, one rounding
        const bf16x4_t xv = *reinterpret_cast<const bf16x4_t*>(static_cast<const bf16_t*>(ga.x) + row * D + d0);
        float g4[4];
        if (ga.per_dim) {
          const float4 gv = *reinterpret_cast<const float4*>(ga.g + row * D + d0);
          g4[0] = gv.x; g4[1] = gv.y; g4[2] = gv.z; g4[3] = gv.w;
        } else {
          g4[0] = g4[1] = g4[2] = g4[3] = ga.g[row];
        }
#pragma unroll
        for (int x = 0; x < 4; x++) a[x] = g4[x] * a[x] + (1.0f - g4[x]) * (float)xv[x];
      }
      bf16x4_t v4;
#pragma unroll
      for (int x = 0; x < 4; x++) v4[x] = (__bf16)a[x];   // v_cvt_pk_bf16_f32 (nearest even)
      *reinterpret_cast<bf16x4_t*>(ot + r * OS + d0) = v4;
    }
  if (lse && half == 0 && row_ok) lse[row] = m_i * scale + logf(l);
  __syncthreads();
  constexpr int PPR = D / 8;                       // 16-byte pieces per row
#pragma unroll
  for (int it = 0; it < PF_ROWS * PPR / NT; it++) {
    const int pce = it * NT + tid;
    const int rr = pce / PPR, ch = pce % PPR;
    const int t2 = t0 + rr / HG;
    if (t2 < q_len) {
      const int h2 = g * G + hs * HG + (rr % HG);
      const size_t row2 = ((size_t)b * Hq + h2) * q_len + t2;
      *reinterpret_cast<uint4*>(out + row2 * D + 8 * ch) = *reinterpret_cast<const uint4*>(ot + rr * OS + 8 * ch);
    }
  }
}

// ---------------------------------------------------------------------------------------
// VALU path (fp32 inputs, or shapes the matrix-core path does not cover): one wave per
// (sequence, head, query), lanes split D, online softmax over the selected keys.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_prefill_valu_kernel(
    const T* __restrict__ q, const int32_t* __restrict__ kv_lens, const T* __restrict__ k_cache,
    const T* __restrict__ v_cache, const int32_t* __restrict__ page_table, const int32_t* __restrict__ block_idx,
    float scale, T* __restrict__ out, float* __restrict__ lse, int q_len, int Hq, int Hkv, int bs, int top_k,
    int num_pages, int pt_stride, long long rows, gate_args ga) {
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
    const int jj = block_id(j, pt_stride);
    const int p = page_id(page_table[(size_t)b * pt_stride + jj], num_pages);
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
  const size_t orow = ((size_t)b * Hq + h) * q_len + t;
  T* op = out + orow * D;
#pragma unroll
  for (int i = 0; i < DPL; i++) {
    float a = acc[i] * inv;
    if (ga.g) {                                        // out = g A + (1 - g) x, one rounding
      const int d = lane + 64 * i;
      const float gv = ga.per_dim ? ga.g[orow * D + d] : ga.g[orow];
      a = gv * a + (1.0f - gv) * ld_any(static_cast<const T*>(ga.x) + orow * D + d);
    }
    st_any(op + lane + 64 * i, a);
  }
  if (lse && lane == 0) lse[((size_t)b * Hq + h) * q_len + t] = m + logf(l);
}

static int mfma_heads_per_tile(int G) {
  // largest power of two dividing G, capped at 32 (a wave holds 32 rows)
  int hg = 1;
  while (hg < 32 && (G % (hg * 2)) == 0) hg *= 2;
  return hg;
}

hipError_t launch_attn_prefill(const bsg_dims& d, const void* q, int q_len, const int32_t* kv_lens,
                               const void* k_cache, const void* v_cache, const int32_t* page_table,
                               const int32_t* block_idx, float scale, void* out, float* lse,
                               hipStream_t stream, gate_args ga) {
  const int G = d.num_q_heads / d.num_kv_heads;
  if (d.dtype == BSG_BF16) {
    const int HG = mfma_heads_per_tile(G);
    const int TT = PF_ROWS / HG;
    const int nbw = (d.pt_stride + 31) / 32;
    const int ucap = TT * d.top_k < d.pt_stride ? TT * d.top_k : d.pt_stride;
    const size_t fixed = (size_t)TT * d.top_k * 4 + (size_t)nbw * 4 + (size_t)ucap * 8;
    const size_t stage = (size_t)2 * PF_SUB * d.head_dim * 2;
    int nst = PF_MAX_STAGES;                       // deepest ring that fits the 160 KiB of LDS
    while (nst > 2 && fixed + nst * stage > 160 * 1024) nst--;
    const size_t smem = fixed + nst * stage;
    // the output rows are staged over the ring (and the schedule after it) at the end
    const size_t ostage = (size_t)PF_ROWS * (d.head_dim + 8) * 2;
    if (smem <= 160 * 1024 && smem >= ostage) {
      const int n_tt = (q_len + TT - 1) / TT;
      const long long nwg = (long long)n_tt * d.num_kv_heads * (G / HG) * d.batch;
      if (nwg < (1LL << 31)) {
        dim3 grid((unsigned)nwg);
#define BSG_PF(DD, BB)                                                                                       \
  do {                                                                                                        \
    auto kfn = nst == 4 ? attn_prefill_mfma_kernel<DD, BB, true> : attn_prefill_mfma_kernel<DD, BB, false>;   \
    { hipError_t ea_ = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem); if (ea_ != hipSuccess) return ea_; } \
    hipLaunchKernelGGL(kfn, grid, dim3(64 * PF_WAVES), smem, stream, (const bf16_t*)q, kv_lens,             \
                       (const bf16_t*)k_cache, (const bf16_t*)v_cache, page_table, block_idx, scale,          \
                       (bf16_t*)out, lse, q_len, d.num_q_heads, d.num_kv_heads, HG, d.top_k, d.num_pages,    \
                       d.pt_stride, n_tt, nst, ga);                                                           \
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
  }
  const long long rows = (long long)d.batch * d.num_q_heads * q_len;
  dim3 grid((unsigned)((rows + 3) / 4));
#define BSG_PV(T, DD)                                                                                          \
  hipLaunchKernelGGL((attn_prefill_valu_kernel<T, DD>), grid, dim3(256), 0, stream, (const T*)q, kv_lens,       \
                     (const T*)k_cache, (const T*)v_cache, page_table, block_idx, scale, (T*)out, lse, q_len,   \
                     d.num_q_heads, d.num_kv_heads, d.page_size, d.top_k, d.num_pages, d.pt_stride, rows, ga)
  if (d.dtype == BSG_BF16) {
    if (d.head_dim == 128) BSG_PV(bf16_t, 128); else BSG_PV(bf16_t, 64);
  } else {
    if (d.head_dim == 128) BSG_PV(float, 128); else BSG_PV(float, 64);
  }
#undef BSG_PV
  return hipGetLastError();
}

BSG_DEBUG_FILE(attn_prefill)

}  // namespace bsg
