// Exact top-(k-1) selection from per-chunk sorted key lists (decode), shared by the fused
// decode step (inside the attention kernel) and the stand-alone decode selection kernel.
#pragma once

#include "bsg_device.h"

namespace bsg {

// Number of keys in a[0, n) that are larger than key; a is 16-byte aligned and read two
// keys per 16-byte load, 16 keys per batch.
__device__ __forceinline__ int count_above(const uint64_t* a, int n, uint64_t key) {
  int rank = 0, i = 0;
  for (; i + 16 <= n; i += 16) {
    ulonglong2 v[8];
#pragma unroll
    for (int u = 0; u < 8; u++) v[u] = reinterpret_cast<const ulonglong2*>(a + i)[u];
#pragma unroll
    for (int u = 0; u < 8; u++) rank += (v[u].x > key ? 1 : 0) + (v[u].y > key ? 1 : 0);
  }
  for (; i < n; i++) rank += a[i] > key ? 1 : 0;
  return rank;
}

// Leading keys of every chunk list the prologue reads at first: the tops (2^lt) and at least
// 8, at most the list length m.
__host__ __device__ inline int decode_prologue_lead(int m, int lt) {
  const int t = 1 << lt;
  const int f = t > 8 ? t : 8;
  return f < m ? f : m;
}

// Selection prologue of the fused decode step (one workgroup, all threads).  `lists` holds,
// per chunk of candidate blocks, the chunk's best m = top_k - 1 keys sorted descending (0 =
// none).  The cnt-th largest of the chunks' first T keys (the tops) is a lower bound `tau` of
// the cnt-th largest key overall (at least cnt keys reach it), so the kept keys are among the
// list keys >= tau, and those are a prefix of every list: typically little more than cnt keys
// in all.  Steps: the first F keys of every list go to LDS (one round trip); tau is found
// among the tops at or above the cnt-th largest of 64 disjoint group maxima of the tops (itself
// a lower bound, so the cnt-th largest top is among them); each chunk's prefix >= tau is
// gathered (read on from memory in the rare case that it runs past F); the survivors are
// ranked against each other and sel[r] receives the block id of rank r (r < cnt, largest score
// first).  smem: decode_prologue_smem_bytes.
__device__ void decode_select_prologue(const uint64_t* __restrict__ lists_row, int nchunks, int m, int lt, int cnt,
                                       uint64_t* smem, int* sel, int* counter, uint64_t* tau_s) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int T = 1 << lt;                      // leading keys of every list that are tops
  const int F = decode_prologue_lead(m, lt);  // leading keys read at first
  const int TT = T < F ? T : F;               // tops that exist (T > m only past the list end)
  const int NT = nchunks * TT;
  const int NP = nchunks * F;
  uint64_t* P = smem;                                     // [nchunks][F]
  uint64_t* S = smem + ((NP + 1) & ~1);                   // candidates of tau, then survivors
  if (tid == 0) {
    *counter = 0;
    *tau_s = 1ull;
  }
  // 1. the leading keys, 8 loads in flight per thread
  constexpr int LU = 8;
  for (int e0 = 0; e0 < NP; e0 += LU * 256) {
    uint64_t v[LU];
#pragma unroll
    for (int u = 0; u < LU; u++) {
      const int e = e0 + u * 256 + tid;
      const int c = e / F;
      v[u] = e < NP ? lists_row[(size_t)c * m + (e - c * F)] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < LU; u++) {
      const int e = e0 + u * 256 + tid;
      if (e < NP) P[e] = v[u];
    }
  }
  __syncthreads();
  // 2a. wave 0: the cnt-th largest of 64 group maxima (group l: tops l, l + 64, ...); with fewer
  // than cnt non-empty groups the bound stays 1 (every top is a candidate)
  __shared__ uint64_t tau0_s;
  if (wave == 0) {
    uint64_t gm = 0ull;
    for (int e = lane; e < NT; e += 64) {
      const int c = e / TT;
      const uint64_t k = P[c * F + (e - c * TT)];
      gm = k > gm ? k : gm;
    }
    int rank = 0;
    for (int o = 0; o < 64; o++) {
      const uint64_t x = ((uint64_t)(uint32_t)__shfl((int)(gm >> 32), o, 64) << 32) |
                         (uint64_t)(uint32_t)__shfl((int)(uint32_t)gm, o, 64);
      rank += x > gm ? 1 : 0;
    }
    // the non-empty maxima are distinct (keys hold the block index): at most one lane has rank
    // cnt - 1
    const uint64_t hit = __ballot(gm != 0ull && rank == cnt - 1);
    if (lane == 0) tau0_s = hit ? 0ull : 1ull;
    if (hit && lane == (int)__builtin_ctzll(hit)) tau0_s = gm;
  }
  __syncthreads();
  const uint64_t tau0 = tau0_s;
  // 2b. the tops >= tau0 (all tops at or above the cnt-th largest one) to S, then the exact
  // cnt-th largest of them
  for (int e = tid; e < NT; e += 256) {
    const int c = e / TT;
    const uint64_t k = P[c * F + (e - c * TT)];
    if (k != 0ull && k >= tau0) S[atomicAdd(counter, 1)] = k;
  }
  __syncthreads();
  const int nc2 = *counter;
  for (int e = tid; e < nc2; e += 256) {
    const uint64_t key = S[e];
    if (count_above(S, nc2, key) == cnt - 1) *tau_s = key;
  }
  __syncthreads();
  const uint64_t tau = *tau_s;                 // 1 if fewer than cnt tops exist: every key
  if (tid == 0) *counter = 0;
  __syncthreads();
  // 3. survivors: every list's prefix >= tau (tau >= 1, so no empty slot), read on from memory
  // past the first F keys
  for (int c = tid; c < nchunks; c += 256) {
    const uint64_t* lc = lists_row + (size_t)c * m;
    int s = 0;
    while (s < F && P[c * F + s] >= tau) s++;
    int more = 0;                               // prefix keys past the first F, 8 per round trip
    if (s == F) {
      for (int i0 = F; i0 < m; i0 += 8) {
        uint64_t v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) v[u] = i0 + u < m ? lc[i0 + u] : 0ull;
        int k = 0;
        while (k < 8 && v[k] >= tau) k++;       // 0 past the list end stops it (tau >= 1)
        more += k;
        if (k < 8) break;
      }
    }
    if (s + more > 0) {
      const int base = atomicAdd(counter, s + more);
      for (int i = 0; i < s; i++) S[base + i] = P[c * F + i];
      for (int i = 0; i < more; i++) S[base + s + i] = lc[F + i];
    }
  }
  __syncthreads();
  const int ns = *counter;
  for (int e = tid; e < ns; e += 256) {
    const uint64_t key = S[e];
    const int rank = count_above(S, ns, key);
    if (rank < cnt) sel[rank] = sel_key_index(key);
  }
  __syncthreads();
}


// Leading keys (2^lt) the prologue takes from every chunk list: chunks * 2^lt >= 2 (k - 1),
// and no more than the list length.
inline int decode_prologue_lt(int nchunks, int m) {
  int lt = 0;
  while (m > 0 && (nchunks << lt) < 2 * m && (1 << lt) < m) lt++;
  return lt;
}

// LDS of the prologue: the lists' leading keys, then the candidates of tau / the survivors
// (at most every list key, or every top), 16-byte aligned.
inline size_t decode_prologue_smem_bytes(int nchunks, int m, int lt) {
  const int mm = m > 0 ? m : 1;
  const size_t np = (size_t)nchunks * decode_prologue_lead(mm, lt);
  const size_t nl = (size_t)nchunks * mm;
  const size_t nt = (size_t)nchunks << lt;
  return (((np + 1) & ~(size_t)1) + (nl > nt ? nl : nt)) * sizeof(uint64_t);
}

}  // namespace bsg
