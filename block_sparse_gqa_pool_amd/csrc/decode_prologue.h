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

// Selection prologue of the fused decode step (one workgroup, all threads).  `lists` holds,
// per chunk of candidate blocks, the chunk's best m = top_k - 1 keys sorted descending (0 =
// none).  The cnt-th largest of the chunks' first T keys is a lower bound `tau` of the
// cnt-th largest key overall (at least cnt keys reach it), so the kept keys are among the
// list keys >= tau, typically little more than cnt keys in all.  Those survivors are
// ranked against each other; sel[r] receives the block id of rank r (r < cnt, largest
// score first).
__device__ void decode_select_prologue(const uint64_t* __restrict__ lists_row, int nchunks, int m, int lt, int cnt,
                                       uint64_t* L, uint64_t* S, int* sel, int* counter, uint64_t* tau_s) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int T = 1 << lt;                      // leading keys taken from every chunk list
  const int NT = nchunks << lt;
  const int NL = nchunks * m;
  uint64_t* tops = S;                         // [NT], reused for the survivors afterwards
  if (tid == 0) {
    *counter = 0;
    *tau_s = 1ull;
  }
  // lists -> LDS, 16 loads in flight per thread (32 KiB per workgroup round trip: the lists
  // of a 16K-block row take two); a list's first T keys also go to tops
  constexpr int LU = 16;
  for (int e0 = 0; e0 < NL; e0 += LU * 256) {
    uint64_t v[LU];
#pragma unroll
    for (int u = 0; u < LU; u++) {
      const int e = e0 + u * 256 + tid;
      v[u] = e < NL ? lists_row[e] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < LU; u++) {
      const int e = e0 + u * 256 + tid;
      if (e < NL) {
        L[e] = v[u];
        const int c = e / m, i = e - c * m;
        if (i < T) tops[(c << lt) + i] = v[u];
      }
    }
  }
  if (T > m)                                  // positions past the list length hold no key
    for (int e = tid; e < NT; e += 256)
      if ((e & (T - 1)) >= m) tops[e] = 0ull;
  __syncthreads();
  // tau = the cnt-th largest top.  With fewer than cnt tops set, no set top has cnt - 1
  // above it, and tau stays 1: every key survives.
  for (int e = tid; e < NT; e += 256) {
    const uint64_t key = tops[e];
    if (key != 0ull && count_above(tops, NT, key) == cnt - 1) *tau_s = key;
  }
  __syncthreads();
  const uint64_t tau = *tau_s;
  // survivors: the list keys >= tau (tau >= 1, so no empty slot), compacted per wave; their
  // order does not matter
  for (int e0 = 0; e0 < NL; e0 += 256) {
    const int e = e0 + tid;
    const uint64_t key = e < NL ? L[e] : 0ull;
    const bool keep = key >= tau;
    const uint64_t bal = __ballot(keep);
    if (bal != 0ull) {
      int base = 0;
      if (lane == 0) base = atomicAdd(counter, __popcll(bal));
      base = __shfl(base, 0, 64);
      if (keep) S[base + __popcll(bal & ((1ull << lane) - 1ull))] = key;
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

// LDS of the prologue: the lists, then the tops / survivors (16-byte aligned).
inline size_t decode_prologue_smem_bytes(int nchunks, int m, int lt) {
  const size_t nl = (size_t)nchunks * (m > 0 ? m : 1);
  const size_t nt = (size_t)nchunks << lt;
  return (((nl + 1) & ~(size_t)1) + (nl > nt ? nl : nt)) * sizeof(uint64_t);
}

}  // namespace bsg
