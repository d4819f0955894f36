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
#include "decode_prologue.h"

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
    const int jj = block_id(j, pt_stride);
    const int p = page_id(page_table[(size_t)b * pt_stride + jj], num_pages);
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
                                                              float* __restrict__ lse, int Hq, int Hkv, int nsplit,
                                                              gate_args ga) {
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh % Hq;
  const int G = Hq / Hkv;
  const int g = h / G, hh = h % G;
  const int d = threadIdx.x;
  const float* base = ws + (((size_t)b * Hkv + g) * nsplit) * G * (D + 2) + (size_t)hh * (D + 2);
  const size_t sstride = (size_t)G * (D + 2);
  // all partials of the row in one batch of loads (up to 8 splits per pass)
  float m = -INFINITY, l = 0.0f, o = 0.0f;
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    float ms[8], ls[8], os[8];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int s = s0 + u;
      const bool v = s < nsplit;
      ms[u] = v ? base[s * sstride] : -INFINITY;
      ls[u] = v ? base[s * sstride + 1] : 0.0f;
      os[u] = v ? base[s * sstride + 2 + d] : 0.0f;
    }
    float mn = m;
#pragma unroll
    for (int u = 0; u < 8; u++) mn = fmaxf(mn, ms[u]);
    if (mn != -INFINITY) {
      const float sc = m == -INFINITY ? 0.0f : __expf(m - mn);
      l *= sc;
      o *= sc;
#pragma unroll
      for (int u = 0; u < 8; u++) {
        if (ms[u] == -INFINITY) continue;
        const float w = __expf(ms[u] - mn);
        l += ls[u] * w;
        o += os[u] * w;
      }
      m = mn;
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const size_t row = (size_t)b * Hq + h;
  float a = o * inv;
  if (ga.g) {                                          // out = g A + (1 - g) x, one rounding
    const float gv = ga.per_dim ? ga.g[row * D + d] : ga.g[row];
    a = gv * a + (1.0f - gv) * ld_any(static_cast<const T*>(ga.x) + row * D + d);
  }
  st_any(out + row * D + d, a);
  if (lse && d == 0) lse[(size_t)b * Hq + h] = m + logf(l);
}

// ---------------------------------------------------------------------------------------
// bf16 matrix-core path (G <= 16).  Each wave takes `ppw` selected pages of one (sequence,
// group) and runs, per 64-key sub-block,
//   S^T (16 keys x 16 heads) = K (keys x D) . Q^T (D x heads)    A = K rows straight from HBM
//   O^T (16 d x 16 heads)   += V^T (d x 32 keys) . P^T (keys x heads)   A = V^T from LDS via
//                                                                  ds_read_b64_tr_b16
// with v_mfma_f32_16x16x32_bf16 (heads beyond G are zero columns).  A head's scores sit in
// the four lanes with the same lane % 16, so the online softmax needs two shuffles.  The
// four waves of a workgroup merge in LDS and the workgroup writes one partial per head;
// attn_decode_merge_kernel then merges the workgroups.
namespace {
constexpr int DM_VPAD = 16;
}

typedef __attribute__((address_space(3))) s16x4_t* dm_lds_s16x4_ptr;

// F8: K and V are OCP E4M3 codes with one scale per (page, head).  Codes become bf16
// exactly; the K scale multiplies the page's scores and the V scale the page's
// probabilities before their bf16 rounding (both powers of two, so both products are
// exact and the result equals the bf16 path on the decoded cache).
template <int D, int BS, bool FUSED, bool F8>
__global__ __launch_bounds__(256, 2) void attn_decode_mfma_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ kv_lens, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const int32_t* __restrict__ page_table, int32_t* __restrict__ block_idx,
    const uint64_t* __restrict__ lists, float scale, float* __restrict__ part, int Hq, int Hkv, int top_k,
    int num_pages, int pt_stride, int nwg, int ppw, int nchunks, int lt, const float* __restrict__ k_scales,
    const float* __restrict__ v_scales, int nunits) {
  constexpr int NDS = D / 32;          // k-steps of the score product
  constexpr int NDT = D / 16;          // 16-wide d tiles of the output
  constexpr int VS = D + DM_VPAD;      // LDS row stride of V (elements)
  constexpr int SUB = 64;              // keys per sub-block
  extern __shared__ __attribute__((aligned(16))) unsigned char dm_smem[];
  const int G = Hq / Hkv;
  // workgroup x is workgroup (x / 8) % nwg of unit (x / 8 nwg) * 8 + x % 8: the nwg workgroups
  // of a (sequence, group) unit sit 8 apart in dispatch order, so on the same XCD (workgroups
  // go to the eight XCDs in turn), and the unit's selection lists come from memory once into
  // that XCD's L2
  const int xw = blockIdx.x;
  const int split = (xw >> 3) % nwg;
  const int unit = (xw / (8 * nwg)) * 8 + (xw & 7);
  if (unit >= nunits) return;
  const int g = unit % Hkv, b = unit / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, qd = lane >> 4;
  bf16_t* Vs = reinterpret_cast<bf16_t*>(dm_smem) + (size_t)wave * SUB * VS;
  const int L = kv_lens[b];
  const int pos = L - 1;
  int32_t* sl = block_idx + ((size_t)b * Hkv + g) * top_k;
  const float c2 = scale * 1.4426950408889634f;
  __shared__ int wl[64];          // fused: the selection in rank order, own block at [cnt]
  __shared__ int cnt_s;
  __shared__ uint64_t tau_s;
  if (FUSED) {
    const int m = top_k - 1;
    const int own = max(pos, 0) / BS;
    const int cnt = min(m, min(own, pt_stride));
    if (cnt > 0) {
      uint64_t* Lk = reinterpret_cast<uint64_t*>(dm_smem);
      decode_select_prologue(lists + ((size_t)b * Hkv + g) * nchunks * m, nchunks, m, lt, cnt, Lk, wl, &cnt_s,
                             &tau_s);
    }
    if (tid == 0) wl[cnt] = own;
    for (int i = cnt + 1 + tid; i < top_k; i += 256) wl[i] = -1;
    __syncthreads();
  }

  bf16x8_t qb[NDS];
  {
    const bool hv = n < G;
    const bf16_t* qp = q + ((size_t)b * Hq + (size_t)g * G + (hv ? n : 0)) * D + 8 * qd;
#pragma unroll
    for (int s = 0; s < NDS; s++) {
      uint4 v = hv ? *reinterpret_cast<const uint4*>(qp + 32 * s) : make_uint4(0, 0, 0, 0);
      qb[s] = *reinterpret_cast<bf16x8_t*>(&v);
    }
  }
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4_t o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; i++) o[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int vtr = (16 * 0 + 4 * qd + ((lane & 15) >> 2)) * VS + 4 * (lane & 3);   // tr-read base (key, d)

  const int e0 = (split * 4 + wave) * ppw;
  const int e1 = min(e0 + min(ppw, 2), top_k);         // ppw is 1 or 2
  // the wave's block ids and their pages, fetched together
  int jv[2], pv[2];
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const int e = e0 + t;
    jv[t] = e < e1 ? (FUSED ? wl[e] : sl[e]) : -1;
  }
#pragma unroll
  for (int t = 0; t < 2; t++)
    pv[t] = jv[t] >= 0 ? page_table[(size_t)b * pt_stride + block_id(jv[t], pt_stride)] : 0;
  constexpr int ES = F8 ? 1 : 2;                        // bytes per K/V element
  constexpr int NSP = BS / SUB;                         // sub-blocks per page
  constexpr int PPR = D / 8;                            // 8-element pieces per row
  constexpr int NV = SUB * PPR / 64;                    // V pieces per lane per sub-block
  const char* kpg[2];
  const char* vpg[2];
  int nkp[2];
  float skp[2], svp[2];
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const int jj = clampi(jv[t], 0, pt_stride - 1);
    const int p = page_id(pv[t], num_pages);
    nkp[t] = jv[t] >= 0 ? clampi(pos - jj * BS + 1, 0, BS) : 0;
    kpg[t] = reinterpret_cast<const char*>(k_cache) + (((size_t)p * Hkv + g) * BS) * D * ES;
    vpg[t] = reinterpret_cast<const char*>(v_cache) + (((size_t)p * Hkv + g) * BS) * D * ES;
    skp[t] = F8 ? k_scales[(size_t)p * Hkv + g] : 1.0f;
    svp[t] = F8 ? v_scales[(size_t)p * Hkv + g] : 1.0f;
  }
  // Raw K/V of one sub-block.  All its loads go out before its first product, so the wave
  // waits for memory once per sub-block; V rows past nk (inside the page) are loaded too and
  // zeroed on their way to LDS; K rows past nk give scores that are masked.
  struct Raw {
    uint4 v[F8 ? 1 : NV];
    uint2 v8[F8 ? NV : 1];
    uint4 k[F8 ? 1 : SUB / 16][NDS];
    uint2 k8[F8 ? SUB / 16 : 1][NDS];
  };
  auto load = [&](int t, int h2, Raw& rw) {
    const int kb = h2 * SUB;
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int pc = i * 64 + lane;
      const int r = pc / PPR, c = pc % PPR;
      const char* src = vpg[t] + ((size_t)(kb + r) * D + 8 * c) * ES;
      if constexpr (F8) rw.v8[i] = *reinterpret_cast<const uint2*>(src);
      else rw.v[i] = *reinterpret_cast<const uint4*>(src);
    }
#pragma unroll
    for (int T = 0; T < SUB / 16; T++) {
      const char* kr = kpg[t] + ((size_t)(kb + 16 * T + n) * D + 8 * qd) * ES;
#pragma unroll
      for (int s2 = 0; s2 < NDS; s2++) {
        if constexpr (F8) rw.k8[T][s2] = *reinterpret_cast<const uint2*>(kr + 32 * s2);
        else rw.k[T][s2] = *reinterpret_cast<const uint4*>(kr + 64 * s2);
      }
    }
  };
  auto compute = [&](int t, int h2, const Raw& rw) {
    const int kb = h2 * SUB;
    const int nk = nkp[t];
    // scores: S^T tiles of 16 keys
    f32x4_t sacc[SUB / 16];
#pragma unroll
    for (int T = 0; T < SUB / 16; T++) {
      sacc[T] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s2 = 0; s2 < NDS; s2++) {
        bf16x8_t ka;
        if constexpr (F8) ka = e4m3x8_to_bf16(rw.k8[T][s2]);
        else ka = *reinterpret_cast<const bf16x8_t*>(&rw.k[T][s2]);
        sacc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[s2], sacc[T], 0, 0, 0);
      }
      if constexpr (F8) sacc[T] *= skp[t];
    }
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int pc = i * 64 + lane;
      const int r = pc / PPR, c = pc % PPR;
      const bool ok = kb + r < nk;
      if constexpr (F8) {
        const bf16x8_t v = e4m3x8_to_bf16(ok ? rw.v8[i] : make_uint2(0, 0));
        *reinterpret_cast<bf16x8_t*>(Vs + r * VS + 8 * c) = v;
      } else {
        *reinterpret_cast<uint4*>(Vs + r * VS + 8 * c) = ok ? rw.v[i] : make_uint4(0, 0, 0, 0);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int T = 0; T < SUB / 16; T++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int key = kb + 16 * T + 4 * qd + i;
        const float sc = key < nk ? sacc[T][i] : -INFINITY;
        sacc[T][i] = sc;
        mx = fmaxf(mx, sc);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
    m_run = m_new;
    float rs = 0.0f;
#pragma unroll
    for (int T = 0; T < SUB / 16; T++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float pe = __builtin_amdgcn_exp2f((sacc[T][i] - m_use) * c2);
        sacc[T][i] = pe;
        rs += pe;
      }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int i = 0; i < NDT; i++) o[i] *= alpha;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int k2 = 0; k2 < SUB / 32; k2++) {
      bf16x8_t pb;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        pb[i] = (__bf16)(F8 ? sacc[2 * k2][i] * svp[t] : sacc[2 * k2][i]);
        pb[4 + i] = (__bf16)(F8 ? sacc[2 * k2 + 1][i] * svp[t] : sacc[2 * k2 + 1][i]);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; dt++) {
        const bf16_t* vb = Vs + vtr + (32 * k2) * VS + 16 * dt;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dm_lds_s16x4_ptr)(vb));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dm_lds_s16x4_ptr)(vb + 16 * VS));
        bf16x8_t va;
        *reinterpret_cast<s16x4_t*>(&va) = lo;
        *(reinterpret_cast<s16x4_t*>(&va) + 1) = hi;
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // units u = (page u / NSP, sub-block u % NSP); a unit exists if its first key is valid
  auto valid = [&](int u) { return (u % NSP) * SUB < nkp[u / NSP]; };
  if constexpr (F8 && NSP == 1) {
    // fp8 sub-blocks take half the registers: with one sub-block per page the next page's
    // loads are in flight while this one is computed
    Raw rw[2];
    if (valid(0)) load(0, 0, rw[0]);
#pragma unroll
    for (int u = 0; u < 2 * NSP; u++) {
      if (u + 1 < 2 * NSP && valid(u + 1)) load((u + 1) / NSP, (u + 1) % NSP, rw[(u + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      if (valid(u)) compute(u / NSP, u % NSP, rw[u & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int u = 0; u < 2 * NSP; u++) {
      if (!valid(u)) continue;
      Raw rw;
      load(u / NSP, u % NSP, rw);
      __builtin_amdgcn_sched_barrier(0);
      compute(u / NSP, u % NSP, rw);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (FUSED && split == 0) {  // the selection, ascending, to block_idx (own block last)
    for (int i = tid; i < top_k; i += 256) {
      const int v = wl[i];
      int r = i;
      if (v >= 0) {
        r = 0;
        for (int i2 = 0; i2 < top_k; i2++) {
          const int o = wl[i2];
          r += (o >= 0 && o < v) ? 1 : 0;
        }
      }
      sl[r] = v;
    }
  }
  // per-head sum over the four lanes of the head
  float l_h = l_run + __shfl_xor(l_run, 16, 64);
  l_h += __shfl_xor(l_h, 32, 64);

  // workgroup merge of the four waves (LDS), then this workgroup's partial to HBM
  __syncthreads();
  float* mrg = reinterpret_cast<float*>(dm_smem);               // [4][16][D + 2]
  {
    float* mw = mrg + ((size_t)wave * 16 + n) * (D + 2);
    if (qd == 0) {
      mw[0] = m_run;
      mw[1] = l_h;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; dt++)
#pragma unroll
      for (int i = 0; i < 4; i++) mw[2 + 16 * dt + 4 * qd + i] = o[dt][i];
  }
  __syncthreads();
  const size_t pstride = (size_t)G * (D + 2);
  float* myp = part + (((size_t)b * Hkv + g) * nwg + split) * pstride;
  for (int e = tid; e < G * D; e += 256) {
    const int h = e / D, d = e % D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; w++) mm = fmaxf(mm, mrg[((size_t)w * 16 + h) * (D + 2)]);
    float ll = 0.0f, oo = 0.0f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; w++) {
        const float* mw = mrg + ((size_t)w * 16 + h) * (D + 2);
        if (mw[0] == -INFINITY) continue;
        const float sc = __builtin_amdgcn_exp2f((mw[0] - mm) * c2);
        ll += mw[1] * sc;
        oo += mw[2 + d] * sc;
      }
    }
    myp[h * (D + 2) + 2 + d] = oo;
    if (d == 0) {
      myp[h * (D + 2)] = mm == -INFINITY ? -INFINITY : mm * scale;   // natural-log units
      myp[h * (D + 2) + 1] = ll;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Attention over a token list (token-level and two-level selection): the decode kernel above
// with its 64-key sub-blocks taken from consecutive entries of the row's ascending token list
// instead of one page.  Each lane looks up the page of one entry; a key row's address then
// reaches the lanes that read it by shuffle.  Entries are kept tokens followed by -1 padding,
// so the valid keys of a sub-block are a prefix of it.  A row is one query position of one
// sequence (RowWindow): decode rows split their list over nwg workgroups and leave partials
// for attn_decode_merge_kernel; with nwg = 1 (prefill rows, each a workgroup of its own) the
// wave takes ppw sub-blocks, two at a time, and the workgroup writes out and lse itself.
template <int D, int BS>
__global__ __launch_bounds__(256, 2) void attn_decode_tokens_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ kv_lens, const bf16_t* __restrict__ k_cache,
    const bf16_t* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ token_idx, int Kt, float scale, float* __restrict__ part, int Hq, int Hkv,
    int num_pages, int pt_stride, int nwg, int ppw, RowWindow rw, bf16_t* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int NDS = D / 32;
  constexpr int NDT = D / 16;
  constexpr int VS = D + DM_VPAD;
  constexpr int SUB = 64;
  constexpr int PPR = D / 8;
  constexpr int NV = SUB * PPR / 64;
  extern __shared__ __attribute__((aligned(16))) unsigned char dm_smem[];
  const int G = Hq / Hkv;
  // rows last first: a prefill row's list is shorter the earlier its position, so those fill the end
  const int g = blockIdx.y, rl = (int)gridDim.z - 1 - (int)blockIdx.z;
  const int b = rw.seq(rl), tq = rw.pos(rl);
  if (tq >= rw.T) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, qd = lane >> 4;
  bf16_t* Vs = reinterpret_cast<bf16_t*>(dm_smem) + (size_t)wave * SUB * VS;
  const float c2 = scale * 1.4426950408889634f;
  const int32_t* trow = token_idx + (((size_t)b * Hkv + g) * rw.T + tq) * Kt;
  (void)kv_lens;

  bf16x8_t qb[NDS];
  {
    const bool hv = n < G;
    const bf16_t* qp = q + (((size_t)b * Hq + (size_t)g * G + (hv ? n : 0)) * rw.T + tq) * D + 8 * qd;
#pragma unroll
    for (int s = 0; s < NDS; s++) {
      uint4 v = hv ? *reinterpret_cast<const uint4*>(qp + 32 * s) : make_uint4(0, 0, 0, 0);
      qb[s] = *reinterpret_cast<bf16x8_t*>(&v);
    }
  }
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4_t o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; i++) o[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int vtr = (4 * qd + ((lane & 15) >> 2)) * VS + 4 * (lane & 3);

  // this wave's sub-blocks of the list, two at a time: tokens, then their pages, together
  for (int i0 = 0; i0 < ppw; i0 += 2) {
  const int u0 = (blockIdx.x * 4 + wave) * ppw + i0;
  int tok[2];
  long long rb[2];
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const int e = (u0 + t) * SUB + lane;
    tok[t] = (i0 + t < ppw && e < Kt) ? trow[e] : -1;
  }
#pragma unroll
  for (int t = 0; t < 2; t++) {
    dbg_flag(tok[t] >= pt_stride * BS, DBG_TOKEN_ID);
    const int pid = tok[t] >= 0 ? page_id(page_table[(size_t)b * pt_stride + min(tok[t] / BS, pt_stride - 1)],
                                          num_pages)
                                : 0;
    rb[t] = tok[t] >= 0 ? ((((long long)pid * Hkv + g) * BS + tok[t] % BS) * D) : 0;
  }
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const int nk = __popcll(__ballot(tok[t] >= 0));     // valid keys: a prefix of the sub-block
    if (nk == 0) break;
    uint4 vr[NV];
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int pc = i * 64 + lane;
      const long long base = __shfl(rb[t], pc / PPR, 64);
      vr[i] = *reinterpret_cast<const uint4*>(v_cache + base + 8 * (pc % PPR));
    }
    uint4 kr[SUB / 16][NDS];
#pragma unroll
    for (int T = 0; T < SUB / 16; T++) {
      const long long base = __shfl(rb[t], 16 * T + n, 64);
#pragma unroll
      for (int s2 = 0; s2 < NDS; s2++) kr[T][s2] = *reinterpret_cast<const uint4*>(k_cache + base + 8 * qd + 32 * s2);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4_t sacc[SUB / 16];
#pragma unroll
    for (int T = 0; T < SUB / 16; T++) {
      sacc[T] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s2 = 0; s2 < NDS; s2++)
        sacc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8_t*>(&kr[T][s2]), qb[s2],
                                                            sacc[T], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int pc = i * 64 + lane;
      const int r = pc / PPR, c = pc % PPR;
      *reinterpret_cast<uint4*>(Vs + r * VS + 8 * c) = r < nk ? vr[i] : make_uint4(0, 0, 0, 0);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int T = 0; T < SUB / 16; T++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int key = 16 * T + 4 * qd + i;
        const float sc = key < nk ? sacc[T][i] : -INFINITY;
        sacc[T][i] = sc;
        mx = fmaxf(mx, sc);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
    m_run = m_new;
    float rs = 0.0f;
#pragma unroll
    for (int T = 0; T < SUB / 16; T++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float pe = __builtin_amdgcn_exp2f((sacc[T][i] - m_use) * c2);
        sacc[T][i] = pe;
        rs += pe;
      }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int i = 0; i < NDT; i++) o[i] *= alpha;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int k2 = 0; k2 < SUB / 32; k2++) {
      bf16x8_t pb;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        pb[i] = (__bf16)sacc[2 * k2][i];
        pb[4 + i] = (__bf16)sacc[2 * k2 + 1][i];
      }
#pragma unroll
      for (int dt = 0; dt < NDT; dt++) {
        const bf16_t* vb = Vs + vtr + (32 * k2) * VS + 16 * dt;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dm_lds_s16x4_ptr)(vb));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dm_lds_s16x4_ptr)(vb + 16 * VS));
        bf16x8_t va;
        *reinterpret_cast<s16x4_t*>(&va) = lo;
        *(reinterpret_cast<s16x4_t*>(&va) + 1) = hi;
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __builtin_amdgcn_sched_barrier(0);
  }
  }  // pairs of sub-blocks
  float l_h = l_run + __shfl_xor(l_run, 16, 64);
  l_h += __shfl_xor(l_h, 32, 64);
  __syncthreads();
  float* mrg = reinterpret_cast<float*>(dm_smem);               // [4][16][D + 2]
  {
    float* mw = mrg + ((size_t)wave * 16 + n) * (D + 2);
    if (qd == 0) {
      mw[0] = m_run;
      mw[1] = l_h;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; dt++)
#pragma unroll
      for (int i = 0; i < 4; i++) mw[2 + 16 * dt + 4 * qd + i] = o[dt][i];
  }
  __syncthreads();
  const size_t pstride = (size_t)G * (D + 2);
  float* myp = part + (((size_t)rl * Hkv + g) * nwg + blockIdx.x) * pstride;
  for (int e = tid; e < G * D; e += 256) {
    const int h = e / D, d = e % D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; w++) mm = fmaxf(mm, mrg[((size_t)w * 16 + h) * (D + 2)]);
    float ll = 0.0f, oo = 0.0f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; w++) {
        const float* mw = mrg + ((size_t)w * 16 + h) * (D + 2);
        if (mw[0] == -INFINITY) continue;
        const float sc = __builtin_amdgcn_exp2f((mw[0] - mm) * c2);
        ll += mw[1] * sc;
        oo += mw[2 + d] * sc;
      }
    }
    if (nwg == 1) {                                  // the whole list: the final row
      const size_t row = ((size_t)b * Hq + (size_t)g * G + h) * rw.T + tq;
      out[row * D + d] = f32_to_bf16(oo * (ll > 0.0f ? 1.0f / ll : 0.0f));
      if (lse && d == 0) lse[row] = mm == -INFINITY ? -INFINITY : mm * scale + logf(ll);
      continue;
    }
    myp[h * (D + 2) + 2 + d] = oo;
    if (d == 0) {
      myp[h * (D + 2)] = mm == -INFINITY ? -INFINITY : mm * scale;
      myp[h * (D + 2) + 1] = ll;
    }
  }
}

static int token_attn_ppw(const bsg_dims& d, int Kt) {
  const long long units = (Kt + 63) / 64;
  const long long wg2 = (long long)d.batch * d.num_kv_heads * ((units + 7) / 8);
  return wg2 >= 512 ? 2 : 1;
}

static int token_attn_nwg(const bsg_dims& d, int Kt) {
  const int ppw = token_attn_ppw(d, Kt);
  const int units = (Kt + 63) / 64;
  return (units + 4 * ppw - 1) / (4 * ppw);
}

bool token_attn_supported(const bsg_dims& d) {
  return d.dtype == BSG_BF16 && d.num_q_heads / d.num_kv_heads <= 16;
}

size_t token_attn_workspace_bytes(const bsg_dims& d, int Kt) {
  const int G = d.num_q_heads / d.num_kv_heads;
  return (size_t)d.batch * d.num_kv_heads * token_attn_nwg(d, Kt) * G * (d.head_dim + 2) * sizeof(float);
}

static hipError_t token_attn_rows(const bsg_dims& d, const void* q, const int32_t* kv_lens, const void* k_cache,
                                  const void* v_cache, const int32_t* page_table, const int32_t* token_idx, int Kt,
                                  float scale, float* part, void* out, float* lse, RowWindow rw, int nrows, int nwg,
                                  int ppw, hipStream_t stream) {
  const size_t smem_v = (size_t)4 * 64 * (d.head_dim + DM_VPAD) * sizeof(bf16_t);
  const size_t smem_m = (size_t)4 * 16 * (d.head_dim + 2) * sizeof(float);
  const size_t smem = smem_v > smem_m ? smem_v : smem_m;
  dim3 grid(nwg, d.num_kv_heads, nrows);
#define BSG_DT(DD, BB)                                                                                            \
  do {                                                                                                             \
    auto kfn = attn_decode_tokens_kernel<DD, BB>;                                                                  \
    hipError_t ea = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);  \
    if (ea != hipSuccess) return ea;                                                                               \
    hipLaunchKernelGGL(kfn, grid, dim3(256), smem, stream, (const bf16_t*)q, kv_lens, (const bf16_t*)k_cache,      \
                       (const bf16_t*)v_cache, page_table, token_idx, Kt, scale, part, d.num_q_heads,              \
                       d.num_kv_heads, d.num_pages, d.pt_stride, nwg, ppw, rw, (bf16_t*)out, lse);                 \
  } while (0)
  if (d.head_dim == 128) {
    if (d.page_size == 64) BSG_DT(128, 64); else BSG_DT(128, 128);
  } else {
    if (d.page_size == 64) BSG_DT(64, 64); else BSG_DT(64, 128);
  }
#undef BSG_DT
  return hipGetLastError();
}

hipError_t launch_attn_decode_tokens(const bsg_dims& d, const void* q, const int32_t* kv_lens, const void* k_cache,
                                     const void* v_cache, const int32_t* page_table, const int32_t* token_idx, int Kt,
                                     float scale, void* workspace, void* out, float* lse, hipStream_t stream) {
  const int nwg = token_attn_nwg(d, Kt);
  const int ppw = token_attn_ppw(d, Kt);
  float* part = (float*)workspace;
  hipError_t e = token_attn_rows(d, q, kv_lens, k_cache, v_cache, page_table, token_idx, Kt, scale, part, out, lse,
                                 RowWindow{1, 0, 1}, d.batch, nwg, ppw, stream);
  if (e != hipSuccess || nwg == 1) return e;         // one workgroup per row wrote the rows itself
  dim3 mgrid(d.batch * d.num_q_heads);
  if (d.head_dim == 128)
    hipLaunchKernelGGL((attn_decode_merge_kernel<bf16_t, 128>), mgrid, dim3(128), 0, stream, part, (bf16_t*)out, lse,
                       d.num_q_heads, d.num_kv_heads, nwg, gate_args{nullptr, 0, nullptr});
  else
    hipLaunchKernelGGL((attn_decode_merge_kernel<bf16_t, 64>), mgrid, dim3(64), 0, stream, part, (bf16_t*)out, lse,
                       d.num_q_heads, d.num_kv_heads, nwg, gate_args{nullptr, 0, nullptr});
  return hipGetLastError();
}

// Prefill rows: one workgroup per (sequence, position, group), the list dealt to its four
// waves (ppw sub-blocks of 64 entries each), the row written directly.
hipError_t launch_attn_prefill_tokens(const bsg_dims& d, const void* q, int q_len, const int32_t* kv_lens,
                                      const void* k_cache, const void* v_cache, const int32_t* page_table,
                                      const int32_t* token_idx, int Kt, float scale, void* out, float* lse,
                                      hipStream_t stream) {
  const int units = (Kt + 63) / 64;
  const int ppw = (units + 3) / 4;
  return token_attn_rows(d, q, kv_lens, k_cache, v_cache, page_table, token_idx, Kt, scale, nullptr, out, lse,
                         RowWindow{q_len, 0, q_len}, d.batch * q_len, 1, ppw, stream);
}

static bool decode_mfma_path(const bsg_dims& d) {
  const int G = d.num_q_heads / d.num_kv_heads;
  return d.dtype == BSG_BF16 && G <= 16;
}

static int decode_mfma_ppw(const bsg_dims& d) {
  // two pages per wave when that still leaves >= 512 workgroups (one resident round)
  const long long wg2 = (long long)d.batch * d.num_kv_heads * ((d.top_k + 7) / 8);
  return wg2 >= 512 ? 2 : 1;
}

static int decode_mfma_nwg(const bsg_dims& d) {
  const int ppw = decode_mfma_ppw(d);
  return (d.top_k + 4 * ppw - 1) / (4 * ppw);
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
  if (decode_mfma_path(d))
    return (size_t)d.batch * d.num_kv_heads * decode_mfma_nwg(d) * G * (d.head_dim + 2) * sizeof(float);
  return (size_t)d.batch * d.num_kv_heads * decode_num_splits(d) * G * (d.head_dim + 2) * sizeof(float);
}

static size_t decode_smem(const bsg_dims& d, size_t elem) {
  const int G = d.num_q_heads / d.num_kv_heads;
  return (size_t)(G * d.head_dim + G * d.page_size + G * 3 + 1) * 4 +
         (size_t)d.page_size * (d.head_dim + 2) * elem + (size_t)d.page_size * d.head_dim * elem;
}

hipError_t launch_attn_decode(const bsg_dims& d, const void* q, const int32_t* kv_lens, const void* k_cache,
                              const void* v_cache, const int32_t* page_table, const int32_t* block_idx,
                              float scale, void* workspace, void* out, float* lse, hipStream_t stream,
                              gate_args ga) {
  if (decode_mfma_path(d)) {
    const int nwg = decode_mfma_nwg(d);
    float* part = (float*)workspace;
    const size_t smem_v = (size_t)4 * 64 * (d.head_dim + DM_VPAD) * sizeof(bf16_t);
    const size_t smem_m = (size_t)4 * 16 * (d.head_dim + 2) * sizeof(float);
    const size_t smem = smem_v > smem_m ? smem_v : smem_m;
    const int nunits = d.batch * d.num_kv_heads;
    dim3 grid((nunits + 7) / 8 * 8 * nwg);
#define BSG_DM(DD, BB)                                                                                            \
  do {                                                                                                             \
    auto kfn = attn_decode_mfma_kernel<DD, BB, false, false>;                                                      \
    hipError_t ea = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);  \
    if (ea != hipSuccess) return ea;                                                                               \
    hipLaunchKernelGGL(kfn, grid, dim3(256), smem, stream, (const bf16_t*)q, kv_lens, (const bf16_t*)k_cache,      \
                       (const bf16_t*)v_cache, page_table, const_cast<int32_t*>(block_idx), nullptr, scale, part,  \
                       d.num_q_heads, d.num_kv_heads, d.top_k, d.num_pages, d.pt_stride, nwg, decode_mfma_ppw(d),  \
                       0, 1, nullptr, nullptr, nunits);                                                            \
  } while (0)
    if (d.head_dim == 128) {
      if (d.page_size == 64) BSG_DM(128, 64); else BSG_DM(128, 128);
    } else {
      if (d.page_size == 64) BSG_DM(64, 64); else BSG_DM(64, 128);
    }
#undef BSG_DM
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 mgrid(d.batch * d.num_q_heads);
    if (d.head_dim == 128)
      hipLaunchKernelGGL((attn_decode_merge_kernel<bf16_t, 128>), mgrid, dim3(128), 0, stream, part, (bf16_t*)out, lse,
                         d.num_q_heads, d.num_kv_heads, nwg, ga);
    else
      hipLaunchKernelGGL((attn_decode_merge_kernel<bf16_t, 64>), mgrid, dim3(64), 0, stream, part, (bf16_t*)out, lse,
                         d.num_q_heads, d.num_kv_heads, nwg, ga);
    return hipGetLastError();
  }
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
                         d.num_q_heads, d.num_kv_heads, nsplit, ga);
    else
      hipLaunchKernelGGL((attn_decode_merge_kernel<bf16_t, 64>), mgrid, dim3(64), 0, stream, ws, (bf16_t*)out, lse,
                         d.num_q_heads, d.num_kv_heads, nsplit, ga);
  } else {
    if (d.head_dim == 128)
      hipLaunchKernelGGL((attn_decode_merge_kernel<float, 128>), mgrid, dim3(128), 0, stream, ws, (float*)out, lse,
                         d.num_q_heads, d.num_kv_heads, nsplit, ga);
    else
      hipLaunchKernelGGL((attn_decode_merge_kernel<float, 64>), mgrid, dim3(64), 0, stream, ws, (float*)out, lse,
                         d.num_q_heads, d.num_kv_heads, nsplit, ga);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// The decode step for page-table rows of at most DU_MAXC candidate blocks (bf16, G <= 16):
// S workgroups ("members", S = 2 or 4 while every member still has a CU of its own, else 1)
// per (sequence, group) unit, eight waves each.  Every member runs phases 1-2 in full (the
// members of a unit sit on the same XCD, so the second reader of a block-cache line finds it
// in that XCD's L2) and takes every S-th kept page in phase 3:
//  0. the group-summed fp32 query (heads in order);
//  1. scan: every candidate block's representative of this group (D bf16 = one 256-byte
//     slice of the page's block-cache row) is dotted with the group-summed query, with the
//     arithmetic of decode_score_chunk_kernel (same per-lane products, same DPP segment sums,
//     so the same fp32 scores); the 64-bit (score, index) keys go to LDS;
//  2. select: the top_k - 1 largest keys, exactly.  The maxima of 64 disjoint groups of keys
//     bound the answer from below (the cnt-th largest group maximum has cnt keys at or above
//     it), so only the keys at or above that bound survive, typically a few dozen; they are
//     ranked against each other.  If more than DU_MAXS survive (keys piled into few groups),
//     a radix select over all keys decides instead (11/11/10-bit digits of the score half,
//     then of the index half).  The kept ids are sorted ascending and the own block appended
//     (member 0 writes them to block_idx);
//  3. attend: page e of the list (own block first) goes to member e % S, wave (e / S) % 8;
//     per 64-key sub-block the layout of attn_decode_mfma_kernel (K straight from HBM as the
//     A operand of v_mfma_f32_16x16x32_bf16, V through LDS with the transposing read), exact
//     running maximum per sub-block;
//  4. merge the eight waves' (max, sum, output) in LDS; with S = 1 write out, lse (and the
//     gate), else the member's partial, which attn_decode_merge_kernel then merges.
// F8: the caches hold OCP E4M3 codes with power-of-two scales per (page, head), taken as in
// the fp8 paths of decode_score_chunk_kernel and attn_decode_mfma_kernel (the scale applied
// to a representative's segment sum, to a page's scores, and to its weights before their
// bf16 rounding), so the result equals the bf16 kernel on the decoded caches.
// Measured on the 128K x 32 workload (128 units, S = 2): a merge in the last-arriving member
// (an arrival counter plus one L2 write-back and one L2 invalidate per workgroup) cost more
// than the second launch, so the merge stays a kernel of its own.
namespace {
constexpr int DU_WAVES = 8;
constexpr int DU_NT = 64 * DU_WAVES;
constexpr int DU_MAXC = 4096;                // candidate blocks per unit (keys in LDS)
constexpr int DU_BINS = 2048;                // radix bins per digit (11 bits)
constexpr int DU_MAXS = 1024;                // survivors ranked directly
}  // namespace

template <int D>
static size_t decode_unit_smem_bytes() {
  const size_t scan = (size_t)D * 4 + (size_t)DU_MAXC * 12 + (size_t)DU_BINS * 4 + (size_t)(DU_MAXS + 128) * 8;
  const size_t stage = (size_t)DU_WAVES * 64 * (D + DM_VPAD) * 2;
  const size_t merge = (size_t)DU_WAVES * 16 * (D + 2) * 4;
  size_t m = scan > stage ? scan : stage;
  return m > merge ? m : merge;
}

template <int D, int BS, bool F8>
__global__ __launch_bounds__(DU_NT, 1) void decode_unit_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ kv_lens, const void* __restrict__ block_cache,
    const void* __restrict__ k_cache, const void* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    float scale, int32_t* __restrict__ block_idx, bf16_t* __restrict__ out, float* __restrict__ lse, int Hq, int Hkv,
    int top_k, int num_pages, int pt_stride, gate_args ga, const float* __restrict__ rep_scales,
    const float* __restrict__ k_scales, const float* __restrict__ v_scales, int nunits, int S,
    float* __restrict__ part, int select_only) {
  constexpr int ES = F8 ? 1 : 2;             // bytes per cache element
  constexpr int VPP = F8 ? 16 : 8;           // values per 16-byte piece of a representative
  constexpr int SEG = D / VPP;               // lanes per representative
  constexpr int BPI = 64 / SEG;              // representatives per wave-wide load
  constexpr int U = 64 / BPI;                // loads per lane of one batch of 64 blocks
  constexpr int NDS = D / 32;
  constexpr int NDT = D / 16;
  constexpr int VS = D + DM_VPAD;
  constexpr int SUB = 64;
  constexpr int NSP = BS / SUB;
  constexpr int PPR = D / 8;
  constexpr int NV = SUB * PPR / 64;
  extern __shared__ __attribute__((aligned(16))) unsigned char du_smem[];
  float* qs = reinterpret_cast<float*>(du_smem);                                   // [D]
  uint64_t* keys = reinterpret_cast<uint64_t*>(du_smem + D * 4);                   // [DU_MAXC]
  uint32_t* hist = reinterpret_cast<uint32_t*>(du_smem + D * 4 + DU_MAXC * 8);     // [DU_BINS]
  int32_t* cpage = reinterpret_cast<int32_t*>(du_smem + D * 4 + DU_MAXC * 8 + DU_BINS * 4);   // [DU_MAXC]
  uint64_t* gmax = reinterpret_cast<uint64_t*>(du_smem + D * 4 + DU_MAXC * 12 + DU_BINS * 4);   // [64]
  uint64_t* surv = gmax + 128;                                                                    // [DU_MAXS]
  __shared__ uint64_t tau_s;
  __shared__ int wl[64];                       // kept blocks, ascending, own block last
  __shared__ int wpg[64];                      // their physical pages
  __shared__ uint64_t kept[DU_MAXC / 64];      // kept candidate blocks, one bit each
  __shared__ uint32_t red[DU_WAVES + 1];
  __shared__ uint32_t sel_s[3];
  __shared__ int counter_s;

  // workgroup x serves unit ((x / 8S) * 8 + x % 8) as its member (x / 8) % S: the S members of
  // a unit sit 8 apart in dispatch order, so on the same XCD (workgroups go to the eight XCDs
  // in turn) and their block-cache reads meet in that XCD's L2
  const int xw = blockIdx.x;
  const int sm = (xw >> 3) % S;
  const int unit = (xw / (8 * S)) * 8 + (xw & 7);
  if (unit >= nunits) return;
  const int g = unit % Hkv, b = unit / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = Hq / Hkv;
  const int L = kv_lens[b];
  const int pos = max(L - 1, 0);
  const int own = pos / BS;
  const int ncand = min(own, min(pt_stride, DU_MAXC));
  const int m = top_k - 1;
  const int cnt = min(m, ncand);
  const int32_t* ptrow = page_table + (size_t)b * pt_stride;

  // the scan's page ids (wave w takes blocks [w0, w1)) and the own block's page go out first,
  // so that their round trip overlaps the query's
  const int nper = ((ncand + DU_WAVES - 1) / DU_WAVES + 63) / 64 * 64;
  const int w0 = wave * nper, w1 = min(w0 + nper, ncand);
  constexpr int NPB = DU_MAXC / DU_WAVES / 64;
  int pids[NPB];
#pragma unroll
  for (int c = 0; c < NPB; c++) {
    const int jb = w0 + 64 * c + lane;
    pids[c] = (cnt > 0 && jb < w1) ? page_id(ptrow[jb], num_pages) : 0;
  }
  const int own_page = page_id(ptrow[min(own, pt_stride - 1)], num_pages);
  if (tid < DU_MAXC / 64) kept[tid] = 0ull;
  // ---- 0. group-summed query (fp32, heads in order): the group's G query rows with one
  // 16-byte load per thread, parked in LDS as floats, then summed
  float* qf = reinterpret_cast<float*>(du_smem + D * 4 + DU_MAXC * 8);   // [G][D] (the histogram area)
  {
    const int nq = G * (D / 8);
    uint4 qv4 = make_uint4(0, 0, 0, 0);
    if (tid < nq) qv4 = *reinterpret_cast<const uint4*>(q + ((size_t)b * Hq + g * G) * D + 8 * tid);
    if (tid < nq) {
      const uint32_t wd[4] = {qv4.x, qv4.y, qv4.z, qv4.w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        qf[8 * tid + 2 * i] = __uint_as_float(wd[i] << 16);
        qf[8 * tid + 2 * i + 1] = __uint_as_float(wd[i] & 0xffff0000u);
      }
    }
    __syncthreads();
    for (int d = tid; d < D; d += DU_NT) {
      float s = 0.0f;
      for (int h = 0; h < G; h++) s += qf[h * D + d];
      qs[d] = s;
    }
    __syncthreads();
  }

  // ---- 1. scan: wave w takes blocks [w0, w1), 64 per batch (BPI per load, U loads per lane)
  if (cnt > 0) {
    const int piece = lane % SEG, sg = lane / SEG;
    float qv[VPP];
#pragma unroll
    for (int i = 0; i < VPP; i++) qv[i] = qs[piece * VPP + i];
    const char* bc = reinterpret_cast<const char*>(block_cache) + (size_t)g * D * ES + piece * 16;
    // the page ids of the wave's range (up to DU_MAXC / DU_WAVES blocks: 8 per lane) are kept
    // in LDS beside the keys for the attention phase
#pragma unroll
    for (int c = 0; c < NPB; c++) {
      const int jb = w0 + 64 * c + lane;
      if (jb < w1) cpage[jb] = pids[c];
    }
    // row loads of half h of batch c (32 blocks, U / 2 per lane), into buffer h: one half in
    // flight while the other is summed (whole 64-block batches in flight measured slower: more
    // outstanding reads only add to the memory system's queues)
    constexpr int UH = U / 2;
    uint4 raw[2][UH];
    float scl[2][UH];                                     // F8: the representative's scale
    auto issue_rows = [&](int c, int h, uint4 (&rw)[UH], float (&sc)[UH]) {
      const int base = w0 + 64 * c;
      int pid = 0;
#pragma unroll
      for (int c2 = 0; c2 < NPB; c2++)
        if (c2 == c) pid = pids[c2];
#pragma unroll
      for (int u = 0; u < UH; u++) {
        const int jl = 32 * h + u * BPI + sg;             // block of this lane, relative to base
        const int p = __shfl(pid, jl, 64);
        rw[u] = base + jl < w1 ? *reinterpret_cast<const uint4*>(bc + (size_t)p * Hkv * D * ES)
                               : make_uint4(0, 0, 0, 0);
        if (F8) sc[u] = (base + jl < w1 && piece == 0) ? rep_scales[(size_t)p * Hkv + g] : 0.0f;
      }
    };
    const int nbat = (w1 - w0 + 63) / 64;
    if (nbat > 0) issue_rows(0, 0, raw[0], scl[0]);
#pragma unroll
    for (int c = 0; c < NPB; c++) {
      if (c >= nbat) break;
#pragma unroll
      for (int h = 0; h < 2; h++) {
        if (h == 0) issue_rows(c, 1, raw[1], scl[1]);
        else if (c + 1 < nbat) issue_rows(c + 1, 0, raw[0], scl[0]);
        const int base = w0 + 64 * c + 32 * h;
#pragma unroll
        for (int u = 0; u < UH; u++) {
          const int jb = base + u * BPI + sg;
          const uint4 rr = raw[h][u];
          const uint32_t wd[4] = {rr.x, rr.y, rr.z, rr.w};
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
          if (F8) s *= scl[h][u];
          if (piece == 0 && jb < w1) keys[jb] = sel_key(s, jb);
        }
      }
    }
  }
  __syncthreads();

  // ---- 2. select the cnt largest keys (distinct: the low half holds the block index).  The
  // kept blocks are marked in a bitmap of the candidates, which gives them in ascending order.
  bool ranked = false;                                      // workgroup-uniform
  if (cnt > 0) {
    // lower bound tau: the cnt-th largest of 64 group maxima.  The groups are disjoint sets of
    // keys: with ncand >= DU_NT, thread t takes keys t, t + DU_NT, ... and a group is 8
    // consecutive threads; with fewer keys, group l takes keys l, l + 64, ...  At least
    // min(64, ncand) >= cnt groups are non-empty, so at least cnt keys are >= tau.
    auto shfl_xor64 = [](uint64_t v, int o) {
      return ((uint64_t)(uint32_t)__shfl_xor((int)(v >> 32), o, 64) << 32) |
             (uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)v, o, 64);
    };
    if (ncand >= DU_NT) {
      uint64_t mx = 0;                                      // 0 is below every real key
      for (int e = tid; e < ncand; e += DU_NT) mx = max(mx, keys[e]);
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) mx = max(mx, shfl_xor64(mx, o));
      if ((lane & 7) == 0) gmax[tid >> 3] = mx;
    } else if (wave == 0) {
      uint64_t mx = 0;
      for (int e = lane; e < ncand; e += 64) mx = max(mx, keys[e]);
      gmax[lane] = mx;
    }
    if (tid == 0) counter_s = 0;
    __syncthreads();
    // every wave ranks the 64 maxima itself, so no barrier separates tau from the survivors
    uint64_t tau;
    {
      const uint64_t gm = gmax[lane];
      const ulonglong2* g2 = reinterpret_cast<const ulonglong2*>(gmax);
      int rank = 0;
#pragma unroll 8
      for (int i = 0; i < 32; i++) {
        const ulonglong2 v = g2[i];
        rank += (v.x > gm ? 1 : 0) + (v.y > gm ? 1 : 0);
      }
      // the real maxima are distinct and empty groups (0) rank last: exactly one lane holds it
      const uint64_t hit = __ballot(gm != 0ull && rank == cnt - 1);
      const int src = (int)__builtin_ctzll(hit);
      tau = ((uint64_t)(uint32_t)__shfl((int)(gm >> 32), src, 64) << 32) |
            (uint64_t)(uint32_t)__shfl((int)(uint32_t)gm, src, 64);
    }
    for (int e = tid; e < ncand; e += DU_NT) {
      const uint64_t k = keys[e];
      if (k >= tau) {
        const int at = atomicAdd(&counter_s, 1);
        if (at < DU_MAXS) surv[at] = k;
      }
    }
    __syncthreads();
    const int ns = counter_s;
    if (ns <= DU_MAXS) {
      const ulonglong2* s2 = reinterpret_cast<const ulonglong2*>(surv);
      for (int e = tid; e < ns; e += DU_NT) {
        const uint64_t k = surv[e];
        int rank = 0;
#pragma unroll 4
        for (int i = 0; i < ns / 2; i++) {
          const ulonglong2 v = s2[i];
          rank += (v.x > k ? 1 : 0) + (v.y > k ? 1 : 0);
        }
        if (ns & 1) rank += surv[ns - 1] > k ? 1 : 0;
        if (rank < cnt) {
          const int j = sel_key_index(k);
          atomicOr(&kept[j >> 6], 1ull << (j & 63));
        }
      }
      ranked = true;
    }
    __syncthreads();
  }
  if (cnt > 0 && !ranked) {
    uint64_t prefix = 0, pmask = 0;
    uint32_t above = 0;
    bool done = false;
    for (int lv = 0; lv < 6 && !done; lv++) {
      const int shift = lv == 0 ? 53 : lv == 1 ? 42 : lv == 2 ? 32 : lv == 3 ? 21 : lv == 4 ? 10 : 0;
      const int nbits = (lv == 2 || lv == 5) ? 10 : 11;
      const uint32_t dmask = (1u << nbits) - 1u;
      for (int i = tid; i < DU_BINS; i += DU_NT) hist[i] = 0u;
      __syncthreads();
      for (int e = tid; e < ncand; e += DU_NT) {
        const uint64_t k = keys[e];
        if ((k & pmask) == prefix) atomicAdd(&hist[(uint32_t)(k >> shift) & dmask], 1u);
      }
      __syncthreads();
      // bins from the top: this thread sums `per` consecutive bins, then a block scan
      const uint32_t need = (uint32_t)cnt - above;
      const int nb = 1 << nbits;
      const int per = nb / DU_NT;
      uint32_t mine = 0;
      for (int k = 0; k < per; k++) mine += hist[nb - 1 - (tid * per + k)];
      uint32_t incl = mine;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      if (lane == 63) red[wave] = incl;
      __syncthreads();
      uint32_t before = incl - mine;
      for (int w2 = 0; w2 < wave; w2++) before += red[w2];
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
      prefix |= (uint64_t)sel_s[0] << shift;
      pmask |= (uint64_t)dmask << shift;
      above += sel_s[1];
      done = above + sel_s[2] == (uint32_t)cnt;
      __syncthreads();
    }
    // the kept keys are those whose masked top bits are >= prefix (exactly cnt of them)
    for (int e = tid; e < ncand; e += DU_NT) {
      const uint64_t k = keys[e];
      if ((k & pmask) >= prefix) atomicOr(&kept[e >> 6], 1ull << (e & 63));
    }
    __syncthreads();
  }
  // ascending list from the bitmap (wave 0: a word per lane, positions by a prefix count),
  // the own block appended
  if (wave == 0) {
    uint64_t bits = lane < DU_MAXC / 64 ? kept[lane] : 0ull;
    const int n1 = __popcll(bits);
    int incl = n1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    int at = incl - n1;
    while (bits) {
      const int b0 = (int)__builtin_ctzll(bits);
      bits &= bits - 1;
      wl[at++] = lane * 64 + b0;
    }
    if (lane == 0) wl[cnt] = own;
  }
  __syncthreads();
  if (sm == 0 && tid < top_k) block_idx[((size_t)b * Hkv + g) * top_k + tid] = tid <= cnt ? wl[tid] : -1;
  if (select_only) return;                             // the block selection alone
  // pages in the attention order: the own block first (its page from the table), then the
  // kept blocks ascending (their pages from the scan)
  if (tid <= cnt) {
    const int jb = tid == 0 ? own : wl[tid - 1];
    wpg[tid] = tid == 0 ? own_page : cpage[jb];
  }
  __syncthreads();

  // ---- 3. attention over the kept pages, page e on member e % S, wave (e / S) % DU_WAVES
  const int n = lane & 15, qd = lane >> 4;
  bf16_t* Vs = reinterpret_cast<bf16_t*>(du_smem) + (size_t)wave * SUB * VS;
  const float c2 = scale * 1.4426950408889634f;
  bf16x8_t qb[NDS];
  {
    const bool hv = n < G;
    const bf16_t* qp = q + ((size_t)b * Hq + (size_t)g * G + (hv ? n : 0)) * D + 8 * qd;
#pragma unroll
    for (int s = 0; s < NDS; s++) {
      uint4 v = hv ? *reinterpret_cast<const uint4*>(qp + 32 * s) : make_uint4(0, 0, 0, 0);
      qb[s] = *reinterpret_cast<bf16x8_t*>(&v);
    }
  }
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4_t o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; i++) o[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int vtr = (4 * qd + ((lane & 15) >> 2)) * VS + 4 * (lane & 3);
  const int npages = cnt + 1;
  for (int e = wave * S + sm; e < npages; e += DU_WAVES * S) {
    const int jj = e == 0 ? own : wl[e - 1];
    const int p = wpg[e];
    const int nk = clampi(pos - jj * BS + 1, 0, BS);
    const char* kpg = reinterpret_cast<const char*>(k_cache) + (((size_t)p * Hkv + g) * BS) * D * ES;
    const char* vpg = reinterpret_cast<const char*>(v_cache) + (((size_t)p * Hkv + g) * BS) * D * ES;
    const float skp = F8 ? k_scales[(size_t)p * Hkv + g] : 1.0f;
    const float svp = F8 ? v_scales[(size_t)p * Hkv + g] : 1.0f;
#pragma unroll
    for (int h2 = 0; h2 < NSP; h2++) {
      const int kb = h2 * SUB;
      if (kb >= nk) break;
      // every K and V load of the sub-block goes out before its first product
      uint4 rv[F8 ? 1 : NV];
      uint2 rv8[F8 ? NV : 1];
      uint4 rk[F8 ? 1 : SUB / 16][NDS];
      uint2 rk8[F8 ? SUB / 16 : 1][NDS];
#pragma unroll
      for (int i = 0; i < NV; i++) {
        const int pc = i * 64 + lane;
        const int r = pc / PPR, c = pc % PPR;
        const char* src = vpg + ((size_t)(kb + r) * D + 8 * c) * ES;
        if constexpr (F8) rv8[i] = *reinterpret_cast<const uint2*>(src);
        else rv[i] = *reinterpret_cast<const uint4*>(src);
      }
#pragma unroll
      for (int T = 0; T < SUB / 16; T++) {
        const char* kr = kpg + ((size_t)(kb + 16 * T + n) * D + 8 * qd) * ES;
#pragma unroll
        for (int s2 = 0; s2 < NDS; s2++) {
          if constexpr (F8) rk8[T][s2] = *reinterpret_cast<const uint2*>(kr + 32 * s2);
          else rk[T][s2] = *reinterpret_cast<const uint4*>(kr + 64 * s2);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x4_t sacc[SUB / 16];
#pragma unroll
      for (int T = 0; T < SUB / 16; T++) {
        sacc[T] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s2 = 0; s2 < NDS; s2++) {
          bf16x8_t ka;
          if constexpr (F8) ka = e4m3x8_to_bf16(rk8[T][s2]);
          else ka = *reinterpret_cast<const bf16x8_t*>(&rk[T][s2]);
          sacc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[s2], sacc[T], 0, 0, 0);
        }
        if constexpr (F8) sacc[T] *= skp;
      }
#pragma unroll
      for (int i = 0; i < NV; i++) {           // V rows past nk (inside the page) are zeroed
        const int pc = i * 64 + lane;
        const int r = pc / PPR, c = pc % PPR;
        const bool ok = kb + r < nk;
        if constexpr (F8) {
          const bf16x8_t v = e4m3x8_to_bf16(ok ? rv8[i] : make_uint2(0, 0));
          *reinterpret_cast<bf16x8_t*>(Vs + r * VS + 8 * c) = v;
        } else {
          *reinterpret_cast<uint4*>(Vs + r * VS + 8 * c) = ok ? rv[i] : make_uint4(0, 0, 0, 0);
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int T = 0; T < SUB / 16; T++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int key = kb + 16 * T + 4 * qd + i;
          const float sc = key < nk ? sacc[T][i] : -INFINITY;
          sacc[T][i] = sc;
          mx = fmaxf(mx, sc);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
      m_run = m_new;
      float rs = 0.0f;
#pragma unroll
      for (int T = 0; T < SUB / 16; T++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float pe = __builtin_amdgcn_exp2f((sacc[T][i] - m_use) * c2);
          sacc[T][i] = pe;
          rs += pe;
        }
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int i = 0; i < NDT; i++) o[i] *= alpha;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int k2 = 0; k2 < SUB / 32; k2++) {
        bf16x8_t pb;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          pb[i] = (__bf16)(F8 ? sacc[2 * k2][i] * svp : sacc[2 * k2][i]);
          pb[4 + i] = (__bf16)(F8 ? sacc[2 * k2 + 1][i] * svp : sacc[2 * k2 + 1][i]);
        }
#pragma unroll
        for (int dt = 0; dt < NDT; dt++) {
          const bf16_t* vb = Vs + vtr + (32 * k2) * VS + 16 * dt;
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dm_lds_s16x4_ptr)(vb));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dm_lds_s16x4_ptr)(vb + 16 * VS));
          bf16x8_t va;
          *reinterpret_cast<s16x4_t*>(&va) = lo;
          *(reinterpret_cast<s16x4_t*>(&va) + 1) = hi;
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[dt], 0, 0, 0);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  float l_h = l_run + __shfl_xor(l_run, 16, 64);
  l_h += __shfl_xor(l_h, 32, 64);

  // ---- 4. merge the waves and write the output
  __syncthreads();
  float* mrg = reinterpret_cast<float*>(du_smem);               // [DU_WAVES][16][D + 2]
  {
    float* mw = mrg + ((size_t)wave * 16 + n) * (D + 2);
    if (qd == 0) {
      mw[0] = m_run;
      mw[1] = l_h;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; dt++)
#pragma unroll
      for (int i = 0; i < 4; i++) mw[2 + 16 * dt + 4 * qd + i] = o[dt][i];
  }
  __syncthreads();
  float* myp = part + ((size_t)unit * S + sm) * G * (D + 2);
  for (int e2 = tid; e2 < G * D; e2 += DU_NT) {
    const int h = e2 / D, d = e2 % D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < DU_WAVES; w++) mm = fmaxf(mm, mrg[((size_t)w * 16 + h) * (D + 2)]);
    float ll = 0.0f, oo = 0.0f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < DU_WAVES; w++) {
        const float* mw = mrg + ((size_t)w * 16 + h) * (D + 2);
        if (mw[0] == -INFINITY) continue;
        const float sc = __builtin_amdgcn_exp2f((mw[0] - mm) * c2);
        ll += mw[1] * sc;
        oo += mw[2 + d] * sc;
      }
    }
    if (S > 1) {             // a partial in the layout attn_decode_merge_kernel reads
      myp[h * (D + 2) + 2 + d] = oo;
      if (d == 0) {
        myp[h * (D + 2)] = mm == -INFINITY ? -INFINITY : mm * scale;   // natural-log units
        myp[h * (D + 2) + 1] = ll;
      }
      continue;
    }
    const size_t row = (size_t)b * Hq + (size_t)g * G + h;
    float a = oo * (ll > 0.0f ? 1.0f / ll : 0.0f);
    if (ga.g) {                                        // out = g A + (1 - g) x, one rounding
      const float gv = ga.per_dim ? ga.g[row * D + d] : ga.g[row];
      a = gv * a + (1.0f - gv) * bf16_to_f32(static_cast<const bf16_t*>(ga.x)[row * D + d]);
    }
    out[row * D + d] = f32_to_bf16(a);
    if (lse && d == 0) lse[row] = mm * scale + logf(ll);
  }
}

static size_t decode_unit_smem(const bsg_dims& d) {
  return d.head_dim == 128 ? decode_unit_smem_bytes<128>() : decode_unit_smem_bytes<64>();
}

bool decode_unit_supported(const bsg_dims& d) {
  const int G = d.num_q_heads / d.num_kv_heads;
  return d.dtype == BSG_BF16 && G <= 16 && d.pt_stride <= DU_MAXC && decode_unit_smem(d) <= 160 * 1024;
}

// workgroups per (sequence, group) unit: 2 or 4 while every member still gets a CU of its own
static int decode_unit_members(const bsg_dims& d) {
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    ncu = 256;
  const long long units = (long long)d.batch * d.num_kv_heads;
  const long long padded = (units + 7) / 8 * 8;
  int S = 1;
  while (S < 4 && padded * S * 2 <= ncu) S *= 2;
  return S;
}

static size_t decode_unit_workspace_bytes(const bsg_dims& d) {
  const int G = d.num_q_heads / d.num_kv_heads;
  const int S = decode_unit_members(d);
  return S > 1 ? (size_t)d.batch * d.num_kv_heads * S * G * (d.head_dim + 2) * sizeof(float) : 0;
}

static hipError_t launch_decode_unit(const bsg_dims& d, const void* q, const int32_t* kv_lens,
                                     const void* block_cache, const void* k_cache, const void* v_cache,
                                     const int32_t* page_table, float scale, int32_t* block_idx, void* out,
                                     float* lse, hipStream_t stream, gate_args ga, const float* rep_scales,
                                     const float* k_scales, const float* v_scales, float* part) {
  const size_t smem = decode_unit_smem(d);
  const bool f8 = k_scales != nullptr;
  const int S = decode_unit_members(d);
  const int nunits = d.batch * d.num_kv_heads;
  dim3 grid((nunits + 7) / 8 * 8 * S);
#define BSG_DU(DD, BB, F)                                                                                          \
  do {                                                                                                              \
    auto kfn = decode_unit_kernel<DD, BB, F>;                                                                       \
    hipError_t ea = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);   \
    if (ea != hipSuccess) return ea;                                                                                \
    hipLaunchKernelGGL(kfn, grid, dim3(DU_NT), smem, stream, (const bf16_t*)q, kv_lens, block_cache, k_cache,       \
                       v_cache, page_table, scale, block_idx, (bf16_t*)out, lse, d.num_q_heads, d.num_kv_heads,     \
                       d.top_k, d.num_pages, d.pt_stride, ga, rep_scales, k_scales, v_scales, nunits, S, part, 0); \
  } while (0)
#define BSG_DU_F(DD, BB)                 \
  do {                                   \
    if (f8) BSG_DU(DD, BB, true);        \
    else BSG_DU(DD, BB, false);          \
  } while (0)
  if (d.head_dim == 128) {
    if (d.page_size == 64) BSG_DU_F(128, 64); else BSG_DU_F(128, 128);
  } else {
    if (d.page_size == 64) BSG_DU_F(64, 64); else BSG_DU_F(64, 128);
  }
#undef BSG_DU_F
#undef BSG_DU
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  dim3 mgrid(d.batch * d.num_q_heads);
  if (d.head_dim == 128)
    hipLaunchKernelGGL((attn_decode_merge_kernel<bf16_t, 128>), mgrid, dim3(128), 0, stream, part, (bf16_t*)out, lse,
                       d.num_q_heads, d.num_kv_heads, S, ga);
  else
    hipLaunchKernelGGL((attn_decode_merge_kernel<bf16_t, 64>), mgrid, dim3(64), 0, stream, part, (bf16_t*)out, lse,
                       d.num_q_heads, d.num_kv_heads, S, ga);
  return hipGetLastError();
}

// The scan and exact block selection of decode_unit_kernel alone, one workgroup per (sequence,
// group), for bsg_group_score_topk at q_len = 1 (and the two-level decode step's block stage).
hipError_t launch_decode_unit_select(const bsg_dims& d, const void* q, const int32_t* kv_lens,
                                     const void* block_cache, const int32_t* page_table, int32_t* block_idx,
                                     hipStream_t stream) {
  const size_t smem = decode_unit_smem(d);
  const int nunits = d.batch * d.num_kv_heads;
  dim3 grid((nunits + 7) / 8 * 8);
#define BSG_DUS(DD, BB)                                                                                             \
  do {                                                                                                              \
    auto kfn = decode_unit_kernel<DD, BB, false>;                                                                   \
    hipError_t ea = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);   \
    if (ea != hipSuccess) return ea;                                                                                \
    hipLaunchKernelGGL(kfn, grid, dim3(DU_NT), smem, stream, (const bf16_t*)q, kv_lens, block_cache, nullptr,       \
                       nullptr, page_table, 1.0f, block_idx, nullptr, nullptr, d.num_q_heads, d.num_kv_heads,       \
                       d.top_k, d.num_pages, d.pt_stride, gate_args{nullptr, 0, nullptr}, nullptr, nullptr, nullptr, \
                       nunits, 1, nullptr, 1);                                                                      \
  } while (0)
  if (d.head_dim == 128) {
    if (d.page_size == 64) BSG_DUS(128, 64); else BSG_DUS(128, 128);
  } else {
    if (d.page_size == 64) BSG_DUS(64, 64); else BSG_DUS(64, 128);
  }
#undef BSG_DUS
  return hipGetLastError();
}

// LDS of the fused decode attention kernel: V staging, the wave merge, or the selection
// prologue's lists plus its tops / survivors, whichever is largest.  lt: log2 of the
// number of leading keys the prologue takes from every chunk list.
static size_t decode_step_smem(const bsg_dims& d, int* lt_out) {
  const int nchunks = decode_select_nchunks(d);
  const int m = d.top_k - 1;
  const int lt = decode_prologue_lt(nchunks, m);
  const size_t smem_v = (size_t)4 * 64 * (d.head_dim + DM_VPAD) * sizeof(bf16_t);
  const size_t smem_m = (size_t)4 * 16 * (d.head_dim + 2) * sizeof(float);
  const size_t smem_s = decode_prologue_smem_bytes(nchunks, m, lt);
  size_t smem = smem_v > smem_m ? smem_v : smem_m;
  if (lt_out) *lt_out = lt;
  return smem > smem_s ? smem : smem_s;
}

bool decode_step_fused_supported(const bsg_dims& d) {
  return decode_mfma_path(d) && decode_select_supported(d, 1) && decode_step_smem(d, nullptr) <= 150 * 1024;
}

size_t decode_step_workspace_bytes(const bsg_dims& d) {
  if (!decode_step_fused_supported(d)) return 0;
  const size_t a = (decode_select_workspace_bytes(d) + 255) / 256 * 256;
  const size_t w = decode_workspace_bytes(d);
  const size_t u = decode_unit_supported(d) ? decode_unit_workspace_bytes(d) : 0;
  return a + (w > u ? w : u);
}

hipError_t launch_decode_step(const bsg_dims& d, const void* q, const int32_t* kv_lens, const void* block_cache,
                              const void* k_cache, const void* v_cache, const int32_t* page_table, float scale,
                              int32_t* block_idx, void* workspace, void* out, float* lse, hipStream_t stream,
                              gate_args ga, const float* rep_scales, const float* k_scales, const float* v_scales) {
  const bool f8 = k_scales != nullptr;
  const size_t a = (decode_select_workspace_bytes(d) + 255) / 256 * 256;
  if (decode_unit_supported(d))
    return launch_decode_unit(d, q, kv_lens, block_cache, k_cache, v_cache, page_table, scale, block_idx, out, lse,
                              stream, ga, rep_scales, k_scales, v_scales, (float*)((char*)workspace + a));
  uint64_t* lists = (uint64_t*)workspace;
  float* part = (float*)((char*)workspace + a);
  hipError_t e = launch_decode_score_chunks(d, q, kv_lens, block_cache, page_table, lists, stream, rep_scales);
  if (e != hipSuccess) return e;
  const int nwg = decode_mfma_nwg(d);
  const int nchunks = decode_select_nchunks(d);
  int lt = 0;
  const size_t smem = decode_step_smem(d, &lt);
  if (smem > 150 * 1024) return hipErrorInvalidValue;
  const int nunits = d.batch * d.num_kv_heads;
  dim3 grid((nunits + 7) / 8 * 8 * nwg);
#define BSG_DF(DD, BB, F)                                                                                         \
  do {                                                                                                             \
    auto kfn = attn_decode_mfma_kernel<DD, BB, true, F>;                                                           \
    hipError_t ea = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);  \
    if (ea != hipSuccess) return ea;                                                                               \
    hipLaunchKernelGGL(kfn, grid, dim3(256), smem, stream, (const bf16_t*)q, kv_lens, k_cache, v_cache,            \
                       page_table, block_idx, lists, scale, part, d.num_q_heads, d.num_kv_heads, d.top_k,           \
                       d.num_pages, d.pt_stride, nwg, decode_mfma_ppw(d), nchunks, lt, k_scales, v_scales, nunits); \
  } while (0)
#define BSG_DF_F(DD, BB)                 \
  do {                                   \
    if (f8) BSG_DF(DD, BB, true);        \
    else BSG_DF(DD, BB, false);          \
  } while (0)
  if (d.head_dim == 128) {
    if (d.page_size == 64) BSG_DF_F(128, 64); else BSG_DF_F(128, 128);
  } else {
    if (d.page_size == 64) BSG_DF_F(64, 64); else BSG_DF_F(64, 128);
  }
#undef BSG_DF_F
#undef BSG_DF
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 mgrid(d.batch * d.num_q_heads);
  if (d.head_dim == 128)
    hipLaunchKernelGGL((attn_decode_merge_kernel<bf16_t, 128>), mgrid, dim3(128), 0, stream, part, (bf16_t*)out, lse,
                       d.num_q_heads, d.num_kv_heads, nwg, ga);
  else
    hipLaunchKernelGGL((attn_decode_merge_kernel<bf16_t, 64>), mgrid, dim3(64), 0, stream, part, (bf16_t*)out, lse,
                       d.num_q_heads, d.num_kv_heads, nwg, ga);
  return hipGetLastError();
}

BSG_DEBUG_FILE(attn_decode)

}  // namespace bsg
