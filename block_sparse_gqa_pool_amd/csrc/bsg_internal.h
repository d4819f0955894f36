// Host-side launchers shared between the kernel sources and the C entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bsg.h"

namespace bsg {
// Gated fusion of an attention output with a caller tensor ("Sparse Attention for
// Long-Context LLMs", section 4.3 "Gating Mechanisms Reduce Risk", step 6: out = Gate * A +
// (1 - Gate) * X, the gate being a scalar or a per-dimension vector).  g == nullptr: no fusion.  g is fp32, one value per
// (sequence, head, query) row (per_dim = 0) or per element (per_dim = 1); x has the output's
// dtype and layout.
struct gate_args {
  const float* g;
  int per_dim;
  const void* x;
};


hipError_t launch_block_pool(const bsg_dims& d, const void* k_cache, const int32_t* page_table,
                             const int32_t* kv_lens, const int32_t* blk_begin, void* block_cache,
                             hipStream_t stream);

hipError_t launch_group_score(const bsg_dims& d, const void* q, int q_len, const int32_t* kv_lens,
                              const void* block_cache, const int32_t* page_table, float* scores,
                              int score_stride, hipStream_t stream);

hipError_t launch_topk(const bsg_dims& d, const float* scores, int q_len, int score_stride,
                       const int32_t* kv_lens, int32_t* block_idx, hipStream_t stream);

// Fused prefill scoring + selection (bf16, q_len > 1): MFMA scores, per-row streaming top-k.
bool group_score_topk_fused_supported(const bsg_dims& d, int q_len);
hipError_t launch_group_score_topk_fused(const bsg_dims& d, const void* q, int q_len,
                                         const int32_t* kv_lens, const void* block_cache,
                                         const int32_t* page_table, int32_t* block_idx,
                                         hipStream_t stream);

// Decode scoring + selection (q_len = 1): chunked block-cache scan + tournament merge.
bool decode_select_supported(const bsg_dims& d, int q_len);
bool decode_unit_supported(const bsg_dims& d);
hipError_t launch_decode_unit_select(const bsg_dims& d, const void* q, const int32_t* kv_lens,
                                     const void* block_cache, const int32_t* page_table, int32_t* block_idx,
                                     hipStream_t stream);
size_t decode_select_workspace_bytes(const bsg_dims& d);
hipError_t launch_decode_select(const bsg_dims& d, const void* q, const int32_t* kv_lens, const void* block_cache,
                                const int32_t* page_table, int32_t* block_idx, void* workspace, hipStream_t stream);

int decode_select_nchunks(const bsg_dims& d);
hipError_t launch_decode_score_chunks(const bsg_dims& d, const void* q, const int32_t* kv_lens,
                                     const void* block_cache, const int32_t* page_table, uint64_t* lists,
                                     hipStream_t stream, const float* rep_scales = nullptr);

// Fused decode step: chunked scoring, then selection + split attention in one kernel, then merge.
bool decode_step_fused_supported(const bsg_dims& d);
size_t decode_step_workspace_bytes(const bsg_dims& d);
hipError_t launch_decode_step(const bsg_dims& d, const void* q, const int32_t* kv_lens, const void* block_cache,
                              const void* k_cache, const void* v_cache, const int32_t* page_table, float scale,
                              int32_t* block_idx, void* workspace, void* out, float* lse, hipStream_t stream,
                              gate_args ga = {nullptr, 0, nullptr}, const float* rep_scales = nullptr,
                              const float* k_scales = nullptr, const float* v_scales = nullptr);

// Token-level / two-level selection (token_select.hip) and attention over token lists.
size_t token_topk_workspace_bytes(const bsg_dims& d, bool two_level);
hipError_t launch_token_topk(const bsg_dims& d, const void* q, const int32_t* kv_lens, const void* k_cache,
                             const int32_t* page_table, const int32_t* block_idx, int top_k_tokens,
                             int32_t* token_idx, void* workspace, hipStream_t stream);
size_t token_topk_prefill_workspace_bytes(const bsg_dims& d, int q_len, bool two_level);
hipError_t launch_token_topk_prefill(const bsg_dims& d, const void* q, int q_len, const int32_t* kv_lens,
                                     const void* k_cache, const int32_t* page_table, const int32_t* block_idx,
                                     int top_k_tokens, int32_t* token_idx, void* workspace, hipStream_t stream);
hipError_t launch_attn_prefill_tokens(const bsg_dims& d, const void* q, int q_len, const int32_t* kv_lens,
                                      const void* k_cache, const void* v_cache, const int32_t* page_table,
                                      const int32_t* token_idx, int Kt, float scale, void* out, float* lse,
                                      hipStream_t stream);
bool token_attn_supported(const bsg_dims& d);
size_t token_attn_workspace_bytes(const bsg_dims& d, int Kt);
hipError_t launch_attn_decode_tokens(const bsg_dims& d, const void* q, const int32_t* kv_lens, const void* k_cache,
                                     const void* v_cache, const int32_t* page_table, const int32_t* token_idx, int Kt,
                                     float scale, void* workspace, void* out, float* lse, hipStream_t stream);

// fp8 (OCP E4M3) caches: per-(page, head) power-of-two scales (fp8_cache.hip)
hipError_t launch_quantize_pages_fp8(const bsg_dims& d, const void* src, const int32_t* page_table,
                                     const int32_t* kv_lens, uint8_t* codes, float* scales, hipStream_t stream);
hipError_t launch_block_pool_fp8(const bsg_dims& d, const uint8_t* k_codes, const float* k_scales,
                                 const int32_t* page_table, const int32_t* kv_lens, const int32_t* blk_begin,
                                 uint8_t* rep_codes, float* rep_scales, hipStream_t stream);

hipError_t launch_attn_prefill(const bsg_dims& d, const void* q, int q_len, const int32_t* kv_lens,
                               const void* k_cache, const void* v_cache, const int32_t* page_table,
                               const int32_t* block_idx, float scale, void* out, float* lse,
                               hipStream_t stream, gate_args ga = {nullptr, 0, nullptr});

int decode_num_splits(const bsg_dims& d);
size_t decode_workspace_bytes(const bsg_dims& d);
hipError_t launch_attn_decode(const bsg_dims& d, const void* q, const int32_t* kv_lens,
                              const void* k_cache, const void* v_cache, const int32_t* page_table,
                              const int32_t* block_idx, float scale, void* workspace, void* out,
                              float* lse, hipStream_t stream, gate_args ga = {nullptr, 0, nullptr});

#ifdef BSG_DEBUG
// the debug words of the kernel files (BSG_DEBUG_FILE in bsg_device.h)
int dbg_fetch_attn_decode(unsigned* out, int reset);
int dbg_fetch_attn_prefill(unsigned* out, int reset);
int dbg_fetch_block_pool(unsigned* out, int reset);
int dbg_fetch_decode_select(unsigned* out, int reset);
int dbg_fetch_fp8_cache(unsigned* out, int reset);
int dbg_fetch_group_score(unsigned* out, int reset);
int dbg_fetch_score_topk_fused(unsigned* out, int reset);
int dbg_fetch_token_select(unsigned* out, int reset);
#endif

}  // namespace bsg
