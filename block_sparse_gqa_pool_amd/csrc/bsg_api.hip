// C entry points: host-side validation, then launches on the caller's stream.
// Every check runs before anything is enqueued, so an error leaves the stream untouched.
#include <stddef.h>
#include <stdint.h>

#include "bsg.h"
#include "bsg_internal.h"

namespace {

int check_dims(const bsg_dims* d) {
  if (!d) return BSG_ERR_NULL;
  if (d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->head_dim < 1 || d->page_size < 1 ||
      d->top_k < 1 || d->num_pages < 1 || d->pt_stride < 1)
    return BSG_ERR_SHAPE;
  if (d->num_q_heads % d->num_kv_heads != 0) return BSG_ERR_SHAPE;
  if (d->dtype != BSG_F32 && d->dtype != BSG_BF16) return BSG_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return BSG_ERR_UNSUPPORTED;
  if (d->page_size != 64 && d->page_size != 128) return BSG_ERR_UNSUPPORTED;
  if (d->top_k > 64) return BSG_ERR_UNSUPPORTED;
  // 32-bit element offsets inside one sequence's page row and safe grid sizes
  if ((long long)d->pt_stride * d->page_size > (1LL << 30)) return BSG_ERR_UNSUPPORTED;
  return BSG_OK;
}

int to_status(hipError_t e) { return e == hipSuccess ? BSG_OK : BSG_ERR_HIP; }

}  // namespace

extern "C" {

int bsg_version(void) { return 10000; }

int bsg_debug_errors(unsigned int* bits, int reset) {
  if (!bits) return BSG_ERR_NULL;
#ifdef BSG_DEBUG
  int (*const fetch[])(unsigned*, int) = {bsg::dbg_fetch_attn_decode,   bsg::dbg_fetch_attn_prefill,
                                          bsg::dbg_fetch_block_pool,    bsg::dbg_fetch_decode_select,
                                          bsg::dbg_fetch_fp8_cache,     bsg::dbg_fetch_group_score,
                                          bsg::dbg_fetch_score_topk_fused, bsg::dbg_fetch_token_select};
  unsigned all = 0;
  for (auto f : fetch) {
    unsigned w = 0;
    if (f(&w, reset)) return BSG_ERR_HIP;
    all |= w;
  }
  *bits = all;
  return BSG_OK;
#else
  (void)reset;
  *bits = 0;
  return BSG_ERR_UNSUPPORTED;
#endif
}

const char* bsg_status_str(int status) {
  switch (status) {
    case BSG_OK: return "BSG_OK";
    case BSG_ERR_NULL: return "BSG_ERR_NULL: a required pointer is NULL";
    case BSG_ERR_SHAPE: return "BSG_ERR_SHAPE: inconsistent or non-positive sizes";
    case BSG_ERR_UNSUPPORTED: return "BSG_ERR_UNSUPPORTED: dtype, head_dim, page_size or top_k not supported";
    case BSG_ERR_WORKSPACE: return "BSG_ERR_WORKSPACE: workspace missing or too small";
    case BSG_ERR_HIP: return "BSG_ERR_HIP: the HIP runtime reported an error";
    case BSG_ERR_SCRATCH:
      return "BSG_ERR_SCRATCH: these sizes need more workspace than the library's static scratch holds";
    default: return "unknown bsg status";
  }
}

int bsg_block_pool(const bsg_dims* dims, const void* k_cache, const int32_t* page_table, const int32_t* kv_lens,
                   const int32_t* blk_begin, void* block_cache, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!k_cache || !page_table || !kv_lens || !block_cache) return BSG_ERR_NULL;
  return to_status(bsg::launch_block_pool(*dims, k_cache, page_table, kv_lens, blk_begin, block_cache,
                                          (hipStream_t)stream));
}

int bsg_group_score(const bsg_dims* dims, const void* q, int32_t q_len, const int32_t* kv_lens,
                    const void* block_cache, const int32_t* page_table, float* scores, int32_t score_stride,
                    void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!q || !kv_lens || !block_cache || !page_table || !scores) return BSG_ERR_NULL;
  if (q_len < 1 || score_stride < 1) return BSG_ERR_SHAPE;
  return to_status(bsg::launch_group_score(*dims, q, q_len, kv_lens, block_cache, page_table, scores, score_stride,
                                           (hipStream_t)stream));
}

int bsg_topk_blocks(const bsg_dims* dims, const float* scores, int32_t q_len, int32_t score_stride,
                    const int32_t* kv_lens, int32_t* block_idx, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!scores || !kv_lens || !block_idx) return BSG_ERR_NULL;
  if (q_len < 1 || score_stride < 1) return BSG_ERR_SHAPE;
  return to_status(bsg::launch_topk(*dims, scores, q_len, score_stride, kv_lens, block_idx, (hipStream_t)stream));
}

size_t bsg_group_score_topk_workspace_bytes(const bsg_dims* dims, int32_t q_len) {
  if (check_dims(dims) || q_len < 1) return 0;
  if (bsg::group_score_topk_fused_supported(*dims, q_len)) return 0;
  if (bsg::decode_select_supported(*dims, q_len)) return bsg::decode_select_workspace_bytes(*dims);
  return (size_t)dims->batch * dims->num_kv_heads * (size_t)q_len * dims->pt_stride * sizeof(float);
}

int bsg_group_score_topk(const bsg_dims* dims, const void* q, int32_t q_len, const int32_t* kv_lens,
                         const void* block_cache, const int32_t* page_table, int32_t* block_idx, void* workspace,
                         size_t workspace_bytes, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!q || !kv_lens || !block_cache || !page_table || !block_idx) return BSG_ERR_NULL;
  if (q_len < 1) return BSG_ERR_SHAPE;
  const size_t need = bsg_group_score_topk_workspace_bytes(dims, q_len);
  if (need > 0 && (!workspace || workspace_bytes < need)) return BSG_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (bsg::group_score_topk_fused_supported(*dims, q_len))
    return to_status(bsg::launch_group_score_topk_fused(*dims, q, q_len, kv_lens, block_cache, page_table,
                                                        block_idx, s));
  if (bsg::decode_select_supported(*dims, q_len))
    return to_status(bsg::launch_decode_select(*dims, q, kv_lens, block_cache, page_table, block_idx, workspace, s));
  float* scores = (float*)workspace;
  hipError_t e = bsg::launch_group_score(*dims, q, q_len, kv_lens, block_cache, page_table, scores,
                                         dims->pt_stride, s);
  if (e != hipSuccess) return BSG_ERR_HIP;
  return to_status(bsg::launch_topk(*dims, scores, q_len, dims->pt_stride, kv_lens, block_idx, s));
}

int bsg_sparse_attn_prefill(const bsg_dims* dims, const void* q, int32_t q_len, const int32_t* kv_lens,
                            const void* k_cache, const void* v_cache, const int32_t* page_table,
                            const int32_t* block_idx, float scale, void* out, float* lse, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!q || !kv_lens || !k_cache || !v_cache || !page_table || !block_idx || !out) return BSG_ERR_NULL;
  if (q_len < 1) return BSG_ERR_SHAPE;
  return to_status(bsg::launch_attn_prefill(*dims, q, q_len, kv_lens, k_cache, v_cache, page_table, block_idx,
                                            scale, out, lse, (hipStream_t)stream));
}

int bsg_sparse_attn_prefill_gated(const bsg_dims* dims, const void* q, int32_t q_len, const int32_t* kv_lens,
                                  const void* k_cache, const void* v_cache, const int32_t* page_table,
                                  const int32_t* block_idx, float scale, const float* gate, int32_t gate_per_dim,
                                  const void* x, void* out, float* lse, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!q || !kv_lens || !k_cache || !v_cache || !page_table || !block_idx || !out || !gate || !x)
    return BSG_ERR_NULL;
  if (q_len < 1 || (gate_per_dim != 0 && gate_per_dim != 1)) return BSG_ERR_SHAPE;
  return to_status(bsg::launch_attn_prefill(*dims, q, q_len, kv_lens, k_cache, v_cache, page_table, block_idx,
                                            scale, out, lse, (hipStream_t)stream, {gate, gate_per_dim, x}));
}

size_t bsg_decode_workspace_bytes(const bsg_dims* dims) {
  if (check_dims(dims)) return 0;
  return bsg::decode_workspace_bytes(*dims);
}

int bsg_sparse_attn_decode(const bsg_dims* dims, const void* q, const int32_t* kv_lens, const void* k_cache,
                           const void* v_cache, const int32_t* page_table, const int32_t* block_idx, float scale,
                           void* workspace, size_t workspace_bytes, void* out, float* lse, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!q || !kv_lens || !k_cache || !v_cache || !page_table || !block_idx || !out) return BSG_ERR_NULL;
  const int G = dims->num_q_heads / dims->num_kv_heads;
  if (G * dims->head_dim > 2048) return BSG_ERR_UNSUPPORTED;
  const size_t need = bsg::decode_workspace_bytes(*dims);
  if (!workspace || workspace_bytes < need) return BSG_ERR_WORKSPACE;
  return to_status(bsg::launch_attn_decode(*dims, q, kv_lens, k_cache, v_cache, page_table, block_idx, scale,
                                           workspace, out, lse, (hipStream_t)stream));
}

static size_t decode_step_ws_split(const bsg_dims* d, size_t* a_out) {
  // [selection workspace | attention partials], each 256-byte aligned
  const size_t a = (bsg_group_score_topk_workspace_bytes(d, 1) + 255) / 256 * 256;
  *a_out = a;
  return a + bsg::decode_workspace_bytes(*d);
}

size_t bsg_decode_step_workspace_bytes(const bsg_dims* dims) {
  if (check_dims(dims)) return 0;
  if (bsg::decode_step_fused_supported(*dims)) return bsg::decode_step_workspace_bytes(*dims);
  size_t a;
  return decode_step_ws_split(dims, &a);
}

static int decode_step_impl(const bsg_dims* dims, const void* q, const int32_t* kv_lens, const void* block_cache,
                            const void* k_cache, const void* v_cache, const int32_t* page_table, float scale,
                            int32_t* block_idx, void* workspace, size_t workspace_bytes, void* out, float* lse,
                            void* stream, bsg::gate_args ga) {
  int st = check_dims(dims);
  if (st) return st;
  if (!q || !kv_lens || !block_cache || !k_cache || !v_cache || !page_table || !block_idx || !out)
    return BSG_ERR_NULL;
  const int G = dims->num_q_heads / dims->num_kv_heads;
  if (G * dims->head_dim > 2048) return BSG_ERR_UNSUPPORTED;
  const size_t need = bsg_decode_step_workspace_bytes(dims);
  if (!workspace || workspace_bytes < need) return BSG_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (bsg::decode_step_fused_supported(*dims))
    return to_status(bsg::launch_decode_step(*dims, q, kv_lens, block_cache, k_cache, v_cache, page_table, scale,
                                             block_idx, workspace, out, lse, s, ga));
  size_t a;
  decode_step_ws_split(dims, &a);
  st = bsg_group_score_topk(dims, q, 1, kv_lens, block_cache, page_table, block_idx, workspace, a, stream);
  if (st) return st;
  if (!ga.g)
    return bsg_sparse_attn_decode(dims, q, kv_lens, k_cache, v_cache, page_table, block_idx, scale,
                                  (char*)workspace + a, workspace_bytes - a, out, lse, stream);
  if (workspace_bytes - a < bsg::decode_workspace_bytes(*dims)) return BSG_ERR_WORKSPACE;
  return to_status(bsg::launch_attn_decode(*dims, q, kv_lens, k_cache, v_cache, page_table, block_idx, scale,
                                           (char*)workspace + a, out, lse, s, ga));
}

int bsg_decode_step(const bsg_dims* dims, const void* q, const int32_t* kv_lens, const void* block_cache,
                    const void* k_cache, const void* v_cache, const int32_t* page_table, float scale,
                    int32_t* block_idx, void* workspace, size_t workspace_bytes, void* out, float* lse, void* stream) {
  return decode_step_impl(dims, q, kv_lens, block_cache, k_cache, v_cache, page_table, scale, block_idx, workspace,
                          workspace_bytes, out, lse, stream, {nullptr, 0, nullptr});
}

int bsg_decode_step_gated(const bsg_dims* dims, const void* q, const int32_t* kv_lens, const void* block_cache,
                          const void* k_cache, const void* v_cache, const int32_t* page_table, float scale,
                          int32_t* block_idx, void* workspace, size_t workspace_bytes, const float* gate,
                          int32_t gate_per_dim, const void* x, void* out, float* lse, void* stream) {
  const int st = check_dims(dims);
  if (st) return st;
  if (!gate || !x) return BSG_ERR_NULL;
  if (gate_per_dim != 0 && gate_per_dim != 1) return BSG_ERR_SHAPE;
  return decode_step_impl(dims, q, kv_lens, block_cache, k_cache, v_cache, page_table, scale, block_idx, workspace,
                          workspace_bytes, out, lse, stream, {gate, gate_per_dim, x});
}

int bsg_quantize_pages_fp8(const bsg_dims* dims, const void* src, const int32_t* page_table,
                           const int32_t* kv_lens, uint8_t* codes, float* scales, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->dtype != BSG_BF16) return BSG_ERR_UNSUPPORTED;
  if (!src || !page_table || !kv_lens || !codes || !scales) return BSG_ERR_NULL;
  return to_status(bsg::launch_quantize_pages_fp8(*dims, src, page_table, kv_lens, codes, scales,
                                                  (hipStream_t)stream));
}

int bsg_block_pool_fp8(const bsg_dims* dims, const uint8_t* k_codes, const float* k_scales,
                       const int32_t* page_table, const int32_t* kv_lens, const int32_t* blk_begin,
                       uint8_t* rep_codes, float* rep_scales, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->dtype != BSG_BF16) return BSG_ERR_UNSUPPORTED;
  if (!k_codes || !k_scales || !page_table || !kv_lens || !rep_codes || !rep_scales) return BSG_ERR_NULL;
  return to_status(bsg::launch_block_pool_fp8(*dims, k_codes, k_scales, page_table, kv_lens, blk_begin, rep_codes,
                                              rep_scales, (hipStream_t)stream));
}

int bsg_decode_step_fp8(const bsg_dims* dims, const void* q, const int32_t* kv_lens,
                        const uint8_t* rep_codes, const float* rep_scales, const uint8_t* k_codes,
                        const float* k_scales, const uint8_t* v_codes, const float* v_scales,
                        const int32_t* page_table, float scale, int32_t* block_idx, void* workspace,
                        size_t workspace_bytes, void* out, float* lse, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->dtype != BSG_BF16) return BSG_ERR_UNSUPPORTED;
  if (!q || !kv_lens || !rep_codes || !rep_scales || !k_codes || !k_scales || !v_codes || !v_scales ||
      !page_table || !block_idx || !out)
    return BSG_ERR_NULL;
  if (!bsg::decode_step_fused_supported(*dims)) return BSG_ERR_UNSUPPORTED;
  const size_t need = bsg_decode_step_workspace_bytes(dims);
  if (!workspace || workspace_bytes < need) return BSG_ERR_WORKSPACE;
  return to_status(bsg::launch_decode_step(*dims, q, kv_lens, rep_codes, k_codes, v_codes, page_table, scale,
                                           block_idx, workspace, out, lse, (hipStream_t)stream,
                                           bsg::gate_args{nullptr, 0, nullptr}, rep_scales, k_scales, v_scales));
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t bsg_token_topk_workspace_bytes(const bsg_dims* dims, int32_t two_level) {
  if (check_dims(dims)) return 0;
  return bsg::token_topk_workspace_bytes(*dims, two_level != 0);
}

int bsg_token_topk(const bsg_dims* dims, const void* q, const int32_t* kv_lens, const void* k_cache,
                   const int32_t* page_table, const int32_t* block_idx, int32_t top_k_tokens, int32_t* token_idx,
                   void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->dtype != BSG_BF16) return BSG_ERR_UNSUPPORTED;
  if (!q || !kv_lens || !k_cache || !page_table || !token_idx) return BSG_ERR_NULL;
  if (top_k_tokens < 1) return BSG_ERR_SHAPE;
  const size_t need = bsg::token_topk_workspace_bytes(*dims, block_idx != nullptr);
  if (!workspace || workspace_bytes < need) return BSG_ERR_WORKSPACE;
  return to_status(bsg::launch_token_topk(*dims, q, kv_lens, k_cache, page_table, block_idx, top_k_tokens,
                                          token_idx, workspace, (hipStream_t)stream));
}

size_t bsg_token_topk_prefill_workspace_bytes(const bsg_dims* dims, int32_t q_len, int32_t two_level) {
  if (check_dims(dims) || q_len < 1) return 0;
  return bsg::token_topk_prefill_workspace_bytes(*dims, q_len, two_level != 0);
}

int bsg_token_topk_prefill(const bsg_dims* dims, const void* q, int32_t q_len, const int32_t* kv_lens,
                           const void* k_cache, const int32_t* page_table, const int32_t* block_idx,
                           int32_t top_k_tokens, int32_t* token_idx, void* workspace, size_t workspace_bytes,
                           void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->dtype != BSG_BF16) return BSG_ERR_UNSUPPORTED;
  if (!q || !kv_lens || !k_cache || !page_table || !token_idx) return BSG_ERR_NULL;
  if (q_len < 1 || top_k_tokens < 1) return BSG_ERR_SHAPE;
  const size_t need = bsg::token_topk_prefill_workspace_bytes(*dims, q_len, block_idx != nullptr);
  if (!workspace || workspace_bytes < need) return BSG_ERR_WORKSPACE;
  return to_status(bsg::launch_token_topk_prefill(*dims, q, q_len, kv_lens, k_cache, page_table, block_idx,
                                                  top_k_tokens, token_idx, workspace, (hipStream_t)stream));
}

int bsg_sparse_attn_prefill_tokens(const bsg_dims* dims, const void* q, int32_t q_len, const int32_t* kv_lens,
                                   const void* k_cache, const void* v_cache, const int32_t* page_table,
                                   const int32_t* token_idx, int32_t top_k_tokens, float scale, void* out,
                                   float* lse, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!bsg::token_attn_supported(*dims)) return BSG_ERR_UNSUPPORTED;
  if (!q || !kv_lens || !k_cache || !v_cache || !page_table || !token_idx || !out) return BSG_ERR_NULL;
  if (q_len < 1 || top_k_tokens < 1) return BSG_ERR_SHAPE;
  return to_status(bsg::launch_attn_prefill_tokens(*dims, q, q_len, kv_lens, k_cache, v_cache, page_table,
                                                   token_idx, top_k_tokens, scale, out, lse, (hipStream_t)stream));
}

size_t bsg_decode_tokens_workspace_bytes(const bsg_dims* dims, int32_t top_k_tokens) {
  if (check_dims(dims) || top_k_tokens < 1) return 0;
  return bsg::token_attn_workspace_bytes(*dims, top_k_tokens);
}

int bsg_sparse_attn_decode_tokens(const bsg_dims* dims, const void* q, const int32_t* kv_lens, const void* k_cache,
                                  const void* v_cache, const int32_t* page_table, const int32_t* token_idx,
                                  int32_t top_k_tokens, float scale, void* workspace, size_t workspace_bytes,
                                  void* out, float* lse, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!bsg::token_attn_supported(*dims)) return BSG_ERR_UNSUPPORTED;
  if (!q || !kv_lens || !k_cache || !v_cache || !page_table || !token_idx || !out) return BSG_ERR_NULL;
  if (top_k_tokens < 1) return BSG_ERR_SHAPE;
  if (!workspace || workspace_bytes < bsg::token_attn_workspace_bytes(*dims, top_k_tokens)) return BSG_ERR_WORKSPACE;
  return to_status(bsg::launch_attn_decode_tokens(*dims, q, kv_lens, k_cache, v_cache, page_table, token_idx,
                                                  top_k_tokens, scale, workspace, out, lse, (hipStream_t)stream));
}

size_t bsg_decode_step_tokens_workspace_bytes(const bsg_dims* dims, int32_t top_k_tokens, int32_t two_level) {
  if (check_dims(dims) || top_k_tokens < 1) return 0;
  const size_t sel = two_level ? align256(bsg_group_score_topk_workspace_bytes(dims, 1)) : 0;
  return sel + align256(bsg::token_topk_workspace_bytes(*dims, two_level != 0)) +
         bsg::token_attn_workspace_bytes(*dims, top_k_tokens);
}

int bsg_decode_step_tokens(const bsg_dims* dims, const void* q, const int32_t* kv_lens, const void* block_cache,
                           const void* k_cache, const void* v_cache, const int32_t* page_table,
                           int32_t top_k_tokens, int32_t two_level, float scale, int32_t* block_idx,
                           int32_t* token_idx, void* workspace, size_t workspace_bytes, void* out, float* lse,
                           void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->dtype != BSG_BF16 || !bsg::token_attn_supported(*dims)) return BSG_ERR_UNSUPPORTED;
  if (!q || !kv_lens || !k_cache || !v_cache || !page_table || !token_idx || !out) return BSG_ERR_NULL;
  if (two_level && (!block_cache || !block_idx)) return BSG_ERR_NULL;
  if (top_k_tokens < 1) return BSG_ERR_SHAPE;
  const size_t need = bsg_decode_step_tokens_workspace_bytes(dims, top_k_tokens, two_level);
  if (!workspace || workspace_bytes < need) return BSG_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  size_t off = 0;
  if (two_level) {
    const size_t a = align256(bsg_group_score_topk_workspace_bytes(dims, 1));
    st = bsg_group_score_topk(dims, q, 1, kv_lens, block_cache, page_table, block_idx, ws, a, stream);
    if (st) return st;
    off = a;
  }
  const size_t b = align256(bsg::token_topk_workspace_bytes(*dims, two_level != 0));
  hipError_t e = bsg::launch_token_topk(*dims, q, kv_lens, k_cache, page_table, two_level ? block_idx : nullptr,
                                        top_k_tokens, token_idx, ws + off, s);
  if (e != hipSuccess) return BSG_ERR_HIP;
  return to_status(bsg::launch_attn_decode_tokens(*dims, q, kv_lens, k_cache, v_cache, page_table, token_idx,
                                                  top_k_tokens, scale, ws + off + b, out, lse, s));
}

}  // extern "C"
