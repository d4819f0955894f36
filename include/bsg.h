/*
 * bsg.h -- C ABI of the block-sparse GQA attention library for AMD MI355X (gfx950).
 *
 * The method (Ling 2.0 sparse attention / MiniMax Sparse Attention):
 *   - keys and values live in a paged KV cache; a block is one page;
 *   - each complete block is summarised by the mean of its keys, per KV head,
 *     in a block cache that is indexed by the same physical page ids as the KV
 *     cache ("Art of Focus: Ling 2.0 and the Revolution in Sparse Attention",
 *     section "Summarizing the Breakthrough": block representations are built
 *     at prefill, kept in a page-aware block cache that shares the KV cache's
 *     indexing, and only the chosen blocks are fetched at decode);
 *   - all query heads of a GQA group share one block selection: the group's
 *     summed query is scored against the block representatives and the top-k
 *     causal blocks are kept, the query's own block always among them
 *     (same section; "MiniMax Sparse Attention (MSA)" post, second paragraph);
 *   - exact softmax attention then runs over the selected blocks only
 *     ("Sparse Attention + Linear Backbones", section 5.5 "Pseudocode Sketch";
 *     MSA post, second paragraph).
 *
 * Conventions shared by every call
 * --------------------------------
 *   - Every tensor pointer is a DEVICE pointer to contiguous row-major memory
 *     owned by the caller.  `dims` points to HOST memory.  The library keeps
 *     no state between calls, allocates no device memory, and is reentrant.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued; nothing synchronises.  Calls on one stream run in order.
 *   - Every call validates its host-side arguments first.  On any error it
 *     returns a negative bsg_status and enqueues nothing.  A failed kernel
 *     launch returns BSG_ERR_HIP.
 *   - Device-side contents are trusted: page ids must be < num_pages, block
 *     ids in block_idx must be -1 or < ceil(kv_len / page_size), and
 *     q_len <= kv_len <= pt_stride * page_size.  Kernels clamp page and block
 *     ids into range (so a bad table cannot make them read out of bounds) but
 *     the results for such inputs are unspecified.
 *   - Layouts (B = batch, Hq / Hkv = query / KV heads, G = Hq / Hkv,
 *     D = head_dim, bs = page_size = block size, P = num_pages):
 *       k_cache, v_cache : [P, Hkv, bs, D]   dtype
 *       block_cache      : [P, Hkv, D]       dtype (representative of the block
 *                                            stored in page p, per KV head)
 *       page_table       : int32 [B, pt_stride]; logical block j of sequence b
 *                          is physical page page_table[b*pt_stride + j]
 *       kv_lens          : int32 [B]; tokens of sequence b in the cache
 *       q                : [B, Hq, q_len, D] dtype; query t of sequence b sits
 *                          at position kv_lens[b] - q_len + t (decode: q_len = 1)
 *       block_idx        : int32 [B, Hkv, q_len, top_k]; logical block ids of
 *                          the selection, ascending, padded with -1 at the end
 *       out              : [B, Hq, q_len, D] dtype;  lse : fp32 [B, Hq, q_len]
 *     Query head h belongs to group g = h / G.
 *   - Supported: dtype f32 or bf16; head_dim 64 or 128; page_size 64 or 128;
 *     1 <= top_k <= 64; Hq a multiple of Hkv.
 */
#ifndef BSG_H
#define BSG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSG_OK = 0,
  BSG_ERR_NULL = -1,        /* a required pointer is NULL */
  BSG_ERR_SHAPE = -2,       /* inconsistent or non-positive sizes */
  BSG_ERR_UNSUPPORTED = -3, /* valid but not implemented (dtype, D, page size, k) */
  BSG_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
  BSG_ERR_HIP = -5,         /* the HIP runtime reported an error at launch */
  BSG_ERR_SCRATCH = -6      /* the sizes need more than the library's static scratch
                               (bsg_decode_step_noalloc only) */
} bsg_status;

typedef enum { BSG_F32 = 0, BSG_BF16 = 1 } bsg_dtype;

typedef struct {
  int32_t batch;        /* B */
  int32_t num_q_heads;  /* Hq */
  int32_t num_kv_heads; /* Hkv */
  int32_t head_dim;     /* D */
  int32_t page_size;    /* bs: tokens per page = tokens per block */
  int32_t top_k;        /* blocks kept per (sequence, group, query), own block included */
  int32_t num_pages;    /* P: pages in the K / V pools and in the block cache */
  int32_t pt_stride;    /* row stride of page_table = max logical blocks per sequence */
  int32_t dtype;        /* bsg_dtype of q, caches and out */
} bsg_dims;

/* Library version (major * 10000 + minor * 100 + patch). */
int bsg_version(void);

/* Human-readable name of a bsg_status value (static string). */
const char* bsg_status_str(int status);

/*
 * bsg_debug_errors -- the ids the kernels had to clamp, in a library built with -DBSG_DEBUG
 * (block_sparse_gqa_pool_amd.build --debug: libbsg_debug.so).  Every kernel clamps the ids
 * it reads from the caller's tables before they address memory, so a bad entry never takes
 * it out of its buffers; the debug build also records each clamped id in a device word:
 *     bit 0 (1): a page-table entry outside [0, num_pages) for a block the call reads,
 *     bit 1 (2): a block id of block_idx at or past pt_stride,
 *     bit 2 (4): a token id of token_idx at or past pt_stride * page_size.
 * *bits receives the OR of the words of the current device; reset != 0 then clears them.
 * Synchronous (waits for the device).  A release build returns BSG_ERR_UNSUPPORTED.
 */
int bsg_debug_errors(unsigned int* bits, int reset);

/*
 * bsg_block_pool -- write block representatives for complete blocks.
 * Follows the Ling 2.0 page, "Summarizing the Breakthrough" (blocks are
 * aggregated into representatives stored in a cache that shares the KV
 * cache's page indexing); the aggregate is the mean of the block's keys.
 *
 * For each sequence b and each complete logical block
 *     j in [blk_begin[b], kv_lens[b] / page_size)
 * with p = page_table[b, j]:
 *     block_cache[p, g, :] = round(  (K[p, g, 0, :] + ... + K[p, g, bs-1, :])
 *                                   * (1 / bs) )
 * where the sum is taken in fp32 in token order and round() is
 * round-to-nearest-even into the cache dtype.  Entries of other pages are not
 * touched.  blk_begin may be NULL (= 0 for every sequence); pass
 * blk_begin[b] = kv_lens[b] / bs - 1 after a page completes to refresh only
 * that page.  The result is bit-identical for every launch configuration.
 */
int bsg_block_pool(const bsg_dims* dims, const void* k_cache, const int32_t* page_table,
                   const int32_t* kv_lens, const int32_t* blk_begin, void* block_cache,
                   void* stream);

/*
 * bsg_group_score -- materialised group scores.
 * Follows the Ling 2.0 page, "Summarizing the Breakthrough" (the heads of a
 * GQA group share the selection) and the MSA post, second paragraph (blocks
 * are scored per GQA group).
 *
 * scores: fp32 [B, Hkv, q_len, score_stride].  For query t at position p and
 * own block o = p / page_size:
 *     scores[b, g, t, j] = sum over the G heads h of group g of
 *                          q[b, h, t, :] . block_cache[page_table[b, j], g, :]
 * for j < min(o, score_stride), computed in fp32; every other entry
 * j < score_stride is -inf.  No 1/sqrt(D) factor (it does not change ranks).
 */
int bsg_group_score(const bsg_dims* dims, const void* q, int32_t q_len, const int32_t* kv_lens,
                    const void* block_cache, const int32_t* page_table, float* scores,
                    int32_t score_stride, void* stream);

/*
 * bsg_topk_blocks -- causal top-k selection from materialised scores.
 * Follows the MSA post, second and third paragraphs (top-k per GQA group,
 * selected without exponentials).
 *
 * For each row (b, g, t) with own block o: the min(top_k - 1, o) candidates
 * j < o with the largest scores[b, g, t, j] are kept (equal scores: the lower
 * block index wins; -0.0 equals +0.0), the own block o is added, and the
 * kept ids are written ascending to block_idx[b, g, t, :], padded with -1.
 * Requires score_stride >= the largest own block of any row.
 */
int bsg_topk_blocks(const bsg_dims* dims, const float* scores, int32_t q_len, int32_t score_stride,
                    const int32_t* kv_lens, int32_t* block_idx, void* stream);

/*
 * bsg_group_score_topk -- fused scoring and selection (no materialised scores).
 * Same result as bsg_group_score followed by bsg_topk_blocks, except that the
 * fp32 scores may be accumulated in a different order, so rows whose k-th
 * and (k+1)-th candidates score within fp32 rounding of each other may
 * differ.  `workspace` (device, may be NULL when the query below returns 0)
 * must hold bsg_group_score_topk_workspace_bytes(dims, q_len) bytes.
 */
size_t bsg_group_score_topk_workspace_bytes(const bsg_dims* dims, int32_t q_len);
int bsg_group_score_topk(const bsg_dims* dims, const void* q, int32_t q_len, const int32_t* kv_lens,
                         const void* block_cache, const int32_t* page_table, int32_t* block_idx,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * bsg_sparse_attn_prefill -- exact attention over the selected blocks.
 * Follows "Sparse Attention + Linear Backbones", section 5.5 (softmax of
 * q.k / sqrt(d) over the selected keys times their values) and "Sparse
 * Attention for Long-Context LLMs", section 4.3 (the top-k mask removes the
 * unselected keys; read as an additive -inf mask, so they are skipped).
 *
 * For query head h (group g) at position p, the keys are the tokens
 * i <= p of the blocks listed in block_idx[b, g, t, :] (-1 entries ignored):
 *     z_i   = scale * (q[b, h, t, :] . K_i)
 *     out   = sum_i softmax(z)_i V_i          (rounded to the dtype)
 *     lse   = max z + ln(sum_i exp(z_i - max z))    (fp32; lse may be NULL)
 * Accumulation is fp32; bf16 inputs use bf16 matrix-core products.  Token
 * slots of a page beyond kv_len are never used (their contents may be
 * anything, NaN included).
 */
int bsg_sparse_attn_prefill(const bsg_dims* dims, const void* q, int32_t q_len,
                            const int32_t* kv_lens, const void* k_cache, const void* v_cache,
                            const int32_t* page_table, const int32_t* block_idx, float scale,
                            void* out, float* lse, void* stream);

/*
 * bsg_sparse_attn_prefill_gated -- bsg_sparse_attn_prefill followed by the gated fusion
 * of its output A with a caller tensor x ("Sparse Attention for Long-Context LLMs",
 * section 4.3 "Gating Mechanisms Reduce Risk", step 6: the output is Gate * A plus
 * (1 - Gate) times the original representation, the gate being a scalar or a
 * per-dimension vector; the pseudocode of the Linear Backbones page, section 5.5, also
 * ends with a gated fusion):
 *     out = g * A + (1 - g) * x
 * computed in fp32 from the fp32 attention output and rounded once to the dtype.
 * gate : fp32, [B, Hq, q_len] (gate_per_dim = 0: one gate per head and query) or
 *        [B, Hq, q_len, D] (gate_per_dim = 1: one gate per element); any values.
 * x    : [B, Hq, q_len, D] in the dtype (the layout of out; may not alias out).
 * lse is that of A.  gate and x must not be NULL (BSG_ERR_NULL); gate_per_dim other than
 * 0 or 1 is BSG_ERR_SHAPE.  Everything else as bsg_sparse_attn_prefill.
 */
int bsg_sparse_attn_prefill_gated(const bsg_dims* dims, const void* q, int32_t q_len,
                                  const int32_t* kv_lens, const void* k_cache, const void* v_cache,
                                  const int32_t* page_table, const int32_t* block_idx, float scale,
                                  const float* gate, int32_t gate_per_dim, const void* x, void* out,
                                  float* lse, void* stream);

/*
 * bsg_sparse_attn_decode -- one query token per sequence (q_len = 1), split
 * over the selected blocks with a log-sum-exp merge.  Same definition as
 * bsg_sparse_attn_prefill with q_len = 1; block_idx is [B, Hkv, top_k].
 * Follows the Ling 2.0 page, "Summarizing the Breakthrough" (at decode only
 * the selected blocks are fetched).
 *
 * The selected blocks of each (sequence, group) are split over several
 * workgroups; each writes a partial (max, sum, unnormalised output) per query
 * head to `workspace`, and the partials are merged:
 *     m = max_s m_s,  l = sum_s l_s e^(m_s - m),  out = sum_s o_s e^(m_s - m) / l.
 * `workspace` (device) must hold bsg_decode_workspace_bytes(dims) bytes; its
 * contents need no initialisation.  Two calls that share a workspace must not
 * run concurrently.
 */
size_t bsg_decode_workspace_bytes(const bsg_dims* dims);
int bsg_sparse_attn_decode(const bsg_dims* dims, const void* q, const int32_t* kv_lens,
                           const void* k_cache, const void* v_cache, const int32_t* page_table,
                           const int32_t* block_idx, float scale, void* workspace,
                           size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * bsg_decode_step -- one whole decode step: group scores against the block
 * cache, causal top-k selection, and sparse attention over the selected
 * blocks, for q_len = 1.  The same selection as bsg_group_score_topk (also
 * written to block_idx, [B, Hkv, top_k]) and the same attention as
 * bsg_sparse_attn_decode on it (outputs within bf16 rounding: the split of the
 * pages over workgroups differs).  Page-table rows of at most 4096 blocks run
 * scan, selection and attention in one kernel plus a merge of partials; longer
 * rows scan in chunks and finish the selection inside the attention kernel.
 * Follows the Ling 2.0 page, "Summarizing the Breakthrough" (decode reads the
 * block cache, picks the top-k blocks and fetches only those).
 * q: [B, Hq, D]; out: [B, Hq, D]; lse: fp32 [B, Hq] or NULL.  `workspace`
 * (device, no initialisation needed) must hold
 * bsg_decode_step_workspace_bytes(dims) bytes.
 */
size_t bsg_decode_step_workspace_bytes(const bsg_dims* dims);
int bsg_decode_step(const bsg_dims* dims, const void* q, const int32_t* kv_lens, const void* block_cache,
                    const void* k_cache, const void* v_cache, const int32_t* page_table, float scale,
                    int32_t* block_idx, void* workspace, size_t workspace_bytes, void* out, float* lse,
                    void* stream);

/*
 * bsg_decode_step_gated -- bsg_decode_step with the same gated fusion as
 * bsg_sparse_attn_prefill_gated applied to its output (gate: fp32 [B, Hq] or [B, Hq, D];
 * x: [B, Hq, D] in the dtype).  Workspace as bsg_decode_step.
 */
int bsg_decode_step_gated(const bsg_dims* dims, const void* q, const int32_t* kv_lens,
                          const void* block_cache, const void* k_cache, const void* v_cache,
                          const int32_t* page_table, float scale, int32_t* block_idx, void* workspace,
                          size_t workspace_bytes, const float* gate, int32_t gate_per_dim, const void* x,
                          void* out, float* lse, void* stream);

/*
 * bsg_decode_step_noalloc -- bsg_decode_step without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a static device array of the library,
 * BSG_NOALLOC_SCRATCH_BYTES bytes per GPU, held until the process ends; the call allocates
 * nothing.  Same arguments, results and validation as bsg_decode_step; if the sizes need more
 * workspace than the array holds (bsg_decode_step_workspace_bytes(dims) >
 * bsg_noalloc_scratch_bytes()) it returns BSG_ERR_SCRATCH and enqueues nothing.  All calls
 * on one GPU share that GPU's array: calls that overlap in time on one GPU (other streams,
 * other host threads) race and must not be issued; calls in order on one stream are safe.
 */
#define BSG_NOALLOC_SCRATCH_BYTES (8u << 20)
size_t bsg_noalloc_scratch_bytes(void);
int bsg_decode_step_noalloc(const bsg_dims* dims, const void* q, const int32_t* kv_lens,
                            const void* block_cache, const void* k_cache, const void* v_cache,
                            const int32_t* page_table, float scale, int32_t* block_idx, void* out,
                            float* lse, void* stream);

/*
 * fp8 KV cache and block cache.  The pages list KV-cache quantisation among the
 * system-level optimisations that leave the model untouched ("Sparse Attention +
 * Linear Backbones", section 3) and as a companion of sparse attention ("Sparse
 * Attention for Long-Context LLMs", section 8); they fix no format.  Format used here:
 * OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest 448;
 * no infinities) with one fp32 power-of-two scale per (page, KV head) tile:
 *     value = decode(code) * scale.
 * dims describes the bf16 cache the codes stand for (dtype must be BSG_BF16, else
 * BSG_ERR_UNSUPPORTED); codes use the cache's layout with 1-byte elements.
 */

/*
 * bsg_quantize_pages_fp8 -- codes and scales of a bf16 paged cache (K or V).
 * src: bf16 [P, Hkv, page_size, D].  For every sequence b and every block
 * j < min(ceil(kv_lens[b] / page_size), pt_stride), with p = page_table[b, j] and
 * n = min(page_size, kv_lens[b] - j * page_size) valid tokens, and every head g:
 *     scale[p, g] = 2^e, e the smallest integer with max|src[p, g, :n, :]| <= 448 * 2^e
 *                   (e = 0 for an all-zero tile; e clamped to [-126, 127]);
 *     codes[p, g, i, :] = nearest-even E4M3 code of src[p, g, i, :] / 2^e  for i < n,
 *     codes[p, g, i, :] = 0                                                for i >= n.
 * codes: uint8 [P, Hkv, page_size, D]; scales: fp32 [P, Hkv].  Tiles of other pages
 * are not touched.  A page may belong to one sequence only (two sequences sharing a
 * page would write it concurrently).  Deterministic, bit-exact.
 */
int bsg_quantize_pages_fp8(const bsg_dims* dims, const void* src, const int32_t* page_table,
                           const int32_t* kv_lens, uint8_t* codes, float* scales, void* stream);

/*
 * bsg_block_pool_fp8 -- fp8 block cache from the fp8 key cache (the block
 * representative of bsg_block_pool, on the decoded keys).  For each sequence b and each
 * complete block j in [blk_begin[b], kv_lens[b] / page_size), p = page_table[b, j]:
 *     mean[g, :] = (sum over tokens i in order, in fp32, of decode(k_codes[p, g, i, :]))
 *                  * (k_scales[p, g] * (1 / page_size))          (fp32; exact scaling)
 *     rep_scales[p, g] = 2^e for max|mean[g, :]| as in bsg_quantize_pages_fp8,
 *     rep_codes[p, g, :] = nearest-even E4M3 codes of mean[g, :] / 2^e.
 * rep_codes: uint8 [P, Hkv, D]; rep_scales: fp32 [P, Hkv]; blk_begin may be NULL.
 * Entries of other pages are not touched.  Deterministic, bit-exact.
 */
int bsg_block_pool_fp8(const bsg_dims* dims, const uint8_t* k_codes, const float* k_scales,
                       const int32_t* page_table, const int32_t* kv_lens, const int32_t* blk_begin,
                       uint8_t* rep_codes, float* rep_scales, void* stream);

/*
 * bsg_decode_step_fp8 -- bsg_decode_step over fp8 caches: the block scores use the
 * decoded representatives (rep code * rep scale), attention the decoded keys and values.
 * The result is the one bsg_decode_step gives on bf16 caches holding the decoded values
 * (bit for bit: every scale is a power of two, applied exactly).  q and out stay bf16
 * ([B, Hq, D]); lse fp32 [B, Hq] or NULL; block_idx int32 [B, Hkv, top_k].  Workspace as
 * bsg_decode_step (bsg_decode_step_workspace_bytes(dims)).  Only the matrix-core decode
 * path is provided: G <= 16 and the fused selection's limits (bsg_decode_step_workspace_bytes
 * returns 0 outside them); elsewhere BSG_ERR_UNSUPPORTED.
 */
int bsg_decode_step_fp8(const bsg_dims* dims, const void* q, const int32_t* kv_lens,
                        const uint8_t* rep_codes, const float* rep_scales, const uint8_t* k_codes,
                        const float* k_scales, const uint8_t* v_codes, const float* v_scales,
                        const int32_t* page_table, float scale, int32_t* block_idx, void* workspace,
                        size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * Token-level and two-level selection for decode (q_len = 1, bf16).
 *
 * Token level follows "Sparse Attention + Linear Backbones", sections 5.1-5.3 and the
 * pseudocode of 5.5: an indexer scores every earlier position, the top_k_tokens
 * highest-scoring positions are kept per query, attention runs over those; the indexer
 * uses no positional encoding.  The learned indexer is absent, so the index is the identity
 * one: for the query heads of group g,
 *     score(s) = sum over the group's heads h of q[b, h, :] . K[token s, g, :]   (fp32)
 * over the candidates s <= kv_lens[b] - 1.  Two level follows "Sparse Attention for
 * Long-Context LLMs", section 8 (coarse filtering, then fine filtering): the candidates are
 * the tokens of the row's selected blocks, block_idx [B, Hkv, dims.top_k] (ascending, -1
 * padded, as bsg_topk_blocks writes it).  The top top_k_tokens candidates are kept by
 * (score, lower token first) and written ascending to token_idx [B, Hkv, top_k_tokens],
 * padded with -1 when there are fewer candidates.
 */

/*
 * bsg_token_topk -- token scores and exact top-K.  block_idx NULL: token level (every
 * token is a candidate; this reads the whole K cache of the batch); else two level.
 * workspace (device, no initialisation) >= bsg_token_topk_workspace_bytes(dims, two_level)
 * bytes: the fp32 scores, B * Hkv * (pt_stride * page_size, or top_k * page_size) of them.
 * dtype must be BSG_BF16.
 */
size_t bsg_token_topk_workspace_bytes(const bsg_dims* dims, int32_t two_level);
int bsg_token_topk(const bsg_dims* dims, const void* q, const int32_t* kv_lens, const void* k_cache,
                   const int32_t* page_table, const int32_t* block_idx, int32_t top_k_tokens,
                   int32_t* token_idx, void* workspace, size_t workspace_bytes, void* stream);

/*
 * bsg_sparse_attn_decode_tokens -- exact attention over the kept tokens of token_idx
 * [B, Hkv, top_k_tokens] (the group's list; -1 entries are skipped):
 *     out[b, h] = sum_s softmax_s(q[b, h] . k_s * scale) v_s,  lse = log sum_s exp(...),
 * split over workgroups with the log-sum-exp merge of bsg_sparse_attn_decode.  bf16 with
 * G = Hq / Hkv <= 16 (else BSG_ERR_UNSUPPORTED).  workspace >=
 * bsg_decode_tokens_workspace_bytes(dims, top_k_tokens) bytes.
 */
size_t bsg_decode_tokens_workspace_bytes(const bsg_dims* dims, int32_t top_k_tokens);
int bsg_sparse_attn_decode_tokens(const bsg_dims* dims, const void* q, const int32_t* kv_lens,
                                  const void* k_cache, const void* v_cache, const int32_t* page_table,
                                  const int32_t* token_idx, int32_t top_k_tokens, float scale,
                                  void* workspace, size_t workspace_bytes, void* out, float* lse,
                                  void* stream);

/*
 * bsg_decode_step_tokens -- a whole token-level (two_level = 0) or two-level (two_level = 1)
 * decode step: [block scores + block top-k into block_idx, as bsg_group_score_topk with
 * q_len = 1,] token top-K into token_idx, attention into out / lse.  block_cache and
 * block_idx are used (and required) for two_level only.  workspace >=
 * bsg_decode_step_tokens_workspace_bytes(dims, top_k_tokens, two_level) bytes.
 */
size_t bsg_decode_step_tokens_workspace_bytes(const bsg_dims* dims, int32_t top_k_tokens,
                                              int32_t two_level);
int bsg_decode_step_tokens(const bsg_dims* dims, const void* q, const int32_t* kv_lens,
                           const void* block_cache, const void* k_cache, const void* v_cache,
                           const int32_t* page_table, int32_t top_k_tokens, int32_t two_level,
                           float scale, int32_t* block_idx, int32_t* token_idx, void* workspace,
                           size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * Token-level and two-level selection for prefill: the same definitions as the decode
 * calls above, for each query position t of q [B, Hq, q_len, D] (cache position
 * kv_lens[b] - q_len + t; candidates s <= that position).  token_idx is
 * [B, Hkv, q_len, top_k_tokens] (ascending, -1 padded); block_idx (two level) is
 * [B, Hkv, q_len, dims.top_k] as bsg_group_score_topk writes it, NULL for token level.
 *
 * bsg_token_topk_prefill -- scores and exact top-K of every row.  Each tile of 128 positions
 * is scored against all earlier tokens on the matrix cores (the fp32 group-summed query as
 * three bf16 terms); two level then selects among the tokens of each row's blocks only.  The
 * positions go through in windows whose scores fit the workspace: >=
 * bsg_token_topk_prefill_workspace_bytes(dims, q_len, two_level) bytes, no initialisation.
 * dtype must be BSG_BF16.
 */
size_t bsg_token_topk_prefill_workspace_bytes(const bsg_dims* dims, int32_t q_len, int32_t two_level);
int bsg_token_topk_prefill(const bsg_dims* dims, const void* q, int32_t q_len, const int32_t* kv_lens,
                           const void* k_cache, const int32_t* page_table, const int32_t* block_idx,
                           int32_t top_k_tokens, int32_t* token_idx, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * bsg_sparse_attn_prefill_tokens -- exact attention of every query position over its kept
 * tokens (token_idx as above; -1 entries skipped):
 *     out[b, h, t] = sum_s softmax_s(q[b, h, t] . k_s * scale) v_s,  lse = log sum_s exp(...)
 * out [B, Hq, q_len, D] bf16, lse [B, Hq, q_len] fp32 or NULL.  One workgroup per
 * (sequence, position, group); no workspace.  bf16 with G = Hq / Hkv <= 16 (else
 * BSG_ERR_UNSUPPORTED).
 */
int bsg_sparse_attn_prefill_tokens(const bsg_dims* dims, const void* q, int32_t q_len, const int32_t* kv_lens,
                                   const void* k_cache, const void* v_cache, const int32_t* page_table,
                                   const int32_t* token_idx, int32_t top_k_tokens, float scale, void* out,
                                   float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSG_H */
