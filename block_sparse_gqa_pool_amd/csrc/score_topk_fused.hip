// Fused prefill scoring + selection.  (Not yet specialised: callers fall back to the
// materialised path.)
#include "bsg_device.h"
#include "bsg_internal.h"

namespace bsg {

bool group_score_topk_fused_supported(const bsg_dims& d, int q_len) {
  (void)d;
  (void)q_len;
  return false;
}

hipError_t launch_group_score_topk_fused(const bsg_dims& d, const void* q, int q_len, const int32_t* kv_lens,
                                         const void* block_cache, const int32_t* page_table, int32_t* block_idx,
                                         hipStream_t stream) {
  (void)d; (void)q; (void)q_len; (void)kv_lens; (void)block_cache; (void)page_table; (void)block_idx; (void)stream;
  return hipErrorNotSupported;
}

}  // namespace bsg
