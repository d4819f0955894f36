// bsg_decode_step_noalloc: the decode step of bsg_decode_step with its workspace (the per-chunk
// selection lists and the split-attention partials) in a static device array of the library,
// for callers that cannot allocate device memory.
//
// The array is file-scope device memory, one copy per GPU, held until the process ends.  Host
// code never passes the array's name to a kernel (on the host that name is only a stand-in for
// the device symbol): the device address of this GPU's copy is looked up once per device with
// hipGetSymbolAddress, on the first call made while that device is current, and kept.  Every
// call on one GPU shares that GPU's copy, so calls that overlap in time on one GPU race (two
// streams, or two host threads); calls on one stream run in order and are safe.  The decode
// step needs no initialised workspace (each call writes every entry it later reads), so nothing
// is cleared between calls.
#include <mutex>

#include "bsg.h"
#include "bsg_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;   // BSG_NOALLOC_SCRATCH_BYTES in bsg.h
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array (looked up on the first call per device).
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return BSG_ERR_HIP;
  if (dev >= kMaxDevices) return BSG_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BSG_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BSG_OK;
}

}  // namespace

extern "C" {

size_t bsg_noalloc_scratch_bytes(void) { return kScratchBytes; }

int bsg_decode_step_noalloc(const bsg_dims* dims, const void* q, const int32_t* kv_lens, const void* block_cache,
                            const void* k_cache, const void* v_cache, const int32_t* page_table, float scale,
                            int32_t* block_idx, void* out, float* lse, void* stream) {
  if (!dims) return BSG_ERR_NULL;
  const size_t need = bsg_decode_step_workspace_bytes(dims);
  if (need == 0) {
    // invalid dims: let the full validation of bsg_decode_step report them
    return bsg_decode_step(dims, q, kv_lens, block_cache, k_cache, v_cache, page_table, scale, block_idx, nullptr,
                           0, out, lse, stream);
  }
  if (need > kScratchBytes) return BSG_ERR_SCRATCH;
  void* ws = nullptr;
  const int st = scratch_for_current_device(&ws);
  if (st) return st;
  return bsg_decode_step(dims, q, kv_lens, block_cache, k_cache, v_cache, page_table, scale, block_idx, ws,
                         kScratchBytes, out, lse, stream);
}

}  // extern "C"
