// Draft pass with no allocation at all: the workspace dflash_draft_block takes
// from the caller lives here in a fixed device array instead, for callers that
// cannot allocate (code under graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  Same kernels and launch sequence as
// dflash_draft_block; only where the scratch comes from differs.
#include <stdio.h>

#include <mutex>

#include "internal.h"

namespace {

// Largest workspace the entry point serves (dflash_draft_workspace_bytes of
// the call): 64 MiB, enough for the Qwen3-8B-shaped draft at batch 1 with a
// 4096-token prefix (17 MiB) or batch 8 with 16384 (60 MiB).
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

// One copy per GPU, held until the process ends.  In host code `scratch` is a
// host-side stand-in for the symbol, never a device address: the device
// address comes from hipGetSymbolAddress, taken once per device.
__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on first use per device).
dflash_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return dflash::set_error(DFLASH_EHIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return dflash::set_error(DFLASH_EUNSUPPORTED, "device index outside the scratch table");
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return dflash::set_error(DFLASH_EHIP, e != hipSuccess ? hipGetErrorString(e)
                                                             : "scratch symbol has no address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DFLASH_OK;
}

}  // namespace

extern "C" {

size_t dflash_draft_block_noalloc_limit(void) { return kScratchBytes; }

dflash_status dflash_draft_block_noalloc(const dflash_config* cfg, const dflash_weights* w,
                                         const dflash_kv_cache* cache, const int32_t* anchor,
                                         const int32_t* prefix_len, const int32_t* page_table,
                                         int32_t max_pages, int32_t batch, int32_t max_prefix_len,
                                         int32_t* block_ids, int32_t* positions, int32_t* slots,
                                         int32_t* candidates, void* logits, void* stream) {
  if (batch == 0) return DFLASH_OK;
  // the size check needs no device: a call too large is refused before any
  // HIP call is made
  const size_t need = dflash_draft_workspace_bytes(cfg, batch, max_prefix_len);
  if (need == 0)
    return dflash::set_error(DFLASH_EINVAL, "invalid config, batch or max_prefix_len");
  if (need > kScratchBytes) {
    char msg[160];
    snprintf(msg, sizeof msg, "the call needs %zu bytes of scratch; the fixed scratch holds %zu",
             need, kScratchBytes);
    return dflash::set_error(DFLASH_EWORKSPACE, msg);
  }
  void* ws = nullptr;
  const dflash_status s = scratch_on_current_device(&ws);
  if (s != DFLASH_OK) return s;
  return dflash_draft_block(cfg, w, cache, anchor, prefix_len, page_table, max_pages, batch,
                            max_prefix_len, block_ids, positions, slots, candidates, logits, ws,
                            kScratchBytes, stream);
}

}  // extern "C"
