// decode_noalloc.hip - kvq_paged_decode_attention_noalloc: the decode
// attention for callers that cannot allocate device memory. Its split
// workspace is the file-scope device array `scratch` below, one copy per
// device, which the library owns until the process ends.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/kvfp8.h"

namespace {

constexpr size_t kScratchBytes = KVQ_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "the workspace sections are 256-byte aligned");

// The split workspace of the no-allocation entry point. In host code this
// name is only a stand-in for the symbol: the device address of each
// device's copy comes from hipGetSymbolAddress (scratch_on_current_device)
// and is the only form ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch`, per device

// The device address of the current device's copy of `scratch`, looked up
// once per device with that device current (the lookup allocates nothing).
int scratch_on_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KVQ_ERR_HIP;
  if (dev >= kMaxDevices) return KVQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return KVQ_OK;
}

}  // namespace

extern "C" int kvq_paged_decode_attention_noalloc(
    const kvq_layer_desc* desc, void* out, int32_t out_dtype, const void* q,
    const void* k_cache, const void* v_cache, int64_t num_pages, const int32_t* block_tables,
    int32_t max_pages_per_seq, const int32_t* context_lens, int32_t num_seqs,
    int32_t max_context_len, const float* k_scale, const float* v_scale, void* stream) {
  // the plan's workspace must fit the array; checked before any device call
  size_t need = 0;
  int st = kvq_decode_workspace_bytes(desc, num_seqs < 0 ? 0 : num_seqs,
                                      max_context_len < 0 ? 0 : max_context_len, &need);
  if (st) return st;
  if (need > kScratchBytes) return KVQ_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (need > 0 && num_seqs > 0) {
    st = scratch_on_current_device(&ws);
    if (st) return st;
  }
  // The split kernel writes every partial slot the reduce kernel weights
  // (empty partitions get m = -inf, l = 0), and slots past a row's
  // partitions get weight 0, so the array needs no clearing between calls.
  return kvq_paged_decode_attention(desc, out, out_dtype, q, k_cache, v_cache, num_pages,
                                    block_tables, max_pages_per_seq, context_lens, num_seqs,
                                    max_context_len, k_scale, v_scale, ws,
                                    ws ? kScratchBytes : 0, stream);
}
