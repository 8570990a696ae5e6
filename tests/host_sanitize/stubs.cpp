// stubs.cpp - the device side of libkvfp8 replaced by recorders, so that the
// host code of the C ABI (api.cpp, prefill_plan.cpp) runs under
// AddressSanitizer and UndefinedBehaviorSanitizer with no GPU: the HIP
// runtime calls it makes report one device of 256 compute units, and every
// kernel launch records its arguments for the driver to check.
// Test infrastructure; never part of the library.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <string.h>

#include "../../fp8_kv_cache_write_amd/csrc/launch.hpp"
#include "stubs.hpp"

LaunchLog g_log;

extern "C" {
hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int device) {
  *value = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
  return device == 0 ? hipSuccess : hipErrorInvalidDevice;
}
hipError_t hipEventCreate(hipEvent_t* event) {
  static int tokens[4096];
  static int next = 0;
  *event = reinterpret_cast<hipEvent_t>(&tokens[next++ % 4096]);
  return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 1.0f;
  return hipSuccess;
}
}

namespace kvfp8 {

hipError_t launch_kv_cache_write(int fmt, const uint16_t*, const uint16_t*, const int64_t*,
                                 int64_t num_tokens, int num_kv_heads, int head_dim, uint8_t*,
                                 uint8_t*, int64_t num_pages, const float*, const float*,
                                 int scale_per_head, hipStream_t) {
  g_log.writes++;
  g_log.last_fmt = fmt;
  g_log.last_tokens = num_tokens;
  g_log.last_heads = num_kv_heads;
  g_log.last_head_dim = head_dim;
  g_log.last_pages = num_pages;
  g_log.last_per_head = scale_per_head;
  return hipSuccess;
}

hipError_t launch_kv_cache_write_dyn(int fmt, const uint16_t*, const uint16_t*, const int64_t*,
                                     int64_t num_tokens, int, int, uint8_t*, uint8_t*, int64_t,
                                     float*, float*, int all_heads, hipStream_t) {
  g_log.dyn_writes++;
  g_log.last_fmt = fmt;
  g_log.last_tokens = num_tokens;
  g_log.last_per_head = all_heads;
  return hipSuccess;
}

hipError_t launch_scale_from_amax(const uint16_t*, int64_t, int, int, int per_head, float fmax,
                                  float*, hipStream_t) {
  g_log.scales++;
  g_log.last_per_head = per_head;
  g_log.last_fmax = fmax;
  return hipSuccess;
}

hipError_t launch_quantize(int fmt, const float*, int64_t n, const float*, uint8_t*, hipStream_t) {
  g_log.quantizes++;
  g_log.last_fmt = fmt;
  g_log.last_tokens = n;
  return hipSuccess;
}

hipError_t launch_stream_read(const void*, int64_t n_bytes, uint32_t*, int, hipStream_t,
                              hipEvent_t, hipEvent_t) {
  g_log.reads++;
  g_log.last_tokens = n_bytes;
  return hipSuccess;
}

hipError_t launch_paged_decode(const DecodeParams& p, int head_dim, int fmt, int num_seqs,
                               bool fused, int slots, int tile_pages, bool att8, bool dyn,
                               hipStream_t, hipEvent_t, hipEvent_t) {
  g_log.decodes++;
  g_log.decode = p;
  g_log.last_head_dim = head_dim;
  g_log.last_fmt = fmt;
  g_log.last_seqs = num_seqs;
  g_log.fused = fused;
  g_log.slots = slots;
  g_log.tile_pages = tile_pages;
  g_log.att8 = att8;
  g_log.dyn = dyn;
  return hipSuccess;
}

hipError_t launch_paged_prefill(const PrefillParams& p, const PrefillPlan& plan, int head_dim,
                                int fmt, bool dyn, bool att8, hipStream_t, hipEvent_t,
                                hipEvent_t) {
  g_log.prefills++;
  g_log.prefill = p;
  g_log.prefill_plan = plan;
  g_log.last_head_dim = head_dim;
  g_log.last_fmt = fmt;
  g_log.dyn = dyn;
  g_log.att8 = att8;
  return hipSuccess;
}

hipError_t launch_partition_merge(const DecodeParams&, int, int, hipStream_t) {
  return hipSuccess;
}

}  // namespace kvfp8
