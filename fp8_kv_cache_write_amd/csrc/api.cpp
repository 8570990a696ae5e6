// api.cpp - the C ABI of include/kvfp8.h: argument checks (host only, before
// any launch), the split-context partition plan, and the launches.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/kvfp8.h"
#include "launch.hpp"

using namespace kvfp8;

namespace {

// kvq_set_tuning overrides, -1 = the plan decides.
constexpr int kTuningKnobs = 5;
std::atomic<int> g_tuning[kTuningKnobs] = {{-1}, {-1}, {-1}, {-1}, {-1}};

}  // namespace

namespace kvfp8 {
int tuning_override(int knob) {
  return knob >= 0 && knob < kTuningKnobs ? g_tuning[knob].load(std::memory_order_relaxed) : -1;
}
}  // namespace kvfp8

namespace {

constexpr int kMaxGroup = 16;       // bf16-MFMA attention (P carried as hi + lo)
constexpr int kMaxGroupFp8 = 16;    // all-FP8 attention
constexpr int kMaxPagesPerWave = 64;
constexpr int kMaxDynHeads = 256;   // dynamic scales: LDS per-head maxima of the write

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_desc(const kvq_layer_desc* d) {
  if (!d) return KVQ_ERR_INVALID_ARG;
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0) return KVQ_ERR_INVALID_ARG;
  if (d->cache_dtype != KVQ_BF16 && d->cache_dtype != KVQ_FP8_E4M3 &&
      d->cache_dtype != KVQ_FP8_E5M2)
    return KVQ_ERR_INVALID_ARG;
  if (d->scale_mode != KVQ_SCALE_PER_TENSOR && d->scale_mode != KVQ_SCALE_PER_KV_HEAD &&
      d->scale_mode != KVQ_SCALE_PER_TOKEN && d->scale_mode != KVQ_SCALE_PER_TOKEN_HEAD)
    return KVQ_ERR_INVALID_ARG;
  if (d->sliding_window < 0) return KVQ_ERR_INVALID_ARG;
  if (!(d->sm_scale >= 0.0f) || !isfinite(d->sm_scale)) return KVQ_ERR_INVALID_ARG;
  if (d->page_size != 16) return KVQ_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) return KVQ_ERR_UNSUPPORTED;
  if (d->num_q_heads % d->num_kv_heads != 0) return KVQ_ERR_UNSUPPORTED;
  if (d->attn_dtype != KVQ_ATTN_BF16 && d->attn_dtype != KVQ_ATTN_FP8) return KVQ_ERR_INVALID_ARG;
  if (d->attn_dtype == KVQ_ATTN_FP8 && d->cache_dtype == KVQ_BF16) return KVQ_ERR_UNSUPPORTED;
  if (d->num_q_heads / d->num_kv_heads >
      (d->attn_dtype == KVQ_ATTN_FP8 ? kMaxGroupFp8 : kMaxGroup))
    return KVQ_ERR_UNSUPPORTED;
  if (d->num_kv_heads > 65535) return KVQ_ERR_UNSUPPORTED;
  if (d->cache_dtype != KVQ_BF16 && d->scale_mode >= KVQ_SCALE_PER_TOKEN) {
    if (d->attn_dtype == KVQ_ATTN_FP8) return KVQ_ERR_UNSUPPORTED;
    if (d->num_kv_heads > kMaxDynHeads) return KVQ_ERR_UNSUPPORTED;
  }
  return KVQ_OK;
}

// An fp8 layer whose scales are per token (computed at write time, stored in
// pools beside the pages).
bool dynamic_scales(const kvq_layer_desc* d) {
  return d->cache_dtype != KVQ_BF16 && d->scale_mode >= KVQ_SCALE_PER_TOKEN;
}

// Compute units of the current device, queried once per device.
int cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

struct Plan {
  int pages_per_wave;
  int num_parts;
  int slots;                   // split-kernel shape: LDS-staged tiles (1) or registers (0)
  int tile_pages;              // pages per tile: 2, or 4 (see make_plan)
  int rotate;                  // partition order rotated per (sequence, KV head)
  size_t off_l, off_o, bytes;  // workspace layout (bytes)
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Split-context plan. Pages of one (sequence, KV head) are cut into
// partitions of kSplitWaves * pages_per_wave pages; each partition is one
// work-group of kSplitWaves waves, each wave streams pages_per_wave pages.
//
// Measured on MI355X: the kernel is fastest when every compute unit gets the
// same number of work-groups and each wave streams a long run. The plan
// tries k = 1..4 work-groups per compute unit: for each, the shortest even
// run (<= 64 pages) that fits the longest sequence into k * CUs work-groups,
// costed as k * run (pages each CU streams) with a small penalty per extra
// co-resident work-group (measured: two work-groups of 32 pages per CU take
// ~3.5 % longer than one of 64). One work-group per CU (one wave per SIMD)
// uses the LDS-staged tile shape up to head_dim 128, so a wave keeps its next
// tile in flight while it computes; more, and head_dim 256, use the register
// shape. When one partition per
// sequence is cheap enough (short contexts, sliding windows) the split kernel
// writes the output itself and the reduce kernel is skipped.
//
// Partition order: work-groups reach the 8 XCDs round-robin in launch order,
// so partition x of every (sequence, KV head) runs on XCD x mod 8 unless the
// kernel rotates the partition index by the unit index. In a batch of
// unequal lengths the short or empty last partitions then pile onto one XCD;
// rotated, they spread (8 sequences of 18k-22k positions: 2-3 % faster).
// With one sequence, A/B runs on MI355X found the rotation 2-3 % faster for
// 64-page runs (the 8B layer at 131072 positions), neutral for the 70B
// layer, and 4-5 % slower for short runs (8k-16k positions, head_dim 256
// at 65536), so it is used for batches and for 64-page runs.
constexpr double kCoResidentPenalty = 0.035;

Plan make_plan(const kvq_layer_desc* d, int num_seqs, int max_context_len) {
  const int W = d->sliding_window;
  const bool att8 = d->attn_dtype == KVQ_ATTN_FP8;
  int64_t pages_max = ((int64_t)max_context_len + 15) / 16;
  // a window's first page; the all-FP8 mode starts on an even page (tiles on
  // aligned 32-position blocks), one more
  if (W > 0) pages_max = std::min<int64_t>(pages_max, ((int64_t)W + 15) / 16 + 1 + (att8 ? 1 : 0));
  if (pages_max < 1) pages_max = 1;
  const int64_t units = (int64_t)std::max(num_seqs, 1) * d->num_kv_heads;
  const int64_t cus = cu_count();
  auto even_run = [](int64_t n) { return std::max<int64_t>((n + 1) / 2 * 2, 2); };
  int64_t ppw = 0;
  int k_best = 0;
  double best = 0.0;
  for (int k = 1; k <= 4; ++k) {
    const int64_t parts_cap = k * cus / units;
    if (parts_cap < 1) continue;
    const int64_t run =
        even_run((pages_max + kSplitWaves * parts_cap - 1) / (kSplitWaves * parts_cap));
    if (run > kMaxPagesPerWave) continue;
    const double cost = (double)k * (double)run * (1.0 + kCoResidentPenalty * (k - 1));
    if (k_best == 0 || cost < best) {
      best = cost;
      ppw = run;
      k_best = k;
    }
  }
  if (k_best == 0)   // many sequences, or very long ones: full-length runs
    ppw = std::min<int64_t>(even_run((pages_max + kSplitWaves - 1) / kSplitWaves),
                            kMaxPagesPerWave);
  const int64_t page_block = 16LL * d->head_dim * (d->cache_dtype == KVQ_BF16 ? 2 : 1);
  // a staged tile: K and V of two pages, with dynamic scales their 2 x 16 fp32 each
  const int64_t tile_bytes = 2 * 2 * page_block + (dynamic_scales(d) ? 2 * 2 * 16 * 4 : 0);
  const bool ring_fits = kSplitWaves * tile_bytes <= 64 * 1024;
  // At head_dim 256 a 2-page tile is 16 KiB per wave: the staged ring fills
  // the whole 64 KiB and a wave's tile occupies 64 VGPRs either way; the
  // register shape measured faster there (fp8, 8 q / 2 KV heads, one
  // sequence: 8192 positions 10.55 -> 10.29 us, 32768 13.70 -> 13.14,
  // 65536 19.07 -> 19.03, 131072 29.74 -> 29.37 per layer step).
  int slots = (k_best == 1 && ring_fits && d->head_dim <= 128) ? 1 : 0;
  int64_t direct_ppw = (pages_max + kSplitWaves - 1) / kSplitWaves;
  direct_ppw = (direct_ppw + 1) / 2 * 2;
  if (direct_ppw <= std::max<int64_t>(ppw, 8)) {
    ppw = direct_ppw;
    slots = 0;
  }
  // an explicit override of the run length (kvq_set_tuning, sweeps and tests)
  if (const int n = tuning_override(KVQ_TUNE_PAGES_PER_WAVE); n >= 1) ppw = n;
  if (att8) ppw = (ppw + 1) / 2 * 2;   // runs of whole 32-position blocks
  Plan p;
  p.pages_per_wave = (int)ppw;
  p.slots = slots;
  // Tiles of 4 pages for fp8 caches at head_dim 64 (1 KiB per page and
  // tensor) in the bf16-arithmetic mode with static scales, LDS-staged: the
  // per-tile softmax and merge work then covers twice the bytes. Measured on
  // MI355X (gpt-oss-like layer, 64 q / 8 KV heads): 131072 positions
  // 33.9 -> 26.6 us, 32768 13.5 -> 12.7 us, 8192 unchanged; at head_dim 128
  // 4-page tiles measured slower. Runs are whole 4-page tiles. The other
  // modes are built for 2-page tiles.
  const bool g_le_8 = d->num_q_heads / d->num_kv_heads <= 8;
  p.tile_pages = (slots == 1 && ppw % 4 == 0 && d->head_dim == 64 &&
                  d->cache_dtype != KVQ_BF16 && !att8 && !dynamic_scales(d) && g_le_8)
                     ? 4
                     : 2;
  p.rotate = (num_seqs > 1 || ppw >= kMaxPagesPerWave) ? 1 : 0;
  // an explicit override of the partition order (kvq_set_tuning)
  if (const int r = tuning_override(KVQ_TUNE_PARTITION_ROTATE); r >= 0) p.rotate = r;
  p.num_parts = (int)((pages_max + kSplitWaves * ppw - 1) / (kSplitWaves * ppw));
  if (p.num_parts <= 1) {
    p.num_parts = 1;
    p.off_l = p.off_o = p.bytes = 0;
    return p;
  }
  // Slots: (m, l, o[D]) per (sequence, query head, partition). The reduce
  // kernel reads whole chunks of up to kReduceChunk partitions and weights
  // the slots past a row's partitions with 0, so the o region ends with a
  // chunk of slack that keeps those reads inside the workspace (the m and l
  // regions are followed by the next region).
  const size_t rows = (size_t)num_seqs * d->num_q_heads * p.num_parts;
  p.off_l = round_up(rows * sizeof(float), 256);
  p.off_o = p.off_l + round_up(rows * sizeof(float), 256);
  p.bytes = p.off_o + round_up((rows + kReduceChunk) * d->head_dim * sizeof(float), 256);
  return p;
}

// Profiling hook (see kvq_profile_begin).
struct Profiler {
  bool on = false;
  int max = 0;
  std::vector<hipEvent_t> ev;
  int used = 0;
} g_prof;

}  // namespace

extern "C" {

const char* kvq_status_string(int32_t status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KVQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int kvq_kv_cache_write(const kvq_layer_desc* desc, const void* k, const void* v,
                       const int64_t* slot_mapping, int64_t num_tokens, void* k_cache,
                       void* v_cache, int64_t num_pages, const float* k_scale,
                       const float* v_scale, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if (num_tokens < 0 || num_pages < 0) return KVQ_ERR_INVALID_ARG;
  if (num_tokens == 0) return KVQ_OK;
  if (num_pages == 0) return KVQ_ERR_INVALID_ARG;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return KVQ_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8))
    return KVQ_ERR_INVALID_ARG;
  const bool fp8 = desc->cache_dtype != KVQ_BF16;
  if (dynamic_scales(desc)) return KVQ_ERR_INVALID_ARG;   // kvq_kv_cache_write_dynamic
  if (fp8 && (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4)))
    return KVQ_ERR_INVALID_ARG;
  const int64_t threads = num_tokens * desc->num_kv_heads * (desc->head_dim / 16);
  if ((threads + 255) / 256 > 0x7FFFFFFFLL) return KVQ_ERR_UNSUPPORTED;
  hipError_t e = launch_kv_cache_write(
      (int)desc->cache_dtype, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), slot_mapping,
      num_tokens, desc->num_kv_heads, desc->head_dim, static_cast<uint8_t*>(k_cache),
      static_cast<uint8_t*>(v_cache), num_pages, k_scale, v_scale,
      desc->scale_mode == KVQ_SCALE_PER_KV_HEAD ? 1 : 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

int kvq_kv_cache_write_dynamic(const kvq_layer_desc* desc, const void* k, const void* v,
                               const int64_t* slot_mapping, int64_t num_tokens, void* k_cache,
                               void* v_cache, int64_t num_pages, float* k_scales,
                               float* v_scales, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if (desc->cache_dtype != KVQ_BF16 && !dynamic_scales(desc)) return KVQ_ERR_INVALID_ARG;
  if (desc->cache_dtype == KVQ_BF16)     // bf16 layers copy; no scales
    return kvq_kv_cache_write(desc, k, v, slot_mapping, num_tokens, k_cache, v_cache,
                              num_pages, nullptr, nullptr, stream);
  if (num_tokens < 0 || num_pages < 0) return KVQ_ERR_INVALID_ARG;
  if (num_tokens == 0) return KVQ_OK;
  if (num_pages == 0) return KVQ_ERR_INVALID_ARG;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache || !k_scales || !v_scales)
    return KVQ_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8) || !aligned(k_scales, 16) || !aligned(v_scales, 16))
    return KVQ_ERR_INVALID_ARG;
  if (num_tokens > 0x7FFFFFFFLL) return KVQ_ERR_UNSUPPORTED;
  hipError_t e = launch_kv_cache_write_dyn(
      (int)desc->cache_dtype, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      slot_mapping, num_tokens, desc->num_kv_heads, desc->head_dim,
      static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), num_pages, k_scales,
      v_scales, desc->scale_mode == KVQ_SCALE_PER_TOKEN ? 1 : 0,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

int kvq_decode_workspace_bytes(const kvq_layer_desc* desc, int32_t num_seqs,
                               int32_t max_context_len, size_t* bytes) {
  int st = check_desc(desc);
  if (st) return st;
  if (!bytes || num_seqs < 0 || max_context_len < 0) return KVQ_ERR_INVALID_ARG;
  *bytes = make_plan(desc, num_seqs, max_context_len).bytes;
  return KVQ_OK;
}

namespace {

// Shared by the attention call and the fused decode step: host checks, the
// plan, the launch.
int decode_common(const kvq_layer_desc* desc, void* out, int32_t out_dtype, const void* q,
                  const void* k_cache, const void* v_cache, int64_t num_pages,
                  const int32_t* block_tables, int32_t max_pages_per_seq,
                  const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                  const float* k_scale, const float* v_scale, void* workspace,
                  size_t workspace_bytes, const void* k_new, const void* v_new, bool fused,
                  void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if (out_dtype != KVQ_OUT_F32 && out_dtype != KVQ_OUT_BF16) return KVQ_ERR_INVALID_ARG;
  if (num_seqs < 0 || max_context_len < 0 || num_pages < 0 || max_pages_per_seq < 0)
    return KVQ_ERR_INVALID_ARG;
  if (num_seqs == 0) return KVQ_OK;
  if (num_seqs > 65535) return KVQ_ERR_UNSUPPORTED;
  if (((int64_t)max_context_len + 15) / 16 > max_pages_per_seq) return KVQ_ERR_INVALID_ARG;
  if (max_context_len > 0 && num_pages == 0) return KVQ_ERR_INVALID_ARG;
  if (!out || !q || !context_lens || !aligned(out, 16) || !aligned(q, 16) ||
      !aligned(context_lens, 4))
    return KVQ_ERR_INVALID_ARG;
  if (max_pages_per_seq > 0 && (!block_tables || !aligned(block_tables, 4)))
    return KVQ_ERR_INVALID_ARG;
  if ((max_context_len > 0 || fused) &&
      (!k_cache || !v_cache || !aligned(k_cache, 16) || !aligned(v_cache, 16)))
    return KVQ_ERR_INVALID_ARG;
  if (fused && (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16)))
    return KVQ_ERR_INVALID_ARG;
  const bool fp8 = desc->cache_dtype != KVQ_BF16;
  const bool dyn = dynamic_scales(desc);
  if (fp8 && (!k_scale || !v_scale || !aligned(k_scale, dyn ? 16 : 4) ||
              !aligned(v_scale, dyn ? 16 : 4)))
    return KVQ_ERR_INVALID_ARG;
  const Plan plan = make_plan(desc, num_seqs, max_context_len);
  if (plan.bytes > 0) {
    if (workspace_bytes < plan.bytes) return KVQ_ERR_WORKSPACE_TOO_SMALL;
    if (!workspace || !aligned(workspace, 256)) return KVQ_ERR_INVALID_ARG;
  }
  DecodeParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k_cache = static_cast<const uint8_t*>(k_cache);
  p.v_cache = static_cast<const uint8_t*>(v_cache);
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.num_pages = num_pages;
  p.k_scale = fp8 ? k_scale : nullptr;
  p.v_scale = fp8 ? v_scale : nullptr;
  char* ws = static_cast<char*>(workspace);
  p.ws_m = plan.bytes ? reinterpret_cast<float*>(ws) : nullptr;
  p.ws_l = plan.bytes ? reinterpret_cast<float*>(ws + plan.off_l) : nullptr;
  p.ws_o = plan.bytes ? reinterpret_cast<float*>(ws + plan.off_o) : nullptr;
  p.out = out;
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.num_q_heads = desc->num_q_heads;
  p.num_kv_heads = desc->num_kv_heads;
  p.group = desc->num_q_heads / desc->num_kv_heads;
  p.max_pages_per_seq = max_pages_per_seq;
  p.window = desc->sliding_window;
  p.pages_per_wave = plan.pages_per_wave;
  p.num_parts = plan.num_parts;
  p.scale_per_head = desc->scale_mode == KVQ_SCALE_PER_KV_HEAD ? 1 : 0;
  p.dyn_all_heads = desc->scale_mode == KVQ_SCALE_PER_TOKEN ? 1 : 0;
  p.out_bf16 = out_dtype == KVQ_OUT_BF16 ? 1 : 0;
  p.direct = plan.num_parts == 1 ? 1 : 0;
  p.rotate = plan.rotate;
  const float sm = desc->sm_scale > 0.0f ? desc->sm_scale
                                         : 1.0f / sqrtf((float)desc->head_dim);
  p.sm_scale_log2 = sm * 1.4426950408889634f;

  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (g_prof.on && g_prof.used < g_prof.max) {
    e0 = g_prof.ev[2 * g_prof.used];
    e1 = g_prof.ev[2 * g_prof.used + 1];
    g_prof.used++;
  }
  hipError_t e = launch_paged_decode(p, desc->head_dim, (int)desc->cache_dtype, num_seqs, fused,
                                     plan.slots, plan.tile_pages,
                                     desc->attn_dtype == KVQ_ATTN_FP8, dyn,
                                     static_cast<hipStream_t>(stream), e0, e1);
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace

int kvq_paged_decode_attention(const kvq_layer_desc* desc, void* out, int32_t out_dtype,
                               const void* q, const void* k_cache, const void* v_cache,
                               int64_t num_pages, const int32_t* block_tables,
                               int32_t max_pages_per_seq, const int32_t* context_lens,
                               int32_t num_seqs, int32_t max_context_len,
                               const float* k_scale, const float* v_scale, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return decode_common(desc, out, out_dtype, q, k_cache, v_cache, num_pages, block_tables,
                       max_pages_per_seq, context_lens, num_seqs, max_context_len, k_scale,
                       v_scale, workspace, workspace_bytes, nullptr, nullptr, false, stream);
}

int kvq_decode_step(const kvq_layer_desc* desc, const void* k_new, const void* v_new,
                    void* k_cache, void* v_cache, int64_t num_pages, void* out,
                    int32_t out_dtype, const void* q, const int32_t* block_tables,
                    int32_t max_pages_per_seq, const int32_t* context_lens, int32_t num_seqs,
                    int32_t max_context_len, const float* k_scale, const float* v_scale,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (desc && dynamic_scales(desc)) return KVQ_ERR_INVALID_ARG;   // kvq_decode_step_dynamic
  return decode_common(desc, out, out_dtype, q, k_cache, v_cache, num_pages, block_tables,
                       max_pages_per_seq, context_lens, num_seqs, max_context_len, k_scale,
                       v_scale, workspace, workspace_bytes, k_new, v_new, true, stream);
}

int kvq_decode_step_dynamic(const kvq_layer_desc* desc, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, int64_t num_pages, void* out,
                            int32_t out_dtype, const void* q, const int32_t* block_tables,
                            int32_t max_pages_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_context_len, float* k_scales,
                            float* v_scales, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (desc && desc->cache_dtype != KVQ_BF16 && !dynamic_scales(desc)) return KVQ_ERR_INVALID_ARG;
  return decode_common(desc, out, out_dtype, q, k_cache, v_cache, num_pages, block_tables,
                       max_pages_per_seq, context_lens, num_seqs, max_context_len, k_scales,
                       v_scales, workspace, workspace_bytes, k_new, v_new, true, stream);
}

static PrefillPlan prefill_plan(const kvq_layer_desc* d, int32_t num_seqs,
                                int32_t max_query_len, int32_t max_pages_per_seq,
                                bool allow_split) {
  return plan_paged_prefill(d->head_dim, (int)d->cache_dtype, d->num_q_heads, d->num_kv_heads,
                            num_seqs, max_query_len, max_pages_per_seq, cu_count(),
                            allow_split);
}

int kvq_prefill_workspace_bytes(const kvq_layer_desc* desc, int32_t num_seqs,
                                int32_t max_query_len, int32_t max_pages_per_seq,
                                size_t* bytes) {
  int st = check_desc(desc);
  if (st) return st;
  if (!bytes || num_seqs < 0 || max_query_len < 0 || max_pages_per_seq < 0)
    return KVQ_ERR_INVALID_ARG;
  *bytes = 0;
  if (num_seqs == 0 || max_query_len == 0 || max_pages_per_seq == 0) return KVQ_OK;
  *bytes = prefill_plan(desc, num_seqs, max_query_len, max_pages_per_seq, true).bytes;
  return KVQ_OK;
}

int kvq_paged_prefill_attention(const kvq_layer_desc* desc, void* out, int32_t out_dtype,
                                const void* q, const void* k_cache, const void* v_cache,
                                int64_t num_pages, const int32_t* block_tables,
                                int32_t max_pages_per_seq, const int32_t* query_start,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t max_query_len, const float* k_scale,
                                const float* v_scale, void* workspace, size_t workspace_bytes,
                                void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  const bool dyn = dynamic_scales(desc);
  const bool att8 = desc->attn_dtype == KVQ_ATTN_FP8;   // fp8 caches only (check_desc)
  if (out_dtype != KVQ_OUT_F32 && out_dtype != KVQ_OUT_BF16) return KVQ_ERR_INVALID_ARG;
  if (num_seqs < 0 || max_query_len < 0 || num_pages < 0 || max_pages_per_seq < 0)
    return KVQ_ERR_INVALID_ARG;
  if (!workspace && workspace_bytes != 0) return KVQ_ERR_INVALID_ARG;
  if (workspace && !aligned(workspace, 256)) return KVQ_ERR_INVALID_ARG;
  if (num_seqs == 0 || max_query_len == 0) return KVQ_OK;
  if (num_pages == 0 || max_pages_per_seq == 0) return KVQ_ERR_INVALID_ARG;
  // no workspace: no key split; a workspace must hold the split's partials
  const PrefillPlan plan =
      prefill_plan(desc, num_seqs, max_query_len, max_pages_per_seq, workspace != nullptr);
  if (workspace_bytes < plan.bytes) return KVQ_ERR_WORKSPACE_TOO_SMALL;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !query_start || !context_lens)
    return KVQ_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(query_start, 4) || !aligned(context_lens, 4))
    return KVQ_ERR_INVALID_ARG;
  const bool fp8 = desc->cache_dtype != KVQ_BF16;
  if (fp8 && (!k_scale || !v_scale || !aligned(k_scale, dyn ? 16 : 4) ||
              !aligned(v_scale, dyn ? 16 : 4)))
    return KVQ_ERR_INVALID_ARG;
  PrefillParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k_cache = static_cast<const uint8_t*>(k_cache);
  p.v_cache = static_cast<const uint8_t*>(v_cache);
  p.block_tables = block_tables;
  p.query_start = query_start;
  p.context_lens = context_lens;
  p.num_pages = num_pages;
  p.k_scale = fp8 ? k_scale : nullptr;
  p.v_scale = fp8 ? v_scale : nullptr;
  p.out = out;
  p.num_seqs = num_seqs;
  p.num_q_heads = desc->num_q_heads;
  p.num_kv_heads = desc->num_kv_heads;
  p.group = desc->num_q_heads / desc->num_kv_heads;
  p.max_pages_per_seq = max_pages_per_seq;
  p.max_query_len = max_query_len;
  p.window = desc->sliding_window;
  p.scale_per_head = desc->scale_mode == KVQ_SCALE_PER_KV_HEAD ? 1 : 0;
  p.out_bf16 = out_dtype == KVQ_OUT_BF16 ? 1 : 0;
  const float sm = desc->sm_scale > 0.0f ? desc->sm_scale
                                         : 1.0f / sqrtf((float)desc->head_dim);
  p.sm_scale_log2 = sm * 1.4426950408889634f;
  if (plan.bytes) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    p.ws_m = reinterpret_cast<float*>(ws);
    p.ws_l = reinterpret_cast<float*>(ws + plan.off_l);
    p.ws_o = reinterpret_cast<float*>(ws + plan.off_o);
  }
  hipError_t e = launch_paged_prefill(p, plan, desc->head_dim, (int)desc->cache_dtype, dyn,
                                      att8, static_cast<hipStream_t>(stream), nullptr, nullptr);
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

int kvq_kv_scale_from_amax(const kvq_layer_desc* desc, const void* x, int64_t num_tokens,
                           float* scale_out, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if (num_tokens < 0 || !x || !scale_out || !aligned(x, 16) || !aligned(scale_out, 4))
    return KVQ_ERR_INVALID_ARG;
  if (desc->scale_mode >= KVQ_SCALE_PER_TOKEN) return KVQ_ERR_INVALID_ARG;   // set by the write
  const float fmax = desc->cache_dtype == KVQ_FP8_E5M2 ? 57344.0f : 448.0f;
  hipError_t e = launch_scale_from_amax(
      static_cast<const uint16_t*>(x), num_tokens, desc->num_kv_heads, desc->head_dim,
      desc->scale_mode == KVQ_SCALE_PER_KV_HEAD ? 1 : 0, fmax, scale_out,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

namespace {
int quantize_common(int fmt, const float* x, int64_t n, const float* scale, uint8_t* out,
                    void* stream) {
  if (n < 0) return KVQ_ERR_INVALID_ARG;
  if (n == 0) return KVQ_OK;
  if (!x || !scale || !out || !aligned(x, 16) || !aligned(out, 4) || !aligned(scale, 4))
    return KVQ_ERR_INVALID_ARG;
  hipError_t e = launch_quantize(fmt, x, n, scale, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}
}  // namespace

int kvq_e4m3_quantize(const float* x, int64_t n, const float* scale, uint8_t* out,
                      void* stream) {
  return quantize_common(KVQ_FP8_E4M3, x, n, scale, out, stream);
}

int kvq_e5m2_quantize(const float* x, int64_t n, const float* scale, uint8_t* out,
                      void* stream) {
  return quantize_common(KVQ_FP8_E5M2, x, n, scale, out, stream);
}

int kvq_stream_read(const void* src, int64_t n_bytes, uint32_t* sink, int32_t num_blocks,
                    void* stream) {
  if (n_bytes < 0 || n_bytes % 16 != 0 || num_blocks <= 0) return KVQ_ERR_INVALID_ARG;
  if (n_bytes == 0) return KVQ_OK;
  if (!src || !sink || !aligned(src, 16) || !aligned(sink, 4)) return KVQ_ERR_INVALID_ARG;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (g_prof.on && g_prof.used < g_prof.max) {
    e0 = g_prof.ev[2 * g_prof.used];
    e1 = g_prof.ev[2 * g_prof.used + 1];
    g_prof.used++;
  }
  return launch_stream_read(src, n_bytes, sink, num_blocks, static_cast<hipStream_t>(stream), e0,
                            e1) == hipSuccess
             ? KVQ_OK
             : KVQ_ERR_HIP;
}

int kvq_set_tuning(int32_t knob, int32_t value) {
  if (knob < 0 || knob >= kTuningKnobs) return KVQ_ERR_INVALID_ARG;
  bool ok = value == -1;
  switch (knob) {
    case KVQ_TUNE_PAGES_PER_WAVE: ok |= value >= 1 && value <= kMaxPagesPerWave; break;
    case KVQ_TUNE_PARTITION_ROTATE: ok |= value == 0 || value == 1; break;
    case KVQ_TUNE_SPLIT_SHAPE:
      ok |= value == 210 || value == 220 || value == 410 || value == 211 || value == 212 ||
            value == 411;
      break;
    case KVQ_TUNE_PREFILL_COLUMN_GROUPS: ok |= value >= 1 && value <= 3; break;
    case KVQ_TUNE_PREFILL_KEY_PARTS: ok |= value >= 1; break;
  }
  if (!ok) return KVQ_ERR_INVALID_ARG;
  g_tuning[knob].store(value, std::memory_order_relaxed);
  return KVQ_OK;
}

int kvq_profile_begin(int32_t max_launches) {
  if (max_launches <= 0) return KVQ_ERR_INVALID_ARG;
  if ((int)g_prof.ev.size() < 2 * max_launches) {
    while ((int)g_prof.ev.size() < 2 * max_launches) {
      hipEvent_t ev;
      if (hipEventCreate(&ev) != hipSuccess) return KVQ_ERR_HIP;
      g_prof.ev.push_back(ev);
    }
  }
  g_prof.max = max_launches;
  g_prof.used = 0;
  g_prof.on = true;
  return KVQ_OK;
}

int kvq_profile_end(double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return KVQ_ERR_INVALID_ARG;
  g_prof.on = false;
  double sum = 0.0;
  for (int i = 0; i < g_prof.used; ++i) {
    if (hipEventSynchronize(g_prof.ev[2 * i + 1]) != hipSuccess) return KVQ_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]) != hipSuccess)
      return KVQ_ERR_HIP;
    sum += ms;
  }
  *total_ms = sum;
  *launches = g_prof.used;
  g_prof.used = 0;
  return KVQ_OK;
}

}  // extern "C"
