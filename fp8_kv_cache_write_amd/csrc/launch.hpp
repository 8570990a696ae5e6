// launch.hpp - internal interface between the C ABI (api.cpp) and the
// kernels. Not installed; the public interface is include/kvfp8.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvfp8 {

// fmt (here and below): cache element format, 0 = bf16, 1 = e4m3, 2 = e5m2.
hipError_t launch_kv_cache_write(int fmt, const uint16_t* k, const uint16_t* v,
                                 const int64_t* slots, int64_t num_tokens,
                                 int num_kv_heads, int head_dim, uint8_t* k_cache,
                                 uint8_t* v_cache, int64_t num_pages,
                                 const float* k_scale, const float* v_scale,
                                 int scale_per_head, hipStream_t stream);

// s = fp32(amax) / fmax (448 for e4m3, 57344 for e5m2).
hipError_t launch_scale_from_amax(const uint16_t* x, int64_t num_tokens,
                                  int num_kv_heads, int head_dim, int per_head,
                                  float fmax, float* scale_out, hipStream_t stream);

hipError_t launch_quantize(int fmt, const float* x, int64_t n, const float* scale,
                           uint8_t* out, hipStream_t stream);

// A plain streaming read of n_bytes (a multiple of 16) with one XOR checksum
// word per work-group written to sink[0..num_blocks) (stream_read.hip).
hipError_t launch_stream_read(const void* src, int64_t n_bytes, uint32_t* sink,
                              int num_blocks, hipStream_t stream, hipEvent_t ev_before,
                              hipEvent_t ev_after);

// Everything the split-decode and reduce kernels read; passed by value.
struct DecodeParams {
  const uint16_t* q;             // bf16 [B][Hq][D]
  const uint8_t* k_cache;        // [P][Hkv][PB]
  const uint8_t* v_cache;
  const int32_t* block_tables;   // [B][max_pages_per_seq]
  const int32_t* context_lens;   // [B]
  int64_t num_pages;             // pool size: page ids outside [0, num_pages) read as empty
  const float* k_scale;          // [1] or [Hkv]; dynamic scales: pools [P][Hkv][16]
  const float* v_scale;          //   (written by the fused step); unused for bf16
  float* ws_m;                   // [B][Hq][num_parts]   (log2 domain)
  float* ws_l;                   // [B][Hq][num_parts]
  float* ws_o;                   // [B][Hq][num_parts][D]
  void* out;                     // [B][Hq][D] f32 or bf16
  const uint16_t* k_new;         // fused decode step only: bf16 [B][Hkv][D] of the
  const uint16_t* v_new;         //   token at position L-1 of every sequence
  int num_q_heads;
  int num_kv_heads;
  int group;                     // G = Hq / Hkv, <= 16
  int max_pages_per_seq;
  int window;                    // 0 = full
  int pages_per_wave;            // <= 64
  int num_parts;                 // partitions allocated per (b, q head)
  int scale_per_head;
  int dyn_all_heads;             // dynamic, one scale per token over all heads (fused step)
  int out_bf16;
  int direct;                    // num_parts == 1: the split kernel finishes
  int rotate;                    // split kernel: work-group x of unit u runs partition
                                 //   (x + u) mod num_parts, u = head + Hkv * sequence
  float sm_scale_log2;           // sm_scale * log2(e)
  const int32_t* row_limit;      // merge only: rows at or past *row_limit are skipped
};

// The value of a kvq_set_tuning override (enum kvq_tuning_knob of kvfp8.h),
// or -1 when the plan decides.
int tuning_override(int knob);

// Waves per work-group of the split kernel.
constexpr int kSplitWaves = 4;

// Partitions the reduce kernel reads per chunk, at most (two per lane); the
// workspaces end with this many partial slots of slack.
constexpr int kReduceChunk = 128;

// fused = true: the split kernel also writes k_new / v_new into the caches at
// position L-1 of every sequence (p.k_cache / p.v_cache must be writable).
// slots: split-kernel tile shape, 1 = LDS-staged tiles, 0 = register tiles.
// tile_pages: pages per tile, 2 (every mode) or 4 (bf16 arithmetic, static
// scales).
// fmt: cache element format, kFmtBf16 / kFmtE4M3 / kFmtE5M2 (device_common.hpp).
// att8: all-FP8 attention (e4m3 Q and P, fp8 MFMA); fp8 caches only.
// dyn: dynamic per-token scales (p.k_scale / p.v_scale are the pools); fp8
// caches, bf16 arithmetic.
hipError_t launch_paged_decode(const DecodeParams& p, int head_dim, int fmt, int num_seqs,
                               bool fused, int slots, int tile_pages, bool att8, bool dyn,
                               hipStream_t stream, hipEvent_t ev_before, hipEvent_t ev_after);

// Cache write with dynamic per-token scales: per token (all_heads = 1) or per
// token and KV head, stored for each slot into the pools [P][Hkv][16].
hipError_t launch_kv_cache_write_dyn(int fmt, const uint16_t* k, const uint16_t* v,
                                     const int64_t* slots, int64_t num_tokens, int num_kv_heads,
                                     int head_dim, uint8_t* k_cache, uint8_t* v_cache,
                                     int64_t num_pages, float* k_pool, float* v_pool,
                                     int all_heads, hipStream_t stream);

// Chunked-prefill attention: sequence b's query rows query_start[b] ..
// query_start[b+1]-1 are its last positions; each attends causally.
struct PrefillParams {
  const uint16_t* q;             // bf16 [T][Hq][D]
  const uint8_t* k_cache;        // [P][Hkv][PB]
  const uint8_t* v_cache;
  const int32_t* block_tables;   // [B][max_pages_per_seq]
  const int32_t* query_start;    // [B+1]
  const int32_t* context_lens;   // [B], the chunk included
  int64_t num_pages;
  const float* k_scale;          // [1] or [Hkv], or the pools [P][Hkv][16]; unused for bf16
  const float* v_scale;
  void* out;                     // [T][Hq][D] f32 or bf16
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;                     // G <= 16
  int max_pages_per_seq;
  int max_query_len;
  int window;                    // 0 = full
  int scale_per_head;
  int out_bf16;
  int qblocks;                   // set from the plan
  int pos_per_block;             // set from the plan
  int num_parts;                 // key partitions (1: no split; set from the plan)
  int part_tiles;                // 32-position tiles per key partition
  float* ws_m;                   // split only: [rows][Hq][num_parts] (log2 domain)
  float* ws_l;                   //   [rows][Hq][num_parts]
  float* ws_o;                   //   [rows][Hq][num_parts][D], unnormalised
  float sm_scale_log2;
};

constexpr int kPrefillWaves = 4;

// The prefill launch geometry, a pure function of its arguments (and the
// prefill overrides of kvq_set_tuning): column
// groups per wave, query blocks, and the key split with its workspace. The
// key range [0, max_pages_per_seq * 16) is cut into num_parts partitions when
// the query blocks alone would leave compute units idle (a short chunk over a
// long context) and a workspace may be used; the partitions' partial results
// are merged by the decode path's FP32 reduce kernel.
struct PrefillPlan {
  int ncg, pos_per_block, qblocks, num_parts, part_tiles;
  size_t off_l, off_o, bytes;    // workspace layout; bytes = 0 without a split
};
PrefillPlan plan_paged_prefill(int head_dim, int fmt, int num_q_heads, int num_kv_heads,
                               int num_seqs, int max_query_len, int max_pages_per_seq, int cus,
                               bool allow_split);

// dyn: dynamic per-token scales (p.k_scale / p.v_scale are the pools
// [P][Hkv][16]). att8: all-FP8 attention (e4m3 q and P, fp8 MFMA); fp8
// caches, static scales. plan: from plan_paged_prefill with the same
// arguments; with a split, p.ws_* point into a workspace of plan.bytes.
hipError_t launch_paged_prefill(const PrefillParams& p, const PrefillPlan& plan, int head_dim,
                                int fmt, bool dyn, bool att8, hipStream_t stream,
                                hipEvent_t ev_before, hipEvent_t ev_after);

// The decode path's FP32 partition merge over `rows` rows of p.num_q_heads
// heads (grid rows x heads): p.ws_*, p.num_parts, p.out, p.out_bf16, the
// static V scale (or null), p.group, p.scale_per_head. Rows at or past
// *row_limit (a device int, when given) are skipped.
hipError_t launch_partition_merge(const DecodeParams& p, int head_dim, int rows,
                                  hipStream_t stream);

}  // namespace kvfp8
