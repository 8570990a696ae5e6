/*
 * kvfp8.h - C ABI of the MI355X (gfx950) FP8 (e4m3, e5m2) paged KV-cache
 * library.
 *
 * Two operations make up one decode step of an attention layer:
 *
 *   kvq_kv_cache_write          quantise each new token's K and V into a paged
 *                               cache (the role the vLLM FP8 KV-cache post
 *                               gives to reshape_and_cache_flash, extended to
 *                               one FP32 scale per KV head: "State of FP8 KV
 *                               cache and attention quantization in vLLM",
 *                               section "Kernel and vLLM improvements",
 *                               paragraph "Per-head scales").
 *   kvq_paged_decode_attention  GQA decode attention softmax(q k^T) v over that
 *                               cache, with FP32 two-level accumulation (same
 *                               post, same section, paragraph "Two-level
 *                               accumulation") and split-context partitions
 *                               merged by a separate FP32 reduce kernel.
 *
 * Each layer carries its own cache dtype, so sliding-window layers can stay in
 * bf16 (same post, paragraph "Skip layers").
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Every pointer argument named as device memory must point to memory on
 *    the current HIP device, 16-byte aligned, contiguous in the layout stated.
 *    The caller owns all memory. The library never allocates, frees or
 *    synchronises on the calls listed as such, and keeps no per-call state:
 *    it is safe to call from several host threads on different streams.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *    All work is enqueued on that stream; the call returns before it runs.
 *  - Return value: KVQ_OK (0) or a negative kvq_status. Every argument check
 *    runs on the host before anything is launched, so a non-zero status means
 *    no device memory was touched (KVQ_ERR_HIP aside: a launch failed).
 *    Device-side faults surface on the caller's next synchronisation.
 *
 * E4M3 (OCP FP8): 1 sign, 4 exponent (bias 7), 3 mantissa bits; largest
 * finite magnitude 448, smallest subnormal 2^-9, no infinities, NaN is
 * S.1111.111 (0x7F / 0xFF). Quantisation of an input x with scale s is
 *     code = E4M3_sat_RNE( fp32(x) / s )        (IEEE fp32 division)
 * with round-to-nearest-even, saturation of finite and infinite overflow to
 * +-448 (codes 0x7E / 0xFE), NaN to 0x7F|sign, and the sign of zero kept.
 * The stored code c stands for decode(c) * s.
 * (Format: "FP8量化与长上下文推理" section 1 table; max 448 and the saturating
 * mode: "cooking-agi: FP8 and the KV cache", section "dynamic vs static scale";
 * s = amax/448 and round(x/s): "FP8量化与长上下文推理" section 1.1.)
 *
 * E5M2 (OCP FP8), the second fp8 cache dtype (fp8_e5m2: "cooking-agi",
 * section "how to enable it in the engine"; format: "FP8量化与长上下文推理"
 * section 1 table): 1 sign, 5 exponent (bias 15), 2 mantissa bits; largest
 * finite magnitude 57344, smallest subnormal 2^-16, infinities S.11111.00,
 * NaNs S.11111.xx. The same rule with E5M2 in place of E4M3: saturation of
 * finite and infinite overflow to +-57344 (0x7B / 0xFB), NaN to 0x7F|sign,
 * and the calibrated scale is s = amax / 57344. Stored infinities (which the
 * write never produces) read back as NaN in the attention output.
 *
 * Paged cache layout (the pages leave it open; this library fixes it)
 * ------------------------------------------------------------------
 * A cache is one byte array per layer and per K / V:
 *     [num_pages][num_kv_heads][PB]   with PB = 16 * head_dim * e bytes,
 * e = 1 for KVQ_FP8_E4M3 and KVQ_FP8_E5M2, 2 for KVQ_BF16 (little-endian bf16
 * bits).
 * A page holds 16 consecutive positions of one sequence. Token position t of
 * a sequence lives in page block_table[t / 16], row r = t % 16; a slot is
 * page * 16 + r. Within the PB-byte block of (page, kv head) the element
 * (row r, dim d) sits at byte
 *   K:  ((d / CE) * 16 + r) * 16 + (d % CE) * e                 CE = 16 / e
 *   V:  (d / DB) * 1024 + (r / 4) * 256 + (d % DB) * 4 * e + (r % 4) * e
 *                                                                DB = 64 / e
 * i.e. K is stored in 16-byte chunks of CE consecutive dims per row, chunk-
 * major; V is stored in 1 KiB groups of DB dims, each holding 4 quads of rows
 * with the 4 rows of a quad adjacent for every dim. Both make every 64-lane
 * 16-byte load of the decode kernel one contiguous 1 KiB span.
 * Example (fp8, head_dim 128): K (r=5, d=17) is at byte (1*16+5)*16+1 = 337;
 * V (r=5, d=17) is at byte 0*1024 + 1*256 + 17*4 + 1 = 325.
 */
#ifndef KVFP8_H
#define KVFP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = -1,       /* null / misaligned pointer, negative size,
                                     inconsistent shapes */
  KVQ_ERR_UNSUPPORTED = -2,       /* head_dim not in {64,128,256}, page size
                                     not 16, Hq % Hkv != 0, group > 16 (either
                                     arithmetic mode), Hkv > 65535,
                                     KVQ_ATTN_FP8 over a bf16 cache, dynamic
                                     scales with KVQ_ATTN_FP8 or Hkv > 256 */
  KVQ_ERR_WORKSPACE_TOO_SMALL = -3,
  KVQ_ERR_HIP = -4                /* a HIP runtime call or launch failed */
};

/* Cache element type of a layer. `auto` in the engine flags maps to bf16. */
enum kvq_dtype { KVQ_BF16 = 0, KVQ_FP8_E4M3 = 1, KVQ_FP8_E5M2 = 2 };

/* Scale granularity. K and V always have separate scales.
 *   KVQ_SCALE_PER_TENSOR, KVQ_SCALE_PER_KV_HEAD: static scales, one FP32 value
 *     for the layer tensor or one per KV head ("cooking-agi", section "how to
 *     enable it in the engine": per tensor or per attention head), set once
 *     (kvq_kv_scale_from_amax) and passed as fp32 [1] or [Hkv].
 *   KVQ_SCALE_PER_TOKEN, KVQ_SCALE_PER_TOKEN_HEAD: dynamic scales, one per
 *     written token ("FP8量化与长上下文推理" section 2.2: every new token gets
 *     its own scale; "cooking-agi", section "dynamic vs static scale": each
 *     token's largest value lands on the format maximum). The write computes
 *     s = amax / 448 (57344 for e5m2; 1 when amax is 0, NaN when a value is
 *     NaN) over all of the token's K (or V) values, PER_TOKEN, or over those of
 *     one KV head, PER_TOKEN_HEAD, and stores it beside the page: the scales
 *     of a layer are two fp32 pools [num_pages][Hkv][16] (K and V), entry
 *     [page][h][row] the scale of slot page * 16 + row for KV head h (with
 *     PER_TOKEN every head holds the same value). Attention reads each
 *     attended position's own scales. Written by kvq_kv_cache_write_dynamic
 *     and kvq_decode_step_dynamic; read by kvq_paged_decode_attention (its
 *     k_scale / v_scale arguments are then the pools, 16-byte aligned). Only
 *     with KVQ_ATTN_BF16 arithmetic, and Hkv <= 256. Ignored for bf16 layers. */
enum kvq_scale_mode {
  KVQ_SCALE_PER_TENSOR = 0,
  KVQ_SCALE_PER_KV_HEAD = 1,
  KVQ_SCALE_PER_TOKEN = 2,
  KVQ_SCALE_PER_TOKEN_HEAD = 3
};

/* Output element type of the attention. */
enum kvq_out_dtype { KVQ_OUT_F32 = 0, KVQ_OUT_BF16 = 1 };

/*
 * Arithmetic of the attention over an fp8 cache.
 *   KVQ_ATTN_BF16  the cache codes expand exactly to bf16 and q stays bf16;
 *                  q k^T has exact products, P is carried to about 2^-16
 *                  (bf16 high part + bf16 residue). Group size G <= 16
 *                  (above 8 the decode kernel runs P*V twice, once per part).
 *   KVQ_ATTN_FP8   the whole attention in FP8 e4m3 ("State of FP8 KV cache
 *                  and attention quantization in vLLM", introduction: QK and
 *                  ScoreV products in FP8): each query row is quantised to
 *                  e4m3 with s_q = amax|q_row| / 448 in the kernel, q k^T
 *                  runs on the codes (fp8 MFMA), and the probabilities of
 *                  every aligned 32-position block (positions 32j .. 32j+31)
 *                  are quantised to e4m3 relative to the block's largest
 *                  logit for the P*V product; each block's product is
 *                  rescaled into the FP32 sum, and the softmax normaliser
 *                  sums the unquantised probabilities. G <= 16. fp8 caches
 *                  only (a bf16 layer gives KVQ_ERR_UNSUPPORTED).
 */
enum kvq_attn_dtype { KVQ_ATTN_BF16 = 0, KVQ_ATTN_FP8 = 1 };

/* Per-layer descriptor. */
typedef struct kvq_layer_desc {
  int32_t num_q_heads;     /* Hq */
  int32_t num_kv_heads;    /* Hkv; Hq % Hkv == 0, G = Hq / Hkv <= 16 */
  int32_t head_dim;        /* D in {64, 128, 256} */
  int32_t page_size;       /* must be 16 */
  int32_t cache_dtype;     /* enum kvq_dtype */
  int32_t scale_mode;      /* enum kvq_scale_mode; ignored for bf16 layers */
  int32_t sliding_window;  /* W > 0: attend to the last W positions (the new
                              token included); 0: full attention */
  float sm_scale;          /* softmax scale; 0 means 1/sqrt(head_dim) */
  int32_t attn_dtype;      /* enum kvq_attn_dtype; 0 (bf16 arithmetic) by default */
} kvq_layer_desc;

/*
 * kvq_kv_cache_write - store T new tokens' K and V into the paged caches.
 *   k, v          device bf16 [T][Hkv][D]
 *   slot_mapping  device int64 [T]; slot = page * 16 + row; a slot < 0 or
 *                 >= num_pages * 16 skips the token (checked on the device).
 *                 Two tokens with the same slot: which one wins is
 *                 unspecified.
 *   k_cache, v_cache  device byte arrays in the layout above, num_pages pages.
 *   k_scale, v_scale  device fp32 [1] (per tensor) or [Hkv] (per KV head);
 *                 ignored and may be NULL for bf16 layers, where the bf16 bits
 *                 are copied unchanged.
 * Only the bytes of the written (slot, head) rows change.
 * For fp8 layers each element becomes E4M3_sat_RNE(fp32(x) / s_h), or
 * E5M2_sat_RNE(fp32(x) / s_h) for an e5m2 layer (above). A layer with dynamic
 * scales (KVQ_SCALE_PER_TOKEN*) gives KVQ_ERR_INVALID_ARG: use
 * kvq_kv_cache_write_dynamic.
 */
int kvq_kv_cache_write(const kvq_layer_desc* desc, const void* k, const void* v,
                       const int64_t* slot_mapping, int64_t num_tokens,
                       void* k_cache, void* v_cache, int64_t num_pages,
                       const float* k_scale, const float* v_scale, void* stream);

/*
 * kvq_kv_cache_write_dynamic - the cache write of a layer with dynamic
 * per-token scales (scale_mode KVQ_SCALE_PER_TOKEN or _PER_TOKEN_HEAD, see
 * kvq_scale_mode): each written token's scales are computed from its own
 * values, stored into the pools at its slot, and its codes are
 * E4M3_sat_RNE(fp32(x) / s) (E5M2 for an e5m2 layer) with those scales.
 *   k_scales, v_scales  device fp32 pools [num_pages][Hkv][16], 16-byte
 *                 aligned; only the entries of written slots change
 *   other arguments as for kvq_kv_cache_write
 * A static scale mode on an fp8 layer gives KVQ_ERR_INVALID_ARG; a bf16 layer
 * copies as kvq_kv_cache_write does (the pools are not used).
 */
int kvq_kv_cache_write_dynamic(const kvq_layer_desc* desc, const void* k, const void* v,
                               const int64_t* slot_mapping, int64_t num_tokens,
                               void* k_cache, void* v_cache, int64_t num_pages,
                               float* k_scales, float* v_scales, void* stream);

/*
 * kvq_decode_workspace_bytes - size of the FP32 split workspace that
 * kvq_paged_decode_attention needs for this layer, batch size and longest
 * context (host only, no device work). Writes the size to *bytes; it is 0
 * when no split is needed. The partition plan depends only on these
 * arguments and the current device's compute-unit count.
 */
int kvq_decode_workspace_bytes(const kvq_layer_desc* desc, int32_t num_seqs,
                               int32_t max_context_len, size_t* bytes);

/*
 * kvq_paged_decode_attention - one decode step of GQA attention over a paged
 * cache. Query head i attends with KV head i / G (consecutive query heads
 * share a KV head). For sequence b with L = context_lens[b] (the positions
 * already written, the new token included) it attends to positions
 * [lo, L), lo = max(0, L - W) when sliding_window W > 0, else 0:
 *     z_t = sm_scale * sum_d q[d] * kh[t][d],  p = softmax(z),
 *     out[d] = sum_t p_t * vh[t][d]
 * where kh = decode(code) * k_scale[h] and vh = decode(code) * v_scale[h] for
 * fp8 layers (with dynamic scales: the pools' entries of position t's slot),
 * and the bf16 values for bf16 layers. L == 0 gives zeros.
 *   out           device [B][Hq][D], fp32 or bf16 per out_dtype
 *   q             device bf16 [B][Hq][D]
 *   k_cache, v_cache  as written by kvq_kv_cache_write; num_pages pages
 *   block_tables  device int32 [B][max_pages_per_seq]; entries for the
 *                 attended pages should be in [0, num_pages): an entry
 *                 outside it reads as an empty page (its positions are
 *                 skipped) and is never dereferenced
 *   context_lens  device int32 [B]; each should be in [0, max_context_len].
 *                 On the device a length is cut to max_pages_per_seq * 16 and
 *                 to the partitions planned for max_context_len, so a larger
 *                 value gives a truncated result, never an access out of
 *                 bounds
 *   max_context_len  host int, an upper bound of every context_lens[b]; it
 *                 sizes the partition plan and must match the value given to
 *                 kvq_decode_workspace_bytes
 *   k_scale, v_scale  as for kvq_kv_cache_write, or the scale pools of a
 *                 layer with dynamic scales
 *   workspace     device scratch of at least the bytes reported by
 *                 kvq_decode_workspace_bytes (may be NULL when that is 0);
 *                 clobbered. Calls that share a workspace must be ordered on
 *                 one stream.
 */
int kvq_paged_decode_attention(const kvq_layer_desc* desc, void* out,
                               int32_t out_dtype, const void* q,
                               const void* k_cache, const void* v_cache,
                               int64_t num_pages, const int32_t* block_tables,
                               int32_t max_pages_per_seq,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t max_context_len, const float* k_scale,
                               const float* v_scale, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * kvq_paged_decode_attention_noalloc - kvq_paged_decode_attention for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). The same kernels
 * and results, bit for bit; the split workspace is a library-owned device
 * array of KVQ_NOALLOC_SCRATCH_BYTES (16 MiB) per device, which each device
 * the library runs on holds until the process ends. The call allocates
 * nothing. Every call on one device shares that device's array and leaves
 * its contents behind (nothing in it needs clearing), so calls on one
 * device must be ordered (one stream, or synchronised streams): calls that
 * overlap on one device race.
 *   arguments as for kvq_paged_decode_attention, without the workspace
 * Returns KVQ_ERR_WORKSPACE_TOO_SMALL, before any device call, when the
 * plan for (desc, num_seqs, max_context_len) needs more workspace than the
 * array holds (kvq_decode_workspace_bytes reports the need): for example
 * 64 sequences of 131072 positions of a 32 q / 8 KV head layer.
 */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int kvq_paged_decode_attention_noalloc(const kvq_layer_desc* desc, void* out,
                                       int32_t out_dtype, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       int64_t num_pages, const int32_t* block_tables,
                                       int32_t max_pages_per_seq,
                                       const int32_t* context_lens, int32_t num_seqs,
                                       int32_t max_context_len, const float* k_scale,
                                       const float* v_scale, void* stream);

/*
 * kvq_decode_step - one decode step of a layer in one call: the cache write
 * of every sequence's newest token followed by the attention, i.e. exactly
 *     kvq_kv_cache_write(k_new, v_new, slot of position L-1 of each sequence)
 *     kvq_paged_decode_attention(...)
 * with L = context_lens[b] (the new token included; sequences with L == 0
 * write nothing). The slot is block_tables[b][(L-1)/16] * 16 + (L-1) % 16;
 * an entry outside [0, num_pages) writes nothing. The split kernel does the
 * write itself (the one wave that streams that page quantises the row,
 * stores it and uses the stored bytes), which saves the separate write
 * kernel and its dependency on the decode path of a step. Same results, bit
 * for bit, as the two calls.
 *   k_new, v_new  device bf16 [B][Hkv][D]
 *   k_cache, v_cache  writable caches (layout above)
 *   all other arguments as for kvq_paged_decode_attention
 * A layer with dynamic scales gives KVQ_ERR_INVALID_ARG: use
 * kvq_decode_step_dynamic.
 */
int kvq_decode_step(const kvq_layer_desc* desc, const void* k_new,
                    const void* v_new, void* k_cache, void* v_cache,
                    int64_t num_pages, void* out, int32_t out_dtype,
                    const void* q, const int32_t* block_tables,
                    int32_t max_pages_per_seq, const int32_t* context_lens,
                    int32_t num_seqs, int32_t max_context_len,
                    const float* k_scale, const float* v_scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvq_decode_step_dynamic - kvq_decode_step for a layer with dynamic
 * per-token scales: the new token's scales are computed as
 * kvq_kv_cache_write_dynamic computes them and stored into the pools, then
 * the attention reads every position's scales from the pools. Same results,
 * bit for bit, as kvq_kv_cache_write_dynamic followed by
 * kvq_paged_decode_attention.
 *   k_scales, v_scales  device fp32 pools [num_pages][Hkv][16], 16-byte
 *                 aligned, writable
 *   other arguments as for kvq_decode_step
 */
int kvq_decode_step_dynamic(const kvq_layer_desc* desc, const void* k_new,
                            const void* v_new, void* k_cache, void* v_cache,
                            int64_t num_pages, void* out, int32_t out_dtype,
                            const void* q, const int32_t* block_tables,
                            int32_t max_pages_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_context_len,
                            float* k_scales, float* v_scales, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * kvq_paged_prefill_attention - the prefill (or chunked-prefill) attention of
 * a chunk of new tokens over the paged cache ("State of FP8 KV cache and
 * attention quantization in vLLM", section "Single-request benchmark":
 * prefill is self-attention over the input, its cost quadratic in the input
 * length). Sequence b contributes n_b = query_start[b+1] - query_start[b]
 * query rows (rows query_start[b] .. query_start[b+1]-1 of q and out); they
 * are its last n_b positions, already written into the caches
 * (kvq_kv_cache_write), so row j sits at position pos = context_lens[b] -
 * n_b + j and attends causally to [lo, pos], lo = max(0, pos + 1 - W) with a
 * sliding window W:
 *     out[row][i][d] = sum_t softmax_t(z) vh[t][d],
 *     z_t = sm_scale * sum_d q[row][i][d] kh[t][d],  t in [lo, pos],
 * with kh, vh as for kvq_paged_decode_attention. Probabilities enter the P*V
 * product rounded to bf16; accumulation is FP32. With KVQ_ATTN_FP8 the
 * arithmetic is that of the all-FP8 decode mode, row by row (e4m3 query per
 * row, P per aligned 32-position block relative to the block's largest
 * logit). A row whose position is below 0 (n_b > context_lens[b]) gives
 * zeros.
 *   out           device [T][Hq][D], fp32 or bf16 per out_dtype; T =
 *                 query_start[num_seqs]
 *   q             device bf16 [T][Hq][D]
 *   query_start   device int32 [num_seqs + 1], query_start[0] = 0,
 *                 non-decreasing
 *   context_lens  device int32 [num_seqs], positions written, the chunk
 *                 included; cut to max_pages_per_seq * 16 on the device
 *   max_query_len host int >= every n_b (sizes the grid; rows past it are
 *                 not computed)
 *   workspace     NULL (workspace_bytes 0): every query block attends its
 *                 whole key range in one work-group. Otherwise device
 *                 scratch, 256-byte aligned, of at least the bytes
 *                 kvq_prefill_workspace_bytes reports for the same
 *                 (desc, num_seqs, max_query_len, max_pages_per_seq): a
 *                 short chunk over a long context then splits its keys into
 *                 partitions whose FP32 partial results the decode path's
 *                 reduce kernel merges (same formula as the decode split).
 *                 Clobbered; calls that share one must be ordered on a
 *                 stream. Too small: KVQ_ERR_WORKSPACE_TOO_SMALL.
 *   other arguments as for kvq_paged_decode_attention (static scales or the
 *   pools of dynamic per-token scales; KVQ_ATTN_FP8 with static scales).
 * A call that would need more than 2^31 - 1 work-groups (num_seqs x Hkv x
 * query blocks of max_query_len x key partitions) launches nothing and
 * returns KVQ_ERR_HIP.
 */
int kvq_paged_prefill_attention(const kvq_layer_desc* desc, void* out,
                                int32_t out_dtype, const void* q,
                                const void* k_cache, const void* v_cache,
                                int64_t num_pages, const int32_t* block_tables,
                                int32_t max_pages_per_seq,
                                const int32_t* query_start,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t max_query_len, const float* k_scale,
                                const float* v_scale, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * kvq_prefill_workspace_bytes - size of the workspace that lets
 * kvq_paged_prefill_attention split the keys of a short chunk over a long
 * context (host only, no device work). Writes the size to *bytes; 0 when the
 * plan for these arguments has no split (then the call needs no workspace).
 * The plan depends only on these arguments and the current device's
 * compute-unit count: it splits when the query blocks alone would leave
 * compute units idle and max_pages_per_seq * 16 is at least twice
 * max_query_len.
 */
int kvq_prefill_workspace_bytes(const kvq_layer_desc* desc, int32_t num_seqs,
                                int32_t max_query_len, int32_t max_pages_per_seq,
                                size_t* bytes);

/*
 * kvq_kv_scale_from_amax - static scale calibration of one layer tensor:
 * s = fp32(amax) / 448 over x, per KV head or over the whole tensor per
 * desc->scale_mode ("FP8量化与长上下文推理" section 1.1: scale = max_abs/448;
 * "cooking-agi", section "dynamic vs static scale": the largest value lands
 * on 448). For an e5m2 layer the divisor is 57344, the e5m2 maximum, so the
 * largest value lands there. amax == 0 gives s = 1 (a zero scale cannot
 * quantise anything); a NaN anywhere in the reduced values gives NaN.
 *   x          device bf16 [T][Hkv][D]
 *   scale_out  device fp32 [1] or [Hkv]
 * A dynamic scale mode gives KVQ_ERR_INVALID_ARG (the write sets those).
 */
int kvq_kv_scale_from_amax(const kvq_layer_desc* desc, const void* x,
                           int64_t num_tokens, float* scale_out, void* stream);

/*
 * kvq_e4m3_quantize - the cache write's conversion on a flat array:
 * out[i] = E4M3_sat_RNE(x[i] / *scale). x device fp32 [n], scale device fp32
 * [1], out device uint8 [n]. For quantising data outside the cache layout
 * with exactly the cache's codec.
 */
int kvq_e4m3_quantize(const float* x, int64_t n, const float* scale,
                      uint8_t* out, void* stream);

/*
 * kvq_e5m2_quantize - the same for the e5m2 cache dtype:
 * out[i] = E5M2_sat_RNE(x[i] / *scale), arguments as for kvq_e4m3_quantize.
 */
int kvq_e5m2_quantize(const float* x, int64_t n, const float* scale,
                      uint8_t* out, void* stream);

/* Human-readable text of a status code (static storage). */
const char* kvq_status_string(int32_t status);

/*
 * Tuning overrides for sweeps and tests (not for serving). The launch plan
 * of the decode and prefill calls is a pure function of their arguments and
 * the device's compute-unit count; kvq_set_tuning replaces one of its
 * choices for every later call in the process, until it is set back to -1
 * (the plan decides). Nothing else changes the plan: the environment is
 * never read. The override is process-wide and not synchronised with calls
 * in flight on other host threads.
 *   KVQ_TUNE_PAGES_PER_WAVE      1..64: pages each split-kernel wave streams
 *   KVQ_TUNE_PARTITION_ROTATE    0 plain, 1 rotated partition order
 *   KVQ_TUNE_SPLIT_SHAPE         100*TP + 10*RING + SLOTS: tile pages,
 *                                register tiles, LDS slots; one of 210, 220,
 *                                410, 211, 212, 411 (a shape a mode is not
 *                                built for fails the launch with KVQ_ERR_HIP)
 *   KVQ_TUNE_PREFILL_COLUMN_GROUPS  1..3 query column groups per prefill wave
 *                                (capped at what the layer's kernel holds:
 *                                3 up to head_dim 128, 2 at 256 with static
 *                                scales and bf16 arithmetic, else 1)
 *   KVQ_TUNE_PREFILL_KEY_PARTS   >= 1 key partitions of a prefill with a
 *                                workspace (1: no split)
 * Returns KVQ_ERR_INVALID_ARG for an unknown knob or a value out of range.
 */
enum kvq_tuning_knob {
  KVQ_TUNE_PAGES_PER_WAVE = 0,
  KVQ_TUNE_PARTITION_ROTATE = 1,
  KVQ_TUNE_SPLIT_SHAPE = 2,
  KVQ_TUNE_PREFILL_COLUMN_GROUPS = 3,
  KVQ_TUNE_PREFILL_KEY_PARTS = 4
};
int kvq_set_tuning(int32_t knob, int32_t value);

/*
 * Profiling aid (not thread-safe): between kvq_profile_begin and
 * kvq_profile_end the library records a HIP event pair around every launch of
 * the split-decode kernel and of kvq_stream_read's kernel (up to
 * max_launches of them) on the stream of that launch. kvq_profile_end synchronises those events and returns the summed
 * kernel time in milliseconds and the number of launches recorded.
 */
int kvq_profile_begin(int32_t max_launches);
int kvq_profile_end(double* total_ms, int64_t* launches);

/*
 * Timing aid: a plain streaming read, the reference point for the split
 * kernel's bandwidth. Reads every byte of src[0, n_bytes) once with 16-byte
 * non-temporal loads (num_blocks work-groups of 256 threads, each a
 * contiguous share) and writes the XOR of each work-group's 32-bit words
 * into sink[0, num_blocks). So the XOR of all of sink equals the XOR of
 * every 32-bit word of src.
 *   src:  device, 16-byte aligned; n_bytes a multiple of 16 (0: no launch)
 *   sink: device uint32 [num_blocks], written
 * Returns KVQ_ERR_INVALID_ARG for a bad size, count or pointer, KVQ_ERR_HIP
 * if the launch fails. Asynchronous on stream; allocates nothing.
 */
int kvq_stream_read(const void* src, int64_t n_bytes, uint32_t* sink, int32_t num_blocks,
                    void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KVFP8_H */
