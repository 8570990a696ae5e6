// driver.cpp - exercises the host code of the C ABI (argument checks, the
// decode and prefill plans, the workspace layouts, the tuning overrides)
// under AddressSanitizer and UndefinedBehaviorSanitizer, with the launches
// recorded by stubs.cpp instead of run. Prints "host checks passed" and
// exits 0, or names the first failed check and exits 1; a sanitizer error
// aborts. Test infrastructure; built and run by tests/test_sanitizers.py.
#include <stdint.h>
#include <stdio.h>

#include "../../include/kvfp8.h"
#include "stubs.hpp"

#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);      \
      return 1;                                                              \
    }                                                                        \
  } while (0)

namespace {

// fake device addresses: aligned, never dereferenced (the launches are stubs)
void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>((uintptr_t)0x10000000 + off); }
const int32_t* fake_i32() { return static_cast<const int32_t*>(fake(0x1000)); }
const float* fake_f32() { return static_cast<const float*>(fake(0x2000)); }

kvq_layer_desc layer(int hq, int hkv, int d, int dtype = KVQ_FP8_E4M3,
                     int scale = KVQ_SCALE_PER_KV_HEAD, int window = 0, int attn = KVQ_ATTN_BF16) {
  kvq_layer_desc x{};
  x.num_q_heads = hq;
  x.num_kv_heads = hkv;
  x.head_dim = d;
  x.page_size = 16;
  x.cache_dtype = dtype;
  x.scale_mode = scale;
  x.sliding_window = window;
  x.sm_scale = 0.0f;
  x.attn_dtype = attn;
  return x;
}

int attend(const kvq_layer_desc& d, int B, int ctx, void* ws, size_t ws_bytes, int out_dtype = 0) {
  const int max_pages = ctx > 0 ? (ctx + 15) / 16 : 1;
  return kvq_paged_decode_attention(&d, fake(0x100000), out_dtype, fake(0x200000), fake(0x300000),
                                    fake(0x400000), 1 << 20, fake_i32(), max_pages, fake_i32(), B,
                                    ctx, fake_f32(), fake_f32(), ws, ws_bytes, nullptr);
}

// Every planned decode launch: the partitions cover the attended pages, the
// run length is in range, and the workspace sections lie inside the bytes
// that kvq_decode_workspace_bytes reported (with the reduce kernel's slack).
int check_decode_plans() {
  const int shapes[][2] = {{4, 2}, {32, 8}, {64, 8}, {8, 2}, {16, 16}, {128, 8}, {8, 1}, {24, 8}};
  const int dims[] = {64, 128, 256};
  const int dtypes[] = {KVQ_BF16, KVQ_FP8_E4M3, KVQ_FP8_E5M2};
  const int batches[] = {1, 2, 8, 64, 1000};
  const int ctxs[] = {0, 1, 15, 16, 17, 31, 33, 4096, 32768, 98304, 131072, 1 << 20, 1 << 27};
  const int windows[] = {0, 1, 16, 128, 4096};
  for (auto& s : shapes)
    for (int D : dims)
      for (int dt : dtypes)
        for (int W : windows)
          for (int B : batches)
            for (int ctx : ctxs) {
              const kvq_layer_desc d = layer(s[0], s[1], D, dt, KVQ_SCALE_PER_KV_HEAD, W);
              size_t bytes = 0;
              CHECK(kvq_decode_workspace_bytes(&d, B, ctx, &bytes) == KVQ_OK);
              const int before = g_log.decodes;
              CHECK(attend(d, B, ctx, bytes ? fake() : nullptr, bytes) == KVQ_OK);
              CHECK(g_log.decodes == before + 1);
              const kvfp8::DecodeParams& p = g_log.decode;
              CHECK(p.num_parts >= 1 && p.pages_per_wave >= 1 && p.pages_per_wave <= 64);
              // a window of W positions may straddle one more page than W / 16
              const int64_t pages =
                  W > 0 && ctx > W ? ((int64_t)W + 15) / 16 + 1 : ((int64_t)ctx + 15) / 16;
              CHECK((int64_t)p.num_parts * 4 * p.pages_per_wave >= pages);
              CHECK(p.group == s[0] / s[1] && p.num_kv_heads == s[1]);
              CHECK(g_log.tile_pages == 2 || g_log.tile_pages == 4);
              if (p.num_parts == 1) {
                CHECK(p.direct == 1 && bytes == 0);
              } else {
                const uintptr_t lo = (uintptr_t)fake(), hi = lo + bytes;
                const uint64_t rows = (uint64_t)B * s[0] * p.num_parts;
                CHECK((uintptr_t)p.ws_m == lo);
                CHECK((uintptr_t)(p.ws_m + rows) <= (uintptr_t)p.ws_l);
                CHECK((uintptr_t)(p.ws_l + rows) <= (uintptr_t)p.ws_o);
                CHECK((uintptr_t)(p.ws_o + (rows + kvfp8::kReduceChunk) * D) <= hi);
                CHECK((uintptr_t)p.ws_o % 256 == 0 && (uintptr_t)p.ws_l % 256 == 0);
                // one byte short: refused before any launch
                CHECK(attend(d, B, ctx, fake(), bytes - 1) == KVQ_ERR_WORKSPACE_TOO_SMALL);
                CHECK(g_log.decodes == before + 1);
              }
            }
  return 0;
}

// Every planned prefill launch: the query blocks cover the chunk, the key
// partitions cover the key tiles, and a split has the workspace it needs.
int check_prefill_plans() {
  const int shapes[][3] = {{32, 8, 128}, {64, 8, 64}, {8, 2, 256}, {6, 2, 128}, {16, 16, 64}};
  const int dtypes[] = {KVQ_BF16, KVQ_FP8_E4M3};
  const int seqs[] = {1, 3, 64};
  const int qlens[] = {1, 7, 48, 512, 2048, 32768};
  const int pagecounts[] = {1, 2, 33, 512, 2048, 8192};
  for (auto& s : shapes)
    for (int dt : dtypes)
      for (int B : seqs)
        for (int mq : qlens)
          for (int mp : pagecounts) {
            const kvq_layer_desc d = layer(s[0], s[1], s[2], dt);
            size_t bytes = 0;
            CHECK(kvq_prefill_workspace_bytes(&d, B, mq, mp, &bytes) == KVQ_OK);
            const int before = g_log.prefills;
            const int st = kvq_paged_prefill_attention(
                &d, fake(0x100000), 0, fake(0x200000), fake(0x300000), fake(0x400000), 1 << 20,
                fake_i32(), mp, fake_i32(), fake_i32(), B, mq, fake_f32(), fake_f32(),
                bytes ? fake() : nullptr, bytes, nullptr);
            CHECK(st == KVQ_OK);
            CHECK(g_log.prefills == before + 1);
            const kvfp8::PrefillPlan& pl = g_log.prefill_plan;
            CHECK(pl.ncg >= 1 && pl.ncg <= 3);
            CHECK((int64_t)pl.qblocks * pl.pos_per_block >= mq);
            CHECK((int64_t)pl.num_parts * pl.part_tiles >= (mp + 1) / 2);
            CHECK(pl.bytes == bytes && (pl.num_parts == 1) == (bytes == 0));
            if (pl.num_parts > 1) {
              const uint64_t slots = (uint64_t)B * mq * s[0] * pl.num_parts;
              CHECK(pl.off_l >= slots * 4 && pl.off_o >= pl.off_l + slots * 4);
              CHECK(pl.off_o + (slots + kvfp8::kReduceChunk) * s[2] * 4 <= pl.bytes);
            }
          }
  return 0;
}

// Argument checks: every refusal happens before a launch.
int check_refusals() {
  const kvq_layer_desc ok = layer(32, 8, 128);
  const int launches = g_log.decodes + g_log.writes + g_log.prefills;
  kvq_layer_desc bad = ok;
  CHECK(attend(ok, 1, 100, nullptr, 0) == KVQ_OK);     // 7 pages: no split, no workspace
  const int base = g_log.decodes + g_log.writes + g_log.prefills;
  bad.head_dim = 96;
  CHECK(attend(bad, 1, 100, nullptr, 0) == KVQ_ERR_UNSUPPORTED);
  bad = ok; bad.page_size = 32;
  CHECK(attend(bad, 1, 100, nullptr, 0) == KVQ_ERR_UNSUPPORTED);
  bad = ok; bad.num_q_heads = 30;
  CHECK(attend(bad, 1, 100, nullptr, 0) == KVQ_ERR_UNSUPPORTED);
  bad = ok; bad.num_q_heads = 8 * 17;
  CHECK(attend(bad, 1, 100, nullptr, 0) == KVQ_ERR_UNSUPPORTED);
  bad = ok; bad.cache_dtype = 7;
  CHECK(attend(bad, 1, 100, nullptr, 0) == KVQ_ERR_INVALID_ARG);
  bad = ok; bad.sm_scale = -1.0f;
  CHECK(attend(bad, 1, 100, nullptr, 0) == KVQ_ERR_INVALID_ARG);
  bad = ok; bad.sliding_window = -3;
  CHECK(attend(bad, 1, 100, nullptr, 0) == KVQ_ERR_INVALID_ARG);
  bad = ok; bad.attn_dtype = KVQ_ATTN_FP8; bad.cache_dtype = KVQ_BF16;
  CHECK(attend(bad, 1, 100, nullptr, 0) == KVQ_ERR_UNSUPPORTED);
  CHECK(attend(ok, -1, 100, nullptr, 0) == KVQ_ERR_INVALID_ARG);
  CHECK(attend(ok, 1, -5, nullptr, 0) == KVQ_ERR_INVALID_ARG);
  CHECK(attend(ok, 70000, 100, nullptr, 0) == KVQ_ERR_UNSUPPORTED);
  CHECK(attend(ok, 1, 100, nullptr, 0, 9) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_paged_decode_attention(nullptr, fake(), 0, fake(), fake(), fake(), 1, fake_i32(), 8,
                                   fake_i32(), 1, 100, fake_f32(), fake_f32(), nullptr, 0,
                                   nullptr) == KVQ_ERR_INVALID_ARG);
  // a block table too short for the longest context
  CHECK(kvq_paged_decode_attention(&ok, fake(), 0, fake(), fake(), fake(), 1, fake_i32(), 6,
                                   fake_i32(), 1, 100, fake_f32(), fake_f32(), nullptr, 0,
                                   nullptr) == KVQ_ERR_INVALID_ARG);
  // misaligned q, missing scales of an fp8 layer
  CHECK(kvq_paged_decode_attention(&ok, fake(), 0, fake(8), fake(), fake(), 1, fake_i32(), 8,
                                   fake_i32(), 1, 100, fake_f32(), fake_f32(), nullptr, 0,
                                   nullptr) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_paged_decode_attention(&ok, fake(), 0, fake(), fake(), fake(), 1, fake_i32(), 8,
                                   fake_i32(), 1, 100, nullptr, fake_f32(), nullptr, 0,
                                   nullptr) == KVQ_ERR_INVALID_ARG);
  // the cache write
  CHECK(kvq_kv_cache_write(&ok, fake(), fake(), static_cast<const int64_t*>(fake()), -1, fake(),
                           fake(), 4, fake_f32(), fake_f32(), nullptr) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_kv_cache_write(&ok, fake(), fake(), static_cast<const int64_t*>(fake()), 4, fake(),
                           fake(), 0, fake_f32(), fake_f32(), nullptr) == KVQ_ERR_INVALID_ARG);
  const kvq_layer_desc dyn = layer(32, 8, 128, KVQ_FP8_E4M3, KVQ_SCALE_PER_TOKEN);
  CHECK(kvq_kv_cache_write(&dyn, fake(), fake(), static_cast<const int64_t*>(fake()), 4, fake(),
                           fake(), 4, fake_f32(), fake_f32(), nullptr) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_decode_step(&dyn, fake(), fake(), fake(), fake(), 4, fake(), 0, fake(), fake_i32(), 8,
                        fake_i32(), 1, 100, fake_f32(), fake_f32(), nullptr, 0, nullptr) ==
        KVQ_ERR_INVALID_ARG);
  CHECK(kvq_e4m3_quantize(fake_f32(), -1, fake_f32(), static_cast<uint8_t*>(fake()), nullptr) ==
        KVQ_ERR_INVALID_ARG);
  CHECK(kvq_stream_read(fake(), 17, static_cast<uint32_t*>(fake()), 4, nullptr) ==
        KVQ_ERR_INVALID_ARG);
  CHECK(g_log.decodes + g_log.writes + g_log.prefills == base);
  (void)launches;
  // and the valid forms launch once each
  CHECK(kvq_kv_cache_write(&ok, fake(), fake(), static_cast<const int64_t*>(fake()), 4, fake(),
                           fake(), 4, fake_f32(), fake_f32(), nullptr) == KVQ_OK);
  CHECK(g_log.writes == 1 && g_log.last_tokens == 4 && g_log.last_per_head == 1);
  CHECK(kvq_kv_cache_write_dynamic(&dyn, fake(), fake(), static_cast<const int64_t*>(fake()), 9,
                                   fake(), fake(), 4, static_cast<float*>(fake()),
                                   static_cast<float*>(fake()), nullptr) == KVQ_OK);
  CHECK(g_log.dyn_writes == 1 && g_log.last_tokens == 9 && g_log.last_per_head == 1);
  CHECK(kvq_kv_scale_from_amax(&ok, fake(), 10, static_cast<float*>(fake()), nullptr) == KVQ_OK);
  CHECK(g_log.scales == 1 && g_log.last_fmax == 448.0f);
  const kvq_layer_desc e5 = layer(32, 8, 128, KVQ_FP8_E5M2);
  CHECK(kvq_kv_scale_from_amax(&e5, fake(), 10, static_cast<float*>(fake()), nullptr) == KVQ_OK);
  CHECK(g_log.last_fmax == 57344.0f);
  CHECK(kvq_e5m2_quantize(fake_f32(), 100, fake_f32(), static_cast<uint8_t*>(fake()), nullptr) ==
        KVQ_OK);
  CHECK(g_log.quantizes == 1 && g_log.last_fmt == KVQ_FP8_E5M2);
  CHECK(kvq_stream_read(fake(), 4096, static_cast<uint32_t*>(fake()), 4, nullptr) == KVQ_OK);
  CHECK(g_log.reads == 1);
  size_t bytes = 0;
  CHECK(kvq_decode_workspace_bytes(&ok, 1, 131072, &bytes) == KVQ_OK && bytes > 0);
  const int before = g_log.decodes;
  CHECK(kvq_decode_step(&ok, fake(), fake(), fake(), fake(), 8192, fake(), 1, fake(), fake_i32(),
                        8192, fake_i32(), 1, 131072, fake_f32(), fake_f32(), fake(), bytes,
                        nullptr) == KVQ_OK);
  CHECK(g_log.decodes == before + 1 && g_log.fused && g_log.decode.out_bf16 == 1);
  return 0;
}

// The tuning overrides: range checks and their effect on the plan.
int check_tuning() {
  const kvq_layer_desc d = layer(32, 8, 128);
  size_t base = 0, small = 0;
  CHECK(kvq_decode_workspace_bytes(&d, 1, 32768, &base) == KVQ_OK);
  CHECK(kvq_set_tuning(KVQ_TUNE_PAGES_PER_WAVE, 2) == KVQ_OK);
  CHECK(kvq_decode_workspace_bytes(&d, 1, 32768, &small) == KVQ_OK && small > base);
  CHECK(kvq_set_tuning(KVQ_TUNE_PAGES_PER_WAVE, -1) == KVQ_OK);
  CHECK(kvq_decode_workspace_bytes(&d, 1, 32768, &small) == KVQ_OK && small == base);
  // (the shape override is applied by the launcher below the recorded call)
  CHECK(kvq_set_tuning(KVQ_TUNE_SPLIT_SHAPE, 212) == KVQ_OK);
  CHECK(kvq_set_tuning(KVQ_TUNE_SPLIT_SHAPE, -1) == KVQ_OK);
  CHECK(kvq_set_tuning(KVQ_TUNE_PARTITION_ROTATE, 1) == KVQ_OK);
  CHECK(attend(d, 1, 32768, fake(), base) == KVQ_OK && g_log.decode.rotate == 1);
  CHECK(kvq_set_tuning(KVQ_TUNE_PARTITION_ROTATE, -1) == KVQ_OK);
  CHECK(attend(d, 1, 32768, fake(), base) == KVQ_OK && g_log.decode.rotate == 0);
  CHECK(kvq_set_tuning(KVQ_TUNE_SPLIT_SHAPE, 999) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_set_tuning(42, 1) == KVQ_ERR_INVALID_ARG);
  return 0;
}

}  // namespace

int main() {
  if (check_refusals()) return 1;
  if (check_decode_plans()) return 1;
  if (check_prefill_plans()) return 1;
  if (check_tuning()) return 1;
  printf("host checks passed: %d decode, %d prefill launches planned\n", g_log.decodes,
         g_log.prefills);
  return 0;
}
