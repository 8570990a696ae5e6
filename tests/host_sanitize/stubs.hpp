// stubs.hpp - what the recording launch stubs saw (test infrastructure).
#pragma once
#include <stdint.h>

#include "../../fp8_kv_cache_write_amd/csrc/launch.hpp"

struct LaunchLog {
  int writes = 0, dyn_writes = 0, scales = 0, quantizes = 0, reads = 0, decodes = 0, prefills = 0;
  int last_fmt = -1, last_heads = 0, last_head_dim = 0, last_per_head = -1, last_seqs = 0;
  int64_t last_tokens = 0, last_pages = 0;
  float last_fmax = 0.0f;
  bool fused = false, att8 = false, dyn = false;
  int slots = -1, tile_pages = 0;
  kvfp8::DecodeParams decode{};
  kvfp8::PrefillParams prefill{};
  kvfp8::PrefillPlan prefill_plan{};
};

extern LaunchLog g_log;
