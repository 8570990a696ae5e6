// prefill_plan.cpp - the launch plan of the chunked-prefill attention
// (kvq_paged_prefill_attention, paged_prefill.hip): column groups per wave,
// query blocks and the key split with its workspace. Host code only; a pure
// function of its arguments, the compute-unit count and the kvq_set_tuning
// overrides.
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/kvfp8.h"
#include "launch.hpp"

namespace kvfp8 {

namespace {

constexpr int kPlanPage = 16;       // positions per page

// Column groups per wave the registers allow (each shares the tile's
// fp8 -> bf16 expansion and LDS reads): three up to head dim 128 (a bf16
// cache at 128 with its K/V codes read just in time), two at 256 (the
// static-scale, bf16-arithmetic instances, just in time); the launcher gives
// the instances that hold fewer what they hold.
int prefill_ncg_max(int head_dim, int fmt) {
  (void)fmt;
  return head_dim >= 256 ? 2 : 3;
}

}  // namespace

// Smallest key partition of the split, in 32-position tiles.
constexpr int kMinPartTiles = 16;

PrefillPlan plan_paged_prefill(int head_dim, int fmt, int num_q_heads, int num_kv_heads,
                               int num_seqs, int max_query_len, int max_pages_per_seq, int cus,
                               bool allow_split) {
  PrefillPlan pl{};
  const int G = num_q_heads / num_kv_heads;
  const int ppc = 16 / G;                                  // positions per column group
  const int ncg_max = prefill_ncg_max(head_dim, fmt);
  // explicit overrides for tests and sweeps (kvq_set_tuning): column groups
  // per wave (1..3) and key partitions (1 = no split)
  int forced = std::max(tuning_override(KVQ_TUNE_PREFILL_COLUMN_GROUPS), 0);
  int forced_parts = std::max(tuning_override(KVQ_TUNE_PREFILL_KEY_PARTS), 0);
  if (forced < 1 || forced > ncg_max) forced = 0;
  auto blocks = [&](int ncg) -> int64_t {
    const int ppb = kPrefillWaves * ncg * ppc;
    return ((int64_t)max_query_len + ppb - 1) / ppb;
  };
  auto groups = [&](int ncg) -> int64_t { return (int64_t)num_seqs * num_kv_heads * blocks(ncg); };
  int ncg = forced ? forced : ncg_max;
  const int64_t rows = (int64_t)num_seqs * max_query_len;
  const int max_tiles = (max_pages_per_seq + 1) / 2;
  // Split the keys when the query blocks leave compute units idle and the
  // key range is at least twice the chunk (a chunk at the end of a long
  // context; whole prompts keep the column-group reduction below). The merge
  // grid has a row per query row, so the rows must fit its y dimension.
  // The partition count is chosen by the waves of work-groups it makes (two
  // resident per CU): time ~ waves / parts, plus 2 % per extra wave for the
  // fixed cost of each work-group; unsplit, ~ the waves of the query blocks.
  int parts = 1;
  if (allow_split && rows <= 65535) {
    const int64_t slots = 2LL * cus, base = groups(ncg);
    if (forced_parts >= 1) {
      parts = std::min(forced_parts, std::max(max_tiles, 1));
    } else if (base < 4 * slots && max_tiles >= 2 * kMinPartTiles &&
               (int64_t)max_pages_per_seq * kPlanPage >= 2LL * max_query_len) {
      double best = (double)((base + slots - 1) / slots);
      for (int k = 1; k <= 4; ++k) {
        const int64_t np = std::min<int64_t>(k * slots / base, max_tiles / kMinPartTiles);
        if (np < 2) continue;
        const int64_t waves = (base * np + slots - 1) / slots;
        const double cost = (double)waves / (double)np * (1.0 + 0.02 * (double)(waves - 1));
        if (cost < best) {
          best = cost;
          parts = (int)np;
        }
      }
    }
  }
  if (parts > 1) {
    pl.part_tiles = (max_tiles + parts - 1) / parts;
    parts = (max_tiles + pl.part_tiles - 1) / pl.part_tiles;
  }
  if (parts <= 1) {
    parts = 1;
    pl.part_tiles = max_tiles;
    // fewer column groups when the grid would leave compute units idle
    // (short prompts), aiming at two work-groups per CU. A chunk over a key
    // range at least twice its length gives every work-group about the same
    // work, so there the smaller groups must still fit in one wave of
    // work-groups: a partial second wave costs more than the idle slots (a
    // 3000-row chunk over 100000 positions: 504 groups of three in one wave,
    // 3.9 ms; 752 groups of two, 6.1 ms). A whole prompt's causal work
    // shrinks from block to block and fills the second wave (1500 to 3000
    // rows: 15-19 % faster with the smaller groups).
    const bool even_work = (int64_t)max_pages_per_seq * kPlanPage >= 2LL * max_query_len;
    if (!forced)
      while (ncg > 1 && groups(ncg) < 2LL * cus && (!even_work || groups(ncg - 1) <= 2LL * cus))
        --ncg;
  }
  pl.ncg = ncg;
  pl.pos_per_block = kPrefillWaves * ncg * ppc;
  pl.qblocks = (int)blocks(ncg);
  pl.num_parts = parts;
  if (parts > 1) {
    // (m, l, o[D]) per (query row, query head, partition), as the decode
    // split's workspace, with the merge's chunk of slack after o
    auto round_up = [](size_t x, size_t a) { return (x + a - 1) / a * a; };
    const size_t slots = (size_t)rows * num_q_heads * parts;
    pl.off_l = round_up(slots * sizeof(float), 256);
    pl.off_o = pl.off_l + round_up(slots * sizeof(float), 256);
    pl.bytes = pl.off_o + round_up((slots + kReduceChunk) * head_dim * sizeof(float), 256);
  }
  return pl;
}

}  // namespace kvfp8
