// paged_prefill.hip - chunked-prefill attention over the paged FP8 (e4m3,
// e5m2) or bf16 KV cache on gfx950: every new query row attends causally to
// its prefix (window-limited), softmax(q k^T) v with online-softmax
// rescaling and FP32 accumulation.
//
// Prefill is the compute-bound phase of the pages' single-request benchmark
// ("State of FP8 KV cache and attention quantization in vLLM", section
// "Single-request benchmark": the quadratic TTFT term is self-attention over
// the input); the same post (section "Large head-dim limits") traces the FA3
// FP8 prefill slowdown to the register cost of two-level accumulation. On
// CDNA4 the MFMA reads and writes its accumulator in FP32 on every
// instruction, so each 32-position product (level 1, inside the MFMA) is
// promoted into the FP32 accumulator (level 2) at once, with no second copy
// of the output tile.
//
// Design (MI355X):
//  * the MFMA layout of the decode kernel: A = 16 key rows straight from the
//    cache layout (fp8 codes expanded exactly to bf16), B = 16 query columns;
//    here a column is one (query position, head of the GQA group) pair, so a
//    16-column group holds 16/G positions of all G heads;
//  * a work-group of 4 waves covers NCG column groups per wave and shares
//    every 2-page K/V tile: the tile is staged once into LDS (direct
//    global->LDS loads, double-buffered) and each wave reads it into its
//    operand registers;
//  * work-groups are mapped XCD-aware: the query blocks of one (sequence, KV
//    head) run on one XCD and share its L2, heaviest (latest) blocks first.
#include <hip/hip_ext.h>
#include <math.h>
#include <stdlib.h>

#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

namespace kvfp8 {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr float kLazyLog2 = 8.0f;   // running max raised only past +8 (P <= 256)
constexpr int kNumXcd = 8;          // MI355X: 8 XCDs, work-groups dealt round-robin

// IEEE maximum (a NaN operand gives NaN): one v_maximum3_f32, with none of
// the input quieting that fmaxf needs on operands of unknown origin. A NaN
// logit makes its row NaN either way (its p is NaN).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Max over the four lanes c, c+16, c+32, c+48 that hold one MFMA column.
__device__ __forceinline__ float col_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float col_sum(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

}  // namespace

// Bf16 arithmetic with static scales at head dim 256 (two column groups;
// one as well for a bf16 cache), and a bf16 cache at head dim 128 (three
// groups): the tile's K and V codes are read from LDS as they are used (K
// per q k^T step or pair of steps, V per group of P*V blocks, every V block
// expanded once and used by each column group) instead of all at the top of
// the tile, which frees the registers of one more column group at two waves
// per SIMD. (An fp8 cache at one group keeps the codes in registers: faster
// there.)
template <int D, int FMT, int NCG, bool DYN, bool ATT8>
constexpr bool prefill_jit() {
  return ((D >= 256 && (FMT == kFmtBf16 || NCG >= 2)) ||
          (D == 128 && FMT == kFmtBf16 && NCG >= 3)) &&
         !DYN && !ATT8;
}

template <int D, int FMT, int NCG, bool DYN, bool ATT8>
__global__ __launch_bounds__(kPrefillWaves * kWave, (prefill_jit<D, FMT, NCG, DYN, ATT8>() ? 2 : 1))
void paged_prefill_kernel(const PrefillParams p) {
  constexpr int NW = kPrefillWaves;
  constexpr bool FP8 = FMT != kFmtBf16;
  constexpr bool JIT = prefill_jit<D, FMT, NCG, DYN, ATT8>();
  constexpr int E = FP8 ? 1 : 2;
  constexpr int PB = kPage * D * E;     // bytes of one (page, head) block
  constexpr int NI = PB / 1024;         // 1 KiB loads per page per tensor
  constexpr int NK = D / 32;            // q k^T MFMAs per page
  constexpr int NBLK = D / 16;          // P*V output blocks of 16 dims
  constexpr int KV_BYTES = 2 * 2 * PB;  // K and V of 2 pages
  // dynamic scales: the tile's 2 pages x (16 K + 16 V) fp32 follow them
  constexpr int TILE = KV_BYTES + (DYN ? 2 * 2 * kPage * 4 : 0);
  constexpr int LPT = 2 * 2 * NI;       // 1 KiB loads per tile
  static_assert(!DYN || FP8, "dynamic scales belong to fp8 caches");
  static_assert(!ATT8 || (FP8 && !DYN), "all-FP8 attention: fp8 caches, static scales");
  static_assert(LPT % NW == 0, "every wave stages the same number of chunks");
  static_assert(2 * TILE <= 64 * 1024, "direct-to-LDS loads address the first 64 KiB");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int qd = lane >> 4;             // row quad of the MFMA layout
  const int c = lane & 15;              // MFMA column

  // ---- which (sequence, KV head, key partition, query block): XCD-aware ---
  // Consecutive logical blocks share a (sequence, KV head, key partition),
  // so the query blocks reading the same keys run on one XCD (one L2), a
  // causal unit's blocks heaviest first. Two cases take another order
  // (none with a key split, whose blocks all see one partition):
  //  * the (sequence, KV head) units do not divide evenly over the XCDs, or
  //    several sequences have unequal work (rows, or a long key range):
  //    the contiguous runs would give one XCD the long rows and another the
  //    short ones. With at least two waves of work-groups (two per CU on
  //    256 CUs) the blocks go round-robin over the XCDs in heaviest-first
  //    order instead. Measured at whole prompts: 2 units (head dim 256)
  //    601 -> 942 TFLOP/s, 10 units 963 -> 1095, 12 units 1025 -> 1113,
  //    ragged batches 16384 + 2048 tokens 617 -> 1013, 12000 / 3000 / 6000
  //    / 500 tokens 397 -> 920; the 8 units of one prompt, or a batch of
  //    equal prompts, keep the grouped order (3-14 % faster there);
  //  * a grid of one wave (more work-groups than CUs, at most two per CU)
  //    runs every block at once, two to a CU: the first work-group of each
  //    CU takes the r-th heaviest block and the second the r-th lightest
  //    (ranked across units), so no CU holds two long rows (1024-2048-token
  //    prompts 3-6 % faster, head dim 256 at 4096 tokens 18 %).
  const int per_bh = p.qblocks * p.num_parts;
  const int total = p.num_seqs * p.num_kv_heads * per_bh;
  const int units = p.num_seqs * p.num_kv_heads;
  bool round_robin = p.num_parts == 1 && total >= 2 * 2 * 256;
  if (round_robin && units % kNumXcd == 0) {
    round_robin = false;
    if (p.num_seqs > 1) {
      const bool long_keys = (int64_t)p.max_pages_per_seq * kPage >= 2LL * p.max_query_len;
      round_robin = long_keys || p.query_start[p.num_seqs] != p.num_seqs * p.max_query_len;
    }
  }
  const bool pair_up = p.num_parts == 1 && total > 256 && total <= 2 * 256;
  const int per_xcd = (int)gridDim.x / kNumXcd;
  int logical;
  if (pair_up) {
    const int w = (int)blockIdx.x;
    if (w >= total) return;
    const int half = (total + 1) / 2;
    const int rank = w < half ? w : total - 1 - (w - half);   // 0: the heaviest block
    logical = (rank % units) * per_bh + rank / units;
  } else {
    logical = round_robin ? (int)blockIdx.x
                          : (int)(blockIdx.x % kNumXcd) * per_xcd + (int)(blockIdx.x / kNumXcd);
  }
  if (logical >= total) return;
  const int bh = logical / per_bh;
  const int part = (logical % per_bh) / p.qblocks;
  const int qb = p.qblocks - 1 - logical % p.qblocks;     // latest (heaviest) block first
  const int b = bh / p.num_kv_heads;
  const int h = bh % p.num_kv_heads;
  const int G = p.group;
  const int ppc = 16 / G;               // positions per column group

  const int q0 = p.query_start[b];
  const int n = p.query_start[b + 1] - q0;
  int L = p.context_lens[b];
  if (L > p.max_pages_per_seq * kPage) L = p.max_pages_per_seq * kPage;
  const int r0 = qb * p.pos_per_block;
  if (r0 >= n) return;
  const int r_last = min(r0 + p.pos_per_block, n) - 1;
  const int off = L - n;                // position of query row r is off + r

  // ---- this lane's query columns ------------------------------------------
  // col_row: the column is a row of this sequence (its output is written);
  // col_ok: that row's position is not below 0 (it attends something)
  int qpos[NCG], qrow[NCG];
  bool col_ok[NCG], col_row[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int slot = c / G;
    const int r = r0 + (wave * NCG + cg) * ppc + slot;
    col_row[cg] = slot < ppc && r < n;
    col_ok[cg] = col_row[cg] && off + r >= 0;
    qpos[cg] = col_ok[cg] ? off + r : -1;
    qrow[cg] = col_row[cg] ? q0 + r : -1;
  }
  const int g = c % G;
  bf16x8 qop[NCG][NK];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const uint16_t* qr = p.q + ((int64_t)max(qrow[cg], 0) * p.num_q_heads + h * G + g) * D;
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const int d0 = FP8 ? 16 * (4 * (s / 2) + qd) + 8 * (s % 2) : 8 * (4 * s + qd);
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (col_ok[cg]) w = *reinterpret_cast<const uint4*>(qr + d0);
      qop[cg][s] = bits_to_bf16x8(w);
    }
  }
  // static scales; dynamic ones (pools [page][head][row]) are per position
  const float ks = FP8 && !DYN ? p.k_scale[p.scale_per_head ? h : 0] : 1.0f;
  const float vs = FP8 && !DYN ? p.v_scale[p.scale_per_head ? h : 0] : 1.0f;
  float c_log2 = ks * p.sm_scale_log2;
  if (c_log2 < 0.0f) {              // keep the scale non-negative: q -> -q is exact
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        uint4 w = __builtin_bit_cast(uint4, qop[cg][s]);
        w.x ^= 0x80008000u; w.y ^= 0x80008000u; w.z ^= 0x80008000u; w.w ^= 0x80008000u;
        qop[cg][s] = bits_to_bf16x8(w);
      }
    c_log2 = -c_log2;
  }
  const float rcp_c = 1.0f / c_log2;   // (the lazy bar's unit change; inf for c = 0)
  // All-FP8 mode: every column's query row as e4m3 codes, s_q per column
  uint64_t qop8[ATT8 ? NCG : 1][ATT8 ? NK : 1];
  float cq[NCG];                    // logit scale of each column group's column
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    cq[cg] = c_log2;
    if constexpr (ATT8) cq[cg] = quantize_q_e4m3<NK>(qop[cg], qop8[cg]) * c_log2;
  }

  // ---- key range of the work-group: [key_lo, key_hi] ----------------------
  const int pos_first = off + r0, pos_last = off + r_last;
  const int key_lo = p.window > 0 ? max(0, pos_first + 1 - p.window) : 0;
  const int key_hi = pos_last;
  int first_page = (key_lo / kPage) & ~1;                   // tiles on 2-page pairs
  const int end_page = key_hi >= 0 ? key_hi / kPage + 1 : 0;
  int ntiles = end_page > first_page ? (end_page - first_page + 1) / 2 : 0;
  if (p.num_parts > 1) {
    // this partition's tiles (absolute tile index = page / 2) of that range
    const int t_lo = max(first_page / 2, part * p.part_tiles);
    const int t_hi = min(first_page / 2 + ntiles, (part + 1) * p.part_tiles);
    first_page = 2 * t_lo;
    ntiles = max(t_hi - t_lo, 0);
  }
  // keys every column of the work-group may see without a mask
  const int free_lo = p.window > 0 ? pos_last + 1 - p.window : 0;
  const int free_hi = pos_first;   // a key <= this is at or before every column's position

  // Page ids of the key range, 64 per register chunk (lane l: page base + l),
  // the next chunk loaded ahead, so a tile's loads never wait for its
  // block-table entries.
  const int32_t* bt_row = p.block_tables + (int64_t)b * p.max_pages_per_seq;
  auto load_chunk = [&](int base) -> int {
    const int idx = base + lane;
    return idx < end_page ? bt_row[idx] : -1;
  };
  int chunk_base = first_page;
  int chunk = load_chunk(first_page);
  int chunk_next = load_chunk(first_page + kWave);
  auto page_id = [&](int idx) -> int {      // uniform, idx non-decreasing; -1: missing or invalid
    if (idx >= end_page) return -1;
    if (idx - chunk_base >= kWave) {
      chunk = chunk_next;
      chunk_base += kWave;
      chunk_next = load_chunk(chunk_base + kWave);
    }
    const int pid = __builtin_amdgcn_readlane(chunk, idx - chunk_base);
    return (pid < 0 || (int64_t)pid >= p.num_pages) ? -1 : pid;
  };

  __shared__ __align__(16) uint8_t smem[2 * TILE];
  const int64_t page_stride = (int64_t)p.num_kv_heads * PB;
  const uint8_t* kbase = p.k_cache + (int64_t)h * PB;
  const uint8_t* vbase = p.v_cache + (int64_t)h * PB;

  // chunk j of a tile slot: page j / (2 NI), K (j % 2NI < NI) or V, 1 KiB i;
  // pid_a / pid_b receive the tile's two page ids (-1: missing, masked)
  auto stage = [&](int t, int& pid_a, int& pid_b) {
    uint8_t* dst = smem + (t & 1) * TILE;
    pid_a = page_id(first_page + 2 * t);
    pid_b = page_id(first_page + 2 * t + 1);
#pragma unroll
    for (int u = 0; u < LPT / NW; ++u) {
      const int j = wave * (LPT / NW) + u;
      const int pg = j / (2 * NI), kv = (j % (2 * NI)) / NI, i = j % NI;
      const int pid = max(pg == 0 ? pid_a : pid_b, 0);          // missing: page 0, masked
      const uint8_t* src = (kv ? vbase : kbase) + (int64_t)pid * page_stride + 1024 * i;
      __builtin_amdgcn_global_load_lds((glb_void_t*)(src + 16 * lane),
                                       (lds_void_t*)(dst + 1024 * j), 16, 0, 0);
    }
    if constexpr (DYN) {
      // lane l < 16: page l / 8, K (l % 8 < 4) or V scales of rows
      // 4 (l % 4) .. +3; every wave loads the same 256 bytes, so each wave's
      // wait covers them
      if (lane < 16) {
        const int pid = max(lane < 8 ? pid_a : pid_b, 0);
        const float* pool = (lane % 8) < 4 ? p.k_scale : p.v_scale;
        const float* src = pool + ((int64_t)pid * p.num_kv_heads + h) * kPage + 4 * (lane % 4);
        __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)(dst + KV_BYTES), 16, 0,
                                         0);
      }
    }
  };

  // m_run: running maximum (log2 domain); neg_m: -m_run, or 0 while m_run is
  // -inf (every logit so far masked), the exponent's offset; it changes only
  // when m_run does
  // t_raw (static scales, bf16 arithmetic): the lazy bar in raw-logit units,
  // (m_run + kLazyLog2) / c; a lane whose raw maximum passes it takes the
  // rescale branch, which decides on the scaled maximum itself
  constexpr bool RAW_BAR = !ATT8 && !DYN;
  float m_run[NCG], neg_m[NCG], l_run[NCG], t_raw[RAW_BAR ? NCG : 1];
  f32x4 acc[NCG][NBLK];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    m_run[cg] = -INFINITY;
    neg_m[cg] = -0.0f;
    if constexpr (RAW_BAR) t_raw[cg] = -INFINITY;
    l_run[cg] = 0.0f;
#pragma unroll
    for (int i = 0; i < NBLK; ++i) acc[cg][i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // Two LDS slots: tile t + 1 is staged while tile t is computed. (A third
  // slot gains nothing: the work-group barrier's release fence waits for
  // every outstanding load; a bare barrier with hand-placed waits measured
  // slower, the compiler then no longer overlapping the slot reads.)
  int pid_next0 = -1, pid_next1 = -1;
  if (ntiles > 0) stage(0, pid_next0, pid_next1);
  for (int t = 0; t < ntiles; ++t) {
    const int pid0 = pid_next0, pid1 = pid_next1;
    // this wave's loads of tile t are done; after the barrier everyone's are,
    // and every wave has finished reading the slot tile t + 1 goes to
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const uint8_t* slot = smem + (t & 1) * TILE;
    // this lane's 16 bytes of 1 KiB chunk i of page pg's K (kv = 0) or V
    auto lds_code = [&](int pg, int kv, int i) -> uint4 {
      return *reinterpret_cast<const uint4*>(slot + 1024 * (2 * NI * pg + kv * NI + i) +
                                             16 * lane);
    };
    uint4 tk[2][JIT ? 1 : NI], tv[2][JIT ? 1 : NI];
    if constexpr (!JIT) {
#pragma unroll
      for (int pg = 0; pg < 2; ++pg)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          tk[pg][i] = lds_code(pg, 0, i);
          tv[pg][i] = lds_code(pg, 1, i);
        }
    }
    // JIT: the V-code masks (fp8: a byte per row; bf16: rows 4qd+{0,1} and
    // 4qd+{2,3} as halves), applied as V is read
    uint32_t vkeep8[2] = {~0u, ~0u}, vkeep_lo[2] = {~0u, ~0u}, vkeep_hi[2] = {~0u, ~0u};
    // dynamic scales of this lane's rows 4qd..4qd+3 of each page
    f32x4 sk[2], sv[2];
    if constexpr (DYN) {
#pragma unroll
      for (int pg = 0; pg < 2; ++pg) {
        sk[pg] = *reinterpret_cast<const f32x4*>(slot + KV_BYTES + 16 * (8 * pg + qd));
        sv[pg] = *reinterpret_cast<const f32x4*>(slot + KV_BYTES + 16 * (8 * pg + 4 + qd));
      }
    }
    if (t + 1 < ntiles) stage(t + 1, pid_next0, pid_next1);

    // ---- masks of the V codes (boundary tiles only) -------------------------
    const int k0 = (first_page + 2 * t) * kPage;            // first key of the tile
    // masked keys get p = 0, but unwritten rows (positions >= L) and rows of
    // missing pages may hold NaN codes, and 0 * NaN is NaN: zero those rows'
    // V codes in the tile registers (rows 4qd..4qd+3 of each page per lane)
    if (k0 + 2 * kPage > L || pid0 < 0 || pid1 < 0) {
#pragma unroll
      for (int pg = 0; pg < 2; ++pg) {
        const bool page_ok = (pg == 0 ? pid0 : pid1) >= 0;
        uint32_t keep_lo = 0u, keep_hi = 0u;              // rows 4qd+{0,1} / {2,3} (bf16)
        uint32_t keep8 = 0u;                              // rows 4qd+0..3, one byte each (fp8)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = page_ok && k0 + pg * kPage + 4 * qd + e < L;
          keep8 |= ok ? 0xFFu << (8 * e) : 0u;
          const uint32_t half = ok ? (e % 2 ? 0xFFFF0000u : 0x0000FFFFu) : 0u;
          if (e < 2) keep_lo |= half; else keep_hi |= half;
        }
        if constexpr (DYN) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!(page_ok && k0 + pg * kPage + 4 * qd + e < L)) sk[pg][e] = sv[pg][e] = 0.0f;
        }
        if constexpr (JIT) {
          vkeep8[pg] = keep8;
          vkeep_lo[pg] = keep_lo;
          vkeep_hi[pg] = keep_hi;
        }
#pragma unroll
        for (int i = 0; i < (JIT ? 0 : NI); ++i) {
          if constexpr (FP8) {
            tv[pg][i].x &= keep8; tv[pg][i].y &= keep8; tv[pg][i].z &= keep8; tv[pg][i].w &= keep8;
          } else {
            tv[pg][i].x &= keep_lo; tv[pg][i].y &= keep_hi;
            tv[pg][i].z &= keep_lo; tv[pg][i].w &= keep_hi;
          }
        }
      }
    }

    // ---- logits S^T[key row 4qd+e of page pg][column c], per column group ----
    // One straight-line block: the q k^T MFMAs with the K expansion, and the
    // V expansion for P*V among them (independent VALU work that issues while
    // the matrix core runs). In the bf16-arithmetic modes the MFMA phases run
    // at raised wave priority: the other wave on the SIMD (from the other
    // work-group on the CU) then fills the issue slots between this wave's
    // MFMAs with its own VALU work (the softmax), rather than both waves
    // sitting in the same phase (measured: 3-4 % faster at long prompts; the
    // all-FP8 mode, with no K/V expansion, measured 2-3 % slower with it).
    f32x4 sacc[NCG][2];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
      for (int pg = 0; pg < 2; ++pg) sacc[cg][pg] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (!ATT8) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < NK; ++s) {
#pragma unroll
      for (int pg = 0; pg < 2; ++pg) {
        if constexpr (ATT8) {
          // the K codes themselves are the operand (fp8 x fp8 MFMA)
          const uint4 w = tk[pg][s / 2];
          const long kop8 = (long)((s % 2 == 0) ? (((uint64_t)w.y << 32) | w.x)
                                                : (((uint64_t)w.w << 32) | w.z));
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg) {
            if constexpr (FMT == kFmtE5M2)
              sacc[cg][pg] = __builtin_amdgcn_mfma_f32_16x16x32_bf8_fp8(
                  kop8, (long)qop8[cg][s], sacc[cg][pg], 0, 0, 0);
            else
              sacc[cg][pg] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
                  kop8, (long)qop8[cg][s], sacc[cg][pg], 0, 0, 0);
          }
          continue;
        }
        bf16x8 kop;
        if constexpr (FP8) {
          const uint4 w = JIT ? lds_code(pg, 0, s / 2) : tk[pg][s / 2];
          kop = (s % 2 == 0) ? fp8x8_to_bf16x8<FMT>(w.x, w.y) : fp8x8_to_bf16x8<FMT>(w.z, w.w);
        } else {
          kop = bits_to_bf16x8(JIT ? lds_code(pg, 0, s) : tk[pg][s]);
        }
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg)
          sacc[cg][pg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[cg][s], sacc[cg][pg],
                                                                 0, 0, 0);
      }
    }
    // P*V A operands: V^T block blk (16 dims x 32 keys); fp8 codes expanded
    // exactly to bf16, a register shuffle for a bf16 cache
    uint4 vop[(ATT8 || JIT) ? 1 : NBLK];
    if constexpr (!ATT8 && !JIT) {
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
        if constexpr (FP8) {
          const int i = blk / 4, ep = blk % 4;
          const uint4 wa = tv[0][i], wb = tv[1][i];
          const uint32_t da = ep == 0 ? wa.x : ep == 1 ? wa.y : ep == 2 ? wa.z : wa.w;
          const uint32_t db = ep == 0 ? wb.x : ep == 1 ? wb.y : ep == 2 ? wb.z : wb.w;
          vop[blk] =
              __builtin_bit_cast(uint4, cat(fp8x4_to_bf16x4<FMT>(da), fp8x4_to_bf16x4<FMT>(db)));
        } else {
          const int i = blk / 2, ep = blk % 2;
          const uint4 wa = tv[0][i], wb = tv[1][i];
          vop[blk] = ep == 0 ? make_uint4(wa.x, wa.y, wb.x, wb.y) : make_uint4(wa.z, wa.w, wb.z, wb.w);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);

    // static scales: raw logits, c_log2 >= 0 applied inside the exponent;
    // dynamic: each row's logits times c_log2 s_k (row), exponent scale 1;
    // all-FP8: logits scaled here (s_q differs per column)
    const float cexp = (DYN || ATT8) ? 1.0f : c_log2;
    if constexpr (DYN || ATT8) {
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
        for (int pg = 0; pg < 2; ++pg)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sacc[cg][pg][e] *= DYN ? c_log2 * sk[pg][e] : cq[cg];
    }
    // causal / window / missing pages: those logits become -inf
    const bool need_mask = k0 < free_lo || k0 + 2 * kPage - 1 > free_hi || pid0 < 0 || pid1 < 0;
    if (need_mask) {
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        const int lo_c = p.window > 0 ? qpos[cg] + 1 - p.window : 0;
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) {
          const bool page_ok = (pg == 0 ? pid0 : pid1) >= 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int kp = k0 + pg * kPage + 4 * qd + e;
            if (!(page_ok && kp <= qpos[cg] && kp >= lo_c)) sacc[cg][pg][e] = -INFINITY;
          }
        }
      }
    }

    // ---- online softmax (log2 domain), lazy rescale --------------------------
    // Every column group's test first, then one (rarely taken) branch for the
    // rescales, so the exponentials and the P*V MFMAs below form one
    // straight-line block that the scheduler is free to interleave (a branch
    // per group used to split it). A column's maximum passes
    // m_run + kLazyLog2 exactly when one of its four lanes' maxima does
    // (c >= 0, and rounding is monotone), so the bf16-arithmetic modes test
    // each lane's own maximum and reduce across the column's lanes only
    // inside the branch: the same decisions, without two lane exchanges per
    // group and tile. The all-FP8 mode needs the column maximum on every
    // tile (its P is quantised relative to it).
    float lmax[NCG];
    float tmax[ATT8 ? NCG : 1];
    bool grow[ATT8 ? NCG : 1];
    bool any_grow = false;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      float mx = sacc[cg][0][0];
#pragma unroll
      for (int pg = 0; pg < 2; ++pg)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = vmax(mx, sacc[cg][pg][e]);
      if constexpr (ATT8) {
        tmax[cg] = col_max(mx) * cexp;
        grow[cg] = tmax[cg] > m_run[cg] + kLazyLog2;
        any_grow |= grow[cg];
      } else {
        lmax[cg] = mx;
        if constexpr (RAW_BAR) any_grow |= mx > t_raw[cg];
        else any_grow |= mx * cexp > m_run[cg] + kLazyLog2;
      }
    }
    if (__builtin_amdgcn_ballot_w64(any_grow) != 0ull) {
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        float m_new;
        if constexpr (ATT8) {
          m_new = grow[cg] ? tmax[cg] : m_run[cg];
        } else {
          const float cmax = col_max(lmax[cg]) * cexp;
          m_new = cmax > m_run[cg] + kLazyLog2 ? cmax : m_run[cg];
        }
        const float alpha = m_new == m_run[cg] ? 1.0f : __builtin_amdgcn_exp2f(m_run[cg] - m_new);
#pragma unroll
        for (int i = 0; i < NBLK; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[cg][i][e] *= alpha;
        l_run[cg] *= alpha;
        m_run[cg] = m_new;
        neg_m[cg] = m_new == -INFINITY ? -0.0f : -m_new;
        if constexpr (RAW_BAR) t_raw[cg] = (m_new + kLazyLog2) * rcp_c;
      }
    }

    // ---- P and P*V, column group by column group (raised priority) -----------
    uint64_t pop8[ATT8 ? NCG : 1];
    float fb[ATT8 ? NCG : 1];          // all-FP8: weight 2^(tile max - running max)
    bf16x8 popj[JIT ? NCG : 1];        // JIT: every group's P, for the block-major P*V
    if constexpr (!ATT8) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      if constexpr (ATT8) {
        // P of this 32-position block as e4m3 relative to the block's own max
        // (tmax); the normaliser takes the FP32 values
        const bool live = tmax[cg] != -INFINITY;
        const float mb = live ? tmax[cg] : 0.0f;
        const float fbw = live ? __builtin_amdgcn_exp2f(tmax[cg] + neg_m[cg]) : 0.0f;
        float ps = -0.0f;
        uint32_t pw[2];
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) {
          float pe[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pe[e] = __builtin_amdgcn_exp2f(sacc[cg][pg][e] - mb);
            ps += pe[e];
          }
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(pe[0], pe[1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(pe[2], pe[3], w, true);
          pw[pg] = (uint32_t)w;
        }
        pop8[cg] = ((uint64_t)pw[1] << 32) | pw[0];
        fb[cg] = fbw;
        l_run[cg] += fbw * ps;
        continue;                          // P*V below, every column group at once
      }
      float ps = -0.0f;                    // -0 + p is p: no add for the first term
      bf16x8 pop;
#pragma unroll
      for (int pg = 0; pg < 2; ++pg) {
        float pe[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[cg][pg][e], cexp, neg_m[cg]));
          ps += pe[e];
        }
        // dynamic scales: the row's V scale joins P (the normaliser took p)
        if constexpr (DYN) {
#pragma unroll
          for (int e = 0; e < 4; ++e) pe[e] *= sv[pg][e];
        }
        // P^T operand: k index 8qd + 4pg + e is key row 4qd+e of page pg
        const bf16x4 p4 = __builtin_convertvector((f32x4){pe[0], pe[1], pe[2], pe[3]}, bf16x4);
#pragma unroll
        for (int e = 0; e < 4; ++e) pop[4 * pg + e] = p4[e];
      }
      l_run[cg] += ps;
      if constexpr (JIT) {
        popj[cg] = pop;
        continue;                          // P*V below, block by block
      }
      // one k=32 MFMA per 16-dim block
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
        acc[cg][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bits_to_bf16x8(vop[blk]), pop,
                                                               acc[cg][blk], 0, 0, 0);
    }
    if constexpr (JIT && !FP8) {
      // bf16 cache: each 16-byte read of V per page serves two blocks
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        uint4 wa = lds_code(0, 1, i), wb = lds_code(1, 1, i);
        wa.x &= vkeep_lo[0]; wa.y &= vkeep_hi[0]; wa.z &= vkeep_lo[0]; wa.w &= vkeep_hi[0];
        wb.x &= vkeep_lo[1]; wb.y &= vkeep_hi[1]; wb.z &= vkeep_lo[1]; wb.w &= vkeep_hi[1];
#pragma unroll
        for (int ep = 0; ep < 2; ++ep) {
          const int blk = 2 * i + ep;
          const bf16x8 vb = bits_to_bf16x8(ep == 0 ? make_uint4(wa.x, wa.y, wb.x, wb.y)
                                                   : make_uint4(wa.z, wa.w, wb.z, wb.w));
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg)
            acc[cg][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, popj[cg], acc[cg][blk],
                                                                   0, 0, 0);
        }
      }
    }
    if constexpr (JIT && FP8) {
      // V^T block blk (16 dims x 32 keys) expanded once, used by every
      // column group; each 16-byte read of V codes serves four blocks
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const uint4 wa = lds_code(0, 1, i), wb = lds_code(1, 1, i);
#pragma unroll
        for (int ep = 0; ep < 4; ++ep) {
          const int blk = 4 * i + ep;
          const uint32_t da = (ep == 0 ? wa.x : ep == 1 ? wa.y : ep == 2 ? wa.z : wa.w) & vkeep8[0];
          const uint32_t db = (ep == 0 ? wb.x : ep == 1 ? wb.y : ep == 2 ? wb.z : wb.w) & vkeep8[1];
          const bf16x8 vb = bits_to_bf16x8(__builtin_bit_cast(
              uint4, cat(fp8x4_to_bf16x4<FMT>(da), fp8x4_to_bf16x4<FMT>(db))));
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg)
            acc[cg][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, popj[cg], acc[cg][blk],
                                                                   0, 0, 0);
        }
      }
    }
    if constexpr (ATT8) {
      // fp8 x fp8 products of the block, each added into the FP32 sum with
      // its weight fb (level 1: the MFMA over 32 positions; level 2: FP32);
      // every column group's MFMA of a block issues before the adds, so each
      // add finds its product ready
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
        const int i = blk / 4, ep = blk % 4;
        const uint4 wa = tv[0][i], wb = tv[1][i];
        const uint32_t da = ep == 0 ? wa.x : ep == 1 ? wa.y : ep == 2 ? wa.z : wa.w;
        const uint32_t db = ep == 0 ? wb.x : ep == 1 ? wb.y : ep == 2 ? wb.z : wb.w;
        const long vop8 = (long)(((uint64_t)db << 32) | da);
        f32x4 tpv[NCG];
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg) {
          if constexpr (FMT == kFmtE5M2)
            tpv[cg] = __builtin_amdgcn_mfma_f32_16x16x32_bf8_fp8(
                vop8, (long)pop8[cg], f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
          else
            tpv[cg] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
                vop8, (long)pop8[cg], f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
        }
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[cg][blk][e] += fb[cg] * tpv[cg][e];
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // ---- key split: this partition's unnormalised partial (m, l, o) -------------
  // (an empty partition leaves m = -inf, l = 0, o = 0; a NaN l carries a NaN
  // m so the merge keeps it; the merge applies the static V scale)
  if (p.num_parts > 1) {
    // the workspace holds num_seqs * max_query_len rows (every row, when each
    // sequence has at most max_query_len of them)
    const int64_t ws_rows = (int64_t)p.num_seqs * p.max_query_len;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const float l = col_sum(l_run[cg]);
      if (!col_row[cg] || qrow[cg] >= ws_rows) continue;
      const int64_t slot =
          ((int64_t)qrow[cg] * p.num_q_heads + h * G + g) * p.num_parts + part;
      if (qd == 0) {
        p.ws_m[slot] = l != l ? __builtin_nanf("") : m_run[cg];
        p.ws_l[slot] = l;
      }
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int d;
          if constexpr (FP8) d = 64 * (blk / 4) + 16 * qd + 4 * e + (blk % 4);
          else d = 32 * (blk / 2) + 8 * qd + 2 * e + (blk % 2);
          p.ws_o[slot * D + d] = acc[cg][blk][e];
        }
      }
    }
    return;
  }

  // ---- output rows: o / l * s_v (rows at negative positions: zeros) ---------
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const float l = col_sum(l_run[cg]);
    if (!col_row[cg]) continue;
    const bool has = l > 0.0f || l != l;                 // NaN stays NaN
    const float scale = has ? vs / l : 0.0f;
    const int64_t orow = ((int64_t)qrow[cg] * p.num_q_heads + h * G + g) * D;
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int d;
        if constexpr (FP8) d = 64 * (blk / 4) + 16 * qd + 4 * e + (blk % 4);
        else d = 32 * (blk / 2) + 8 * qd + 2 * e + (blk % 2);
        const float r = has ? acc[cg][blk][e] * scale : 0.0f;
        if (p.out_bf16) reinterpret_cast<__bf16*>(p.out)[orow + d] = (__bf16)r;
        else reinterpret_cast<float*>(p.out)[orow + d] = r;
      }
    }
  }
}

namespace {

template <int D, int FMT, int NCG, bool DYN, bool ATT8>
hipError_t launch_prefill_shape(const PrefillParams& p, int64_t total, hipStream_t stream,
                                hipEvent_t ev_before, hipEvent_t ev_after) {
  const int64_t grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;   // no launch: too many blocks
  if (ev_before && ev_after) {
    hipExtLaunchKernelGGL((paged_prefill_kernel<D, FMT, NCG, DYN, ATT8>), dim3((unsigned)grid),
                          dim3(kPrefillWaves * kWave), 0, stream, ev_before, ev_after, 0, p);
  } else {
    hipLaunchKernelGGL((paged_prefill_kernel<D, FMT, NCG, DYN, ATT8>), dim3((unsigned)grid),
                       dim3(kPrefillWaves * kWave), 0, stream, p);
  }
  return hipGetLastError();
}

template <int D, int FMT, bool DYN, bool ATT8>
hipError_t launch_prefill_typed(PrefillParams p, const PrefillPlan& pl, hipStream_t stream,
                                hipEvent_t ev_before, hipEvent_t ev_after) {
  // column groups per wave the registers hold (at head dim 256: two with
  // the just-in-time codes of the static-scale, bf16-arithmetic instances;
  // a bf16 cache at head dim 128: three with them)
  constexpr int NCG_MAX = D >= 256 ? (prefill_jit<D, FMT, 2, DYN, ATT8>() ? 2 : 1) : 3;
  p.pos_per_block = pl.pos_per_block;
  p.qblocks = pl.qblocks;
  PrefillPlan plc = pl;
  if (plc.ncg > NCG_MAX) {
    // the plan allows two groups at head dim 256; the other instances there
    // hold one: fewer rows per work-group, more work-groups
    p.pos_per_block = pl.pos_per_block / pl.ncg * NCG_MAX;
    p.qblocks = (p.max_query_len + p.pos_per_block - 1) / p.pos_per_block;
    plc.ncg = NCG_MAX;
  }
  p.num_parts = pl.num_parts;
  p.part_tiles = pl.part_tiles;
  const int64_t total = (int64_t)p.num_seqs * p.num_kv_heads * p.qblocks * p.num_parts;
  if (total == 0) return hipSuccess;
  if (plc.ncg > NCG_MAX) return hipErrorInvalidValue;
  if constexpr (NCG_MAX >= 3) {
    if (plc.ncg == 3)
      return launch_prefill_shape<D, FMT, 3, DYN, ATT8>(p, total, stream, ev_before, ev_after);
  }
  if constexpr (NCG_MAX >= 2) {
    if (plc.ncg == 2)
      return launch_prefill_shape<D, FMT, 2, DYN, ATT8>(p, total, stream, ev_before, ev_after);
  }
  return launch_prefill_shape<D, FMT, 1, DYN, ATT8>(p, total, stream, ev_before, ev_after);
}

template <int D>
hipError_t launch_prefill_dim(const PrefillParams& p, const PrefillPlan& pl, int fmt, bool dyn,
                              bool att8, hipStream_t stream, hipEvent_t ev_before,
                              hipEvent_t ev_after) {
  if (dyn && att8) return hipErrorInvalidValue;
  if (dyn || att8) {
    switch (fmt) {
      case kFmtE4M3:
        return dyn ? launch_prefill_typed<D, kFmtE4M3, true, false>(p, pl, stream, ev_before,
                                                                     ev_after)
                   : launch_prefill_typed<D, kFmtE4M3, false, true>(p, pl, stream, ev_before,
                                                                     ev_after);
      case kFmtE5M2:
        return dyn ? launch_prefill_typed<D, kFmtE5M2, true, false>(p, pl, stream, ev_before,
                                                                     ev_after)
                   : launch_prefill_typed<D, kFmtE5M2, false, true>(p, pl, stream, ev_before,
                                                                     ev_after);
      default: return hipErrorInvalidValue;
    }
  }
  switch (fmt) {
    case kFmtBf16:
      return launch_prefill_typed<D, kFmtBf16, false, false>(p, pl, stream, ev_before,
                                                             ev_after);
    case kFmtE4M3:
      return launch_prefill_typed<D, kFmtE4M3, false, false>(p, pl, stream, ev_before,
                                                             ev_after);
    case kFmtE5M2:
      return launch_prefill_typed<D, kFmtE5M2, false, false>(p, pl, stream, ev_before,
                                                             ev_after);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_paged_prefill(const PrefillParams& p, const PrefillPlan& pl, int head_dim,
                                int fmt, bool dyn, bool att8, hipStream_t stream,
                                hipEvent_t ev_before, hipEvent_t ev_after) {
  if (p.group < 1 || p.group > 16) return hipErrorInvalidValue;
  if (pl.num_parts > 1 && (!p.ws_m || !p.ws_l || !p.ws_o)) return hipErrorInvalidValue;
  hipError_t e;
  switch (head_dim) {
    case 64: e = launch_prefill_dim<64>(p, pl, fmt, dyn, att8, stream, ev_before, ev_after); break;
    case 128: e = launch_prefill_dim<128>(p, pl, fmt, dyn, att8, stream, ev_before, ev_after); break;
    case 256: e = launch_prefill_dim<256>(p, pl, fmt, dyn, att8, stream, ev_before, ev_after); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || pl.num_parts <= 1) return e;
  // merge the partitions: FP32, the static V scale applied here (dynamic
  // scales are already in P; bf16 caches have none)
  DecodeParams dp{};
  dp.ws_m = p.ws_m;
  dp.ws_l = p.ws_l;
  dp.ws_o = p.ws_o;
  dp.out = p.out;
  dp.num_q_heads = p.num_q_heads;
  dp.num_kv_heads = p.num_kv_heads;
  dp.group = p.group;
  dp.num_parts = pl.num_parts;
  dp.scale_per_head = p.scale_per_head;
  dp.out_bf16 = p.out_bf16;
  dp.v_scale = (fmt != kFmtBf16 && !dyn) ? p.v_scale : nullptr;
  dp.row_limit = p.query_start + p.num_seqs;
  return launch_partition_merge(dp, head_dim, p.num_seqs * p.max_query_len, stream);
}

}  // namespace kvfp8
