// paged_decode.hpp - GQA decode attention over the paged FP8 (e4m3 or e5m2) or bf16
// KV cache on gfx950: a split kernel over context partitions and an FP32
// reduce kernel that merges the partitions.
//
// What is computed is softmax(q k^T) v over the attended positions with the
// online-softmax rescaling and FP32 two-level accumulation described in
// "State of FP8 KV cache and attention quantization in vLLM" (section "Kernel
// and vLLM improvements", paragraph "Two-level accumulation"; section
// "Single-request benchmark": online softmax rescaling). The FA3 Hopper
// kernels that post describes are prior art; this is a design for CDNA4:
//
//  * one wave streams a run of pages of one (sequence, KV head); every load is
//    a 16-byte-per-lane, 1 KiB-contiguous global load (the cache layout is
//    chosen so that the loaded registers already are MFMA operands);
//  * e4m3 codes expand exactly to bf16 in registers (gfx950 packed convert),
//    so q k^T runs on the 16x16x32 bf16 MFMA with q unrounded and products
//    exact; the K head scale, the softmax scale and log2(e) are applied to the
//    FP32 logits;
//  * the GQA group shares each K/V tile through the MFMA B operand: columns
//    0..G-1 carry the group's queries, columns G..2G-1 carry the same queries
//    again and receive the low half of P (P = hi + lo, both bf16), so P*V is
//    accurate to ~2^-17 at no extra MFMA cost (for G > 8 the 16 columns hold
//    queries and a second P*V MFMA takes the low halves);
//  * per 2-page tile the P*V MFMA result (level 1, FP32) is added to the FP32
//    running accumulator after the online-softmax rescale (level 2);
//  * the waves of a work-group merge their (m, l, o) through LDS; the reduce
//    kernel merges partitions in FP32 and applies the V head scale.
//
// The kernels are templates; paged_decode_d{64,128,256}.hip instantiate them
// for one head dimension each (separate compilation units, built in
// parallel) and paged_decode.hip dispatches.
#pragma once

#include <hip/hip_ext.h>
#include <math.h>
#include <stdlib.h>

#include "../../include/kvfp8.h"
#include "device_common.hpp"
#include "launch.hpp"

namespace kvfp8 {

// K/V pages are read exactly once per step: non-temporal loads keep them
// from displacing other lines in the caches (measured on MI355X: bf16 pages
// 97 -> 87 us, fp8 54 -> 52 us at 131072 positions).
typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p)));
}

// IEEE maximum (a NaN operand gives NaN): one v_maximum3_f32, with none of
// the input quieting that fmaxf needs on operands of unknown origin. A NaN
// logit makes its column's result NaN either way (its p is NaN).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Max over the four lanes c, c+16, c+32, c+48 that hold one MFMA column,
// with the gfx950 row swaps (VALU, no LDS round trip).
__device__ __forceinline__ float col_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

constexpr float kLazyLog2 = 8.0f;   // running max raised only past +8 (P <= 256)
constexpr int kFoldTiles = 4;       // level-1 P*V accumulation length in tiles
typedef float float2_t __attribute__((ext_vector_type(2)));

// Sum over the four lanes c, c+16, c+32, c+48 that hold one MFMA column (the
// row swaps give both lanes of a pair the same operands, so every lane of the
// column ends with the same value).
__device__ __forceinline__ float wave_sum_col(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---- LDS staging of K/V tiles -------------------------------------------------
// With SLOTS > 0 every wave owns a ring of SLOTS tile buffers in LDS and
// fills them with direct global->LDS loads (16 bytes per lane, 1 KiB per
// wave instruction, written at lane * 16 of the destination), so SLOTS tiles
// are in flight while the wave computes on the registers of the current one,
// at the register cost of a single tile. The compiler's wait insertion
// cannot tell the buffers apart and would wait for every outstanding load
// before any LDS read, so the reads of a staged tile are written as one
// instruction group that first waits for all but the loads issued after
// that tile (vmcnt) and ends by waiting for its own LDS reads (lgkmcnt).
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kAuxNonTemporal = 2;          // cache policy bit NT of the load
// The LDS address of a direct-to-LDS load comes from M0; on MI355X rings
// that reached past 64 KiB read back wrong data, so a ring stays below.
constexpr int kMaxLdsRing = 64 * 1024;

__device__ __forceinline__ void dma_1k(const uint8_t* src_wave_chunk, int lane, uint8_t* lds_dst) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)(src_wave_chunk + 16 * lane), (lds_void_t*)lds_dst,
                                   16, 0, kAuxNonTemporal);
}

// Four 1 KiB chunks at lds_addr + {0, 1, 2, 3} KiB (lds_addr includes lane*16),
// after waiting until at most PENDING vector-memory operations are
// outstanding.
template <int PENDING>
__device__ __forceinline__ void lds_read4(uint32_t lds_addr, uint4& a, uint4& b, uint4& c,
                                          uint4& d) {
  u32x4_t ra, rb, rc, rd;
  asm volatile(
      "s_waitcnt vmcnt(%4)\n\t"
      "ds_read_b128 %0, %5\n\t"
      "ds_read_b128 %1, %5 offset:1024\n\t"
      "ds_read_b128 %2, %5 offset:2048\n\t"
      "ds_read_b128 %3, %5 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(ra), "=v"(rb), "=v"(rc), "=v"(rd)
      : "n"(PENDING), "v"(lds_addr)
      : "memory");
  a = __builtin_bit_cast(uint4, ra);
  b = __builtin_bit_cast(uint4, rb);
  c = __builtin_bit_cast(uint4, rc);
  d = __builtin_bit_cast(uint4, rd);
}

// Four 16-byte LDS reads at lds_addr + {0, 64, 128, 192} once the loads that
// filled them are known to be complete (no vector-memory wait).
__device__ __forceinline__ void lds_read4_s64(uint32_t lds_addr, f32x4& a, f32x4& b, f32x4& c,
                                              f32x4& d) {
  u32x4_t ra, rb, rc, rd;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:64\n\t"
      "ds_read_b128 %2, %4 offset:128\n\t"
      "ds_read_b128 %3, %4 offset:192\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(ra), "=v"(rb), "=v"(rc), "=v"(rd)
      : "v"(lds_addr)
      : "memory");
  a = __builtin_bit_cast(f32x4, ra);
  b = __builtin_bit_cast(f32x4, rb);
  c = __builtin_bit_cast(f32x4, rc);
  d = __builtin_bit_cast(f32x4, rd);
}

// Bytes of a staged tile's scales in dynamic-scale mode: per page 16 rows of
// K scales and 16 of V scales (fp32).
constexpr int kTileScaleBytesPerPage = 2 * kPage * 4;

struct PartitionRange {
  int L, lo, first_page, end_page, num_parts_b;
};

// The partitions of one sequence: pages [first_page, end_page) cover the
// attended positions [lo, L); partition j holds part_pages pages of them.
__device__ __forceinline__ PartitionRange partition_range(const DecodeParams& p,
                                                          int b, int part_pages,
                                                          bool even_pages) {
  PartitionRange r;
  r.L = p.context_lens[b];
  if (r.L < 0 || p.num_pages <= 0) r.L = 0;         // no page can be valid without a pool
  r.lo = (p.window > 0 && r.L > p.window) ? r.L - p.window : 0;
  // Device-side values are never trusted to stay in bounds: positions past
  // the block-table row are ignored and partitions past the plan are dropped.
  if (r.L > p.max_pages_per_seq * kPage) r.L = p.max_pages_per_seq * kPage;
  if (r.lo > r.L) r.lo = r.L;
  r.first_page = r.lo / kPage;
  if (even_pages) r.first_page &= ~1;   // tiles on aligned 32-position blocks
  r.end_page = (r.L + kPage - 1) / kPage;
  const int n = r.end_page - r.first_page;
  r.num_parts_b = n > 0 ? (n + part_pages - 1) / part_pages : 0;
  if (r.num_parts_b > p.num_parts) r.num_parts_b = p.num_parts;
  return r;
}

template <int D, int FMT, int NW, int TP, int RING, int SLOTS, bool FUSED, bool ATT8, bool DYN,
          bool WIDE>
__global__ __launch_bounds__(NW * kWave) void paged_decode_split_kernel(
    const DecodeParams p) {
  constexpr bool FP8 = FMT != kFmtBf16;
  constexpr int E = FP8 ? 1 : 2;
  constexpr int PB = kPage * D * E;     // bytes of one (page, head) block
  constexpr int NI = PB / 1024;         // 1 KiB wave loads per page per tensor
  constexpr int NK = D / 32;            // q k^T MFMAs per page
  constexpr int NBLK = D / 16;          // P*V output blocks of 16 dims
  constexpr int GMAX = 16;              // query columns: G (+ G low halves of P)
  static_assert(!ATT8 || FP8, "the all-FP8 mode reads fp8 caches");
  static_assert(!DYN || (FP8 && !ATT8), "dynamic scales: fp8 caches, bf16 arithmetic");
  static_assert(!WIDE || !ATT8, "the all-FP8 mode has no low halves of P");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // Work-groups reach the XCDs round-robin in launch order (blockIdx.x
  // fastest), so partition x of every (sequence, KV head) runs on XCD x mod 8.
  // With p.rotate the partition index is rotated by the unit index, which
  // spreads the short or empty last partitions of a batch over the XCDs
  // (the plan decides; it is an ordering only, every partition still runs).
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  // (the grid is (num_parts, num_kv_heads, num_seqs): the sizes come from
  // the parameters, which arrive with the first kernel-argument load, rather
  // than from the dispatch's hidden arguments, a second dependent load)
  const int rot = p.rotate ? (int)(blockIdx.y + (unsigned)p.num_kv_heads * blockIdx.z) : 0;
  const int part = (int)((blockIdx.x + (unsigned)rot) % (unsigned)p.num_parts);
  const int G = p.group;
  const int qd = lane >> 4;             // row quad of the MFMA layout
  const int c = lane & 15;              // MFMA column
  const int part_pages = NW * p.pages_per_wave;

  // Column c < G: query c (high half of P); 8 <= c < 8 + G: query c - 8
  // (low half of P); other columns idle. The low half of query g sits 8
  // columns after its high half for every G <= 8, so the final fold of the
  // low columns into the high ones is one fixed DPP row shift. With G > 8
  // (wide) the 16 columns hold queries only, and P*V runs twice into the
  // same accumulator: once with the high halves, once with the low ones.
  // The all-FP8 mode has no low halves (P is e4m3 on purpose).
  constexpr bool wide = WIDE;           // G > 8 (the launcher picks the instance)
  constexpr bool has_lo = !ATT8 && !wide;
  const bool lo_col = has_lo && c >= 8 && c - 8 < G;
  const int g = c < G ? c : (lo_col ? c - 8 : -1);

  // Loads that do not depend on the context length go out before it is
  // known, so a work-group waits for one memory round trip, not two, before
  // its first page loads: the query operands and, for full attention (where
  // the run of pages starts at a fixed place), this wave's block-table slice.
  // q k^T B operand: lane (qd, c) holds query g's dims of K-slice s, in the
  // same order the K loads deliver them.
  bf16x8 qop[NK];
  {
    const uint16_t* qrow =
        p.q + ((int64_t)b * p.num_q_heads + h * G + (g < 0 ? 0 : g)) * D;
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const int d0 = FP8 ? 16 * (4 * (s / 2) + qd) + 8 * (s % 2) : 8 * (4 * s + qd);
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (g >= 0) w = *reinterpret_cast<const uint4*>(qrow + d0);
      qop[s] = bits_to_bf16x8(w);
    }
  }
  // All-FP8 mode: the query row as e4m3 codes (quantize_q_e4m3), run once
  // the first tile's loads are in flight, so it overlaps their latency.
  uint64_t qop8[ATT8 ? NK : 1];
  float q_scale = 1.0f;
  auto quantize_q = [&]() {
    if constexpr (ATT8) q_scale = quantize_q_e4m3<NK>(qop, qop8);
  };
  // static scales: one per head or tensor; dynamic ones are per position
  // (the pools p.k_scale / p.v_scale [page][head][row]), applied per row
  const float ks = FP8 && !DYN ? p.k_scale[p.scale_per_head ? h : 0] : 1.0f;
  const float vs = FP8 && !DYN ? p.v_scale[p.scale_per_head ? h : 0] : 1.0f;
  const int32_t* bt_row = p.block_tables + (int64_t)b * p.max_pages_per_seq;
  int my_page = -1;
  if (p.window == 0) {
    const int idx = part * part_pages + wave * p.pages_per_wave + lane;
    if (lane < p.pages_per_wave && idx < p.max_pages_per_seq) my_page = bt_row[idx];
  }

  const PartitionRange pr = partition_range(p, b, part_pages, ATT8);
  if (part >= pr.num_parts_b) {
    // Nothing to attend here. In direct mode the first partition still owns
    // the output rows (empty context -> zeros); otherwise the partition's
    // slots get an empty partial (m = -inf, l = 0; o is never read), so the
    // reduce kernel can merge every planned partition without the length.
    if (p.direct) {
      if (part == 0) {
        for (int i = threadIdx.x; i < G * D; i += NW * kWave) {
          const int64_t o = ((int64_t)b * p.num_q_heads + h * G + i / D) * D + i % D;
          if (p.out_bf16) reinterpret_cast<__bf16*>(p.out)[o] = (__bf16)0.0f;
          else reinterpret_cast<float*>(p.out)[o] = 0.0f;
        }
      }
    } else if ((int)threadIdx.x < G) {
      const int64_t slot = ((int64_t)b * p.num_q_heads + h * G + threadIdx.x) * p.num_parts + part;
      p.ws_m[slot] = -INFINITY;
      p.ws_l[slot] = 0.0f;
    }
    return;
  }

  // This wave's run of pages. A partial (last) partition spreads its pages
  // evenly over the work-group's waves, so its waves - among them the one
  // holding the newest position - finish early instead of two running full.
  const int part_start = pr.first_page + part * part_pages;
  const int part_end = min(part_start + part_pages, pr.end_page);
  int ppw = p.pages_per_wave;
  if (part_end - part_start < part_pages)
    ppw = min(ppw, (((part_end - part_start) + NW - 1) / NW + 1) & ~1);
  const int wbeg = part_start + wave * ppw;
  const int wend = min(wbeg + ppw, part_end);
  const int npages = wend > wbeg ? wend - wbeg : 0;

  // Page ids of this wave's run, one per lane. The early read holds them
  // when the run starts where it was guessed (full attention, full
  // partition); a window or a partial partition reads them now.
  if (p.window != 0 || ppw != p.pages_per_wave) {
    my_page = -1;
    if (lane < npages) my_page = bt_row[wbeg + lane];
  } else if (lane >= npages) {
    my_page = -1;
  }
  if (my_page < 0 || (int64_t)my_page >= p.num_pages) my_page = -1;   // empty page
  const uint64_t bad_pages = __ballot(my_page < 0 && lane < npages);
  // what a tile loads for page index idx: the page, or pool page 0 for a
  // missing or invalid one (its positions are masked)
  const int page_or0 = my_page < 0 ? 0 : my_page;

  // Per-wave LDS region: the tile ring while streaming, then the wave's
  // unnormalised output rows for the merge (written after the wave's last
  // staged tile has been read, so no load is still landing there).
  constexpr int KV_BYTES = TP * 2 * PB;               // K and V of TP pages
  constexpr int TILE_BYTES = KV_BYTES + (DYN ? TP * kTileScaleBytesPerPage : 0);
  constexpr int LPT = TP * 2 * NI;                    // 1 KiB loads per tile
  constexpr int VPT = LPT + (DYN ? 1 : 0);            // vector-memory ops per staged tile
  constexpr int O_BYTES = GMAX * D * 4;
  constexpr int REGION = (SLOTS * TILE_BYTES > O_BYTES) ? SLOTS * TILE_BYTES : O_BYTES;
  static_assert(LPT % 4 == 0, "staged tiles are read in groups of four 1 KiB chunks");
  static_assert(SLOTS == 0 || NW * REGION <= kMaxLdsRing,
                "direct-to-LDS loads address the first 64 KiB only");
  // One LDS block, so the ring starts at address 0: the per-wave regions,
  // then the waves' m and l, then the staged new rows of the fused step.
  constexpr int M_OFF = NW * REGION;
  constexpr int L_OFF = M_OFF + NW * GMAX * 4;
  constexpr int NEW_OFF = L_OFF + NW * GMAX * 4;
  constexpr int SMEM_BYTES = NEW_OFF + (FUSED ? 2 * D * E : 16);
  __shared__ __align__(16) uint8_t smem[SMEM_BYTES];
  uint8_t* const my_region = smem + wave * REGION;
  float (*const sm_m)[GMAX] = reinterpret_cast<float (*)[GMAX]>(smem + M_OFF);
  float (*const sm_l)[GMAX] = reinterpret_cast<float (*)[GMAX]>(smem + L_OFF);
  uint8_t* const new_rows = smem + NEW_OFF;

  const int64_t page_stride = (int64_t)p.num_kv_heads * PB;
  const uint8_t* kbase = p.k_cache + (int64_t)h * PB;
  const uint8_t* vbase = p.v_cache + (int64_t)h * PB;
  float c_log2 = ks * p.sm_scale_log2;              // times q_scale in the all-FP8 mode

  // ---- fused decode step: the cache write of position L-1 -----------------
  // Exactly one wave streams the page that holds the newest position of this
  // (sequence, KV head). That wave quantises the new K and V rows (the same
  // arithmetic as the cache-write kernel), stores them into the cache and
  // keeps the stored bytes in LDS; when it reaches that page it patches them
  // into its tile registers. No other wave reads that page, so no ordering
  // across waves is needed, and the page load never has to observe the store.
  int t_new = -1, pg_new = 0, r_new = 0;
  int idx_new = -1;
  if constexpr (FUSED) {
    const int pos = pr.L - 1;
    const int pn = pos >= 0 ? pos / kPage : -1;
    if (pn >= wbeg && pn < wend && !((bad_pages >> (pn - wbeg)) & 1ull)) {
      idx_new = pn - wbeg;
      t_new = idx_new / TP;
      pg_new = idx_new % TP;
      r_new = pos % kPage;
    }
  }
  // The owning wave issues the loads of the new rows before its first tiles'
  // loads (lane j holds dims VPL*j .. VPL*j+VPL-1 of K and of V, so the whole
  // wave shares the quantisation) and quantises and stages them in LDS right
  // after: memory operations retire in order, so waiting for the rows does
  // not wait for the tiles, and the conversion overlaps their latency. The
  // global stores of the new rows go out only after the wave's last tile:
  // stores count in the same vector-memory counter as loads, so a store
  // issued before the stream would make the wave's first tile wait for the
  // store's write acknowledgement as well (a second memory round trip on the
  // path of the work-group that holds the newest position).
  constexpr int VPL = D / kWave;
  uint32_t kx_new[(VPL + 1) / 2] = {}, vx_new[(VPL + 1) / 2] = {};
  auto fused_prefetch = [&]() {
    if constexpr (FUSED) {
      if (t_new < 0) return;
      const int64_t src = ((int64_t)b * p.num_kv_heads + h) * D + VPL * lane;
      if constexpr (VPL == 1) {
        kx_new[0] = p.k_new[src];
        vx_new[0] = p.v_new[src];
      } else {
#pragma unroll
        for (int i = 0; i < VPL / 2; ++i) {
          kx_new[i] = reinterpret_cast<const uint32_t*>(p.k_new + src)[i];
          vx_new[i] = reinterpret_cast<const uint32_t*>(p.v_new + src)[i];
        }
      }
    }
  };
  float sk_new = 1.0f, sv_new = 1.0f;   // dynamic scales of the new row
  // the new rows' stored form (codes, or bf16 bits), kept for the late stores
  uint16_t kst[FUSED ? VPL : 1] = {}, vst[FUSED ? VPL : 1] = {};
  auto fused_commit = [&]() {
    if constexpr (FUSED) {
      const int d0 = VPL * lane;
      uint16_t kb[VPL], vb[VPL];
#pragma unroll
      for (int e = 0; e < VPL; ++e) {
        kb[e] = (uint16_t)(kx_new[e / 2] >> (16 * (e % 2)));
        vb[e] = (uint16_t)(vx_new[e / 2] >> (16 * (e % 2)));
      }
      if constexpr (FP8) {
        float sk = ks, sv = vs;
        if constexpr (DYN) {
          // the token's own scales, as the dynamic cache write takes them:
          // integer max of the bf16 magnitude bits (NaN > Inf > finite) over
          // this head's row, or over every head's row of the token
          uint32_t km = 0u, vm = 0u;
#pragma unroll
          for (int e = 0; e < VPL; ++e) {
            km = max(km, (uint32_t)kb[e] & 0x7FFFu);
            vm = max(vm, (uint32_t)vb[e] & 0x7FFFu);
          }
          if (p.dyn_all_heads) {
            // the token's whole K and V rows (all heads) in 16-byte chunks,
            // two per lane in flight at a time
            const int nch = p.num_kv_heads * (D / 8);
            const uint4* kr = reinterpret_cast<const uint4*>(p.k_new + (int64_t)b * p.num_kv_heads * D);
            const uint4* vr = reinterpret_cast<const uint4*>(p.v_new + (int64_t)b * p.num_kv_heads * D);
            for (int base = 0; base < nch; base += 2 * kWave) {
              uint4 kc[2], vc[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const int j = base + u * kWave + lane;
                kc[u] = j < nch ? kr[j] : make_uint4(0u, 0u, 0u, 0u);
                vc[u] = j < nch ? vr[j] : make_uint4(0u, 0u, 0u, 0u);
              }
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const uint32_t kw4[4] = {kc[u].x, kc[u].y, kc[u].z, kc[u].w};
                const uint32_t vw4[4] = {vc[u].x, vc[u].y, vc[u].z, vc[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  km = max(km, max(kw4[i] & 0x7FFFu, (kw4[i] >> 16) & 0x7FFFu));
                  vm = max(vm, max(vw4[i] & 0x7FFFu, (vw4[i] >> 16) & 0x7FFFu));
                }
              }
            }
          }
#pragma unroll
          for (int off = kWave / 2; off > 0; off /= 2) {
            km = max(km, (uint32_t)__shfl_xor((int)km, off));
            vm = max(vm, (uint32_t)__shfl_xor((int)vm, off));
          }
          constexpr float fmax = FMT == kFmtE5M2 ? 57344.0f : 448.0f;
          const float ak = bf16_bits_to_f32(km), av = bf16_bits_to_f32(vm);
          sk = ak == 0.0f ? 1.0f : ak / fmax;
          sv = av == 0.0f ? 1.0f : av / fmax;
          sk_new = sk;
          sv_new = sv;
        }
        uint8_t kq[VPL], vq[VPL];
#pragma unroll
        for (int e = 0; e < VPL; ++e) {
          kq[e] = (uint8_t)fp8_encode_sat<FMT>(bf16_bits_to_f32(kb[e]) / sk);
          vq[e] = (uint8_t)fp8_encode_sat<FMT>(bf16_bits_to_f32(vb[e]) / sv);
        }
#pragma unroll
        for (int e = 0; e < VPL; ++e) {
          new_rows[d0 + e] = kq[e];
          new_rows[D + d0 + e] = vq[e];
          kst[e] = kq[e];
          vst[e] = vq[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < VPL; ++e) {
          reinterpret_cast<uint16_t*>(new_rows)[d0 + e] = kb[e];
          reinterpret_cast<uint16_t*>(new_rows)[D + d0 + e] = vb[e];
          kst[e] = kb[e];
          vst[e] = vb[e];
        }
      }
    }
  };
  // The new rows (and, with dynamic scales, their scales) into the caches:
  // after the wave's last tile, so no tile waits for these stores.
  auto fused_store = [&]() {
    if constexpr (FUSED) {
      const int pid = __builtin_amdgcn_readlane(my_page, idx_new);
      uint8_t* kblk = const_cast<uint8_t*>(p.k_cache) + ((int64_t)pid * p.num_kv_heads + h) * PB;
      uint8_t* vblk = const_cast<uint8_t*>(p.v_cache) + ((int64_t)pid * p.num_kv_heads + h) * PB;
      const int d0 = VPL * lane;
      // K: the lane's dims are adjacent in one 16-byte chunk; V: 4 bytes apart
#pragma unroll
      for (int e = 0; e < VPL; ++e) {
        if constexpr (FP8) {
          kblk[k_byte<1>(r_new, d0 + e)] = (uint8_t)kst[e];
          vblk[v_byte<1>(r_new, d0 + e)] = (uint8_t)vst[e];
        } else {
          *reinterpret_cast<uint16_t*>(kblk + k_byte<2>(r_new, d0 + e)) = kst[e];
          *reinterpret_cast<uint16_t*>(vblk + v_byte<2>(r_new, d0 + e)) = vst[e];
        }
      }
      if constexpr (DYN) {
        if (lane == 0) {
          const int64_t so = ((int64_t)pid * p.num_kv_heads + h) * kPage + r_new;
          const_cast<float*>(p.k_scale)[so] = sk_new;
          const_cast<float*>(p.v_scale)[so] = sv_new;
        }
      }
    }
  };

  // Online softmax state per column (log2 domain). The running max is raised
  // lazily - only when a tile's max exceeds it by more than kLazyLog2 - so
  // most tiles need no rescale and P stays below 2^kLazyLog2. P*V is
  // accumulated in two FP32 levels: the MFMA accumulator `lvl1` (level 1)
  // takes up to kFoldTiles tiles, then is added into `acc` (level 2); a
  // rescale folds first.
  float m_run = -INFINITY;
  float l_run = 0.0f;
  f32x4 acc[NBLK], lvl1[NBLK];
#pragma unroll
  for (int i = 0; i < NBLK; ++i) {
    acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    lvl1[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  auto fold = [&]() {
#pragma unroll
    for (int i = 0; i < NBLK; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][e] += lvl1[i][e];
      lvl1[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };

  // A tile is TP pages (an even number: the P*V MFMA contracts 32 positions,
  // two pages). Missing pages (past the run, an odd tail) and invalid ids
  // load pool page 0 instead: their positions are masked, so the values never
  // matter, and the registers never hold uninitialised data.
  struct Tile {
    uint4 k[TP][NI];
    uint4 v[TP][NI];
    f32x4 sk[DYN ? TP : 1];     // dynamic scales of rows 4qd..4qd+3 of each page
    f32x4 sv[DYN ? TP : 1];
  };
  const int64_t scale_row0 = (int64_t)h * kPage + 4 * qd;   // in a pool page: [head][row]

  auto load_tile = [&](int t, Tile& tl) {
#pragma unroll
    for (int pg = 0; pg < TP; ++pg) {
      const int idx = TP * t + pg;
      const int pid = __builtin_amdgcn_readlane(page_or0, idx & (kWave - 1));
      const uint4* kp = reinterpret_cast<const uint4*>(kbase + (int64_t)pid * page_stride);
      const uint4* vp = reinterpret_cast<const uint4*>(vbase + (int64_t)pid * page_stride);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        tl.k[pg][i] = load_stream(kp + i * kWave + lane);
        tl.v[pg][i] = load_stream(vp + i * kWave + lane);
      }
      if constexpr (DYN) {
        const int64_t so = (int64_t)pid * p.num_kv_heads * kPage + scale_row0;
        tl.sk[pg] = *reinterpret_cast<const f32x4*>(p.k_scale + so);
        tl.sv[pg] = *reinterpret_cast<const f32x4*>(p.v_scale + so);
      }
    }
  };

  // Replace row r_new of page pg_new in the tile registers by the bytes
  // stored for the newest position (fused decode step).
  auto patch_tile = [&](Tile& tl) {
    const uint8_t* kr = new_rows;
    const uint8_t* vr = new_rows + D * E;
#pragma unroll
    for (int pg = 0; pg < TP; ++pg) {
      if (pg != pg_new) continue;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        // K: lane (qd, c) holds row c, 16-byte chunk 4i + qd of the row
        if (c == r_new) tl.k[pg][i] = *reinterpret_cast<const uint4*>(kr + 16 * (4 * i + qd));
        // V: lane (qd, c) holds rows 4qd..4qd+3 of 16/(4E) dims
        if (qd == r_new / 4) {
          uint4 w = tl.v[pg][i];
          if constexpr (FP8) {
            const uint32_t nv = *reinterpret_cast<const uint32_t*>(vr + 64 * i + 4 * c);
            const int sh = 8 * (r_new % 4);
            const uint32_t m = ~(0xFFu << sh);
            w.x = (w.x & m) | (((nv >> 0) & 0xFFu) << sh);
            w.y = (w.y & m) | (((nv >> 8) & 0xFFu) << sh);
            w.z = (w.z & m) | (((nv >> 16) & 0xFFu) << sh);
            w.w = (w.w & m) | (((nv >> 24) & 0xFFu) << sh);
          } else {
            const uint32_t nv = *reinterpret_cast<const uint32_t*>(vr + 2 * (32 * i + 2 * c));
            const int sh = 16 * (r_new % 2);
            const uint32_t m = ~(0xFFFFu << sh);
            const uint32_t d0 = nv & 0xFFFFu, d1 = nv >> 16;
            if ((r_new % 4) < 2) {
              w.x = (w.x & m) | (d0 << sh);
              w.z = (w.z & m) | (d1 << sh);
            } else {
              w.y = (w.y & m) | (d0 << sh);
              w.w = (w.w & m) | (d1 << sh);
            }
          }
          tl.v[pg][i] = w;
        }
      }
      if constexpr (DYN) {
        if (qd == r_new / 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (e == r_new % 4) {
              tl.sk[pg][e] = sk_new;
              tl.sv[pg][e] = sv_new;
            }
          }
        }
      }
    }
  };

  auto compute_tile = [&](int t, const Tile& tl) {
    // ---- logits: S^T[row 4qd+e][col c] for every page of the tile --------
    float x[TP][4];
#pragma unroll
    for (int pg = 0; pg < TP; ++pg) {
      f32x4 sacc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        if constexpr (ATT8) {
          // the K codes themselves are the operand (fp8 x fp8 MFMA)
          const uint4 w = tl.k[pg][s / 2];
          const long kop8 = (long)((s % 2 == 0) ? (((uint64_t)w.y << 32) | w.x)
                                                : (((uint64_t)w.w << 32) | w.z));
          if constexpr (FMT == kFmtE5M2)
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf8_fp8(kop8, (long)qop8[s], sacc, 0, 0, 0);
          else
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(kop8, (long)qop8[s], sacc, 0, 0, 0);
          continue;
        }
        bf16x8 kop;
        if constexpr (FP8) {
          const uint4 w = tl.k[pg][s / 2];
          kop = (s % 2 == 0) ? fp8x8_to_bf16x8<FMT>(w.x, w.y) : fp8x8_to_bf16x8<FMT>(w.z, w.w);
        } else {
          kop = bits_to_bf16x8(tl.k[pg][s]);
        }
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[s], sacc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) x[pg][e] = sacc[e] * c_log2;
      if constexpr (DYN) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[pg][e] *= tl.sk[pg][e];
      }
    }
    // ---- masking: positions outside [lo, L), past the run, invalid pages --
    // (wave-uniform decision; only boundary tiles take it)
    const int pos0 = (wbeg + TP * t) * kPage;           // first position of the tile
    const uint64_t tile_bits = ((1ull << TP) - 1ull) << (TP * t);
    const uint64_t run_bits = npages >= 64 ? ~0ull : ((1ull << npages) - 1ull);
    const bool any_missing = ((tile_bits & ~run_bits) | (tile_bits & bad_pages)) != 0ull;
    const bool need_mask = (pos0 < pr.lo) || (pos0 + TP * kPage > pr.L) || any_missing;
    // masked V rows: per 32-position MFMA, AND masks for the four packed
    // bf16 pairs of the operand (set, and used, only on boundary tiles)
    uint32_t vmask[TP / 2][4];
    uint32_t vmask8[TP];                                 // all-FP8 mode: byte masks per page
    if (need_mask) {
      uint32_t vkeep = 0u;                               // bit 4*pg+e: row 4qd+e of page pg
#pragma unroll
      for (int pg = 0; pg < TP; ++pg) {
        const int idx = TP * t + pg;
        const bool page_ok = idx < npages && !((bad_pages >> idx) & 1ull);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pos = pos0 + pg * kPage + 4 * qd + e;
          const bool ok = page_ok && pos >= pr.lo && pos < pr.L;
          if (!ok) x[pg][e] = -INFINITY;
          vkeep |= (ok ? 1u : 0u) << (4 * pg + e);
        }
      }
      if constexpr (ATT8) {
#pragma unroll
        for (int pg = 0; pg < TP; ++pg) {
          uint32_t m8 = 0u;
#pragma unroll
          for (int e = 0; e < 4; ++e) m8 |= ((vkeep >> (4 * pg + e)) & 1u) ? (0xFFu << (8 * e)) : 0u;
          vmask8[pg] = m8;
        }
      } else {
#pragma unroll
        for (int pp = 0; pp < TP / 2; ++pp) {
          const uint32_t kk = vkeep >> (8 * pp);
#pragma unroll
          for (int k2 = 0; k2 < 4; ++k2)
            vmask[pp][k2] = (((kk >> (2 * k2)) & 1u) ? 0x0000FFFFu : 0u) |
                            (((kk >> (2 * k2 + 1)) & 1u) ? 0xFFFF0000u : 0u);
        }
      }
    }
    // ---- online softmax (log2 domain), lazy rescale -----------------------
    float tmax = x[0][0];
#pragma unroll
    for (int pg = 0; pg < TP; ++pg)
#pragma unroll
      for (int e = 0; e < 4; ++e) tmax = vmax(tmax, x[pg][e]);
    tmax = col_max(tmax);
    const bool grow = tmax > m_run + kLazyLog2;          // -inf > -inf is false
    if (__builtin_amdgcn_ballot_w64(grow) != 0ull) {
      if constexpr (!ATT8) fold();
      const float m_new = grow ? tmax : m_run;
      const float alpha = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < NBLK; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][e] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
    if constexpr (ATT8) {
      // ---- all-FP8 P*V: P of this 32-position block quantised to e4m3
      // relative to the block's own max (tmax), the fp8 MFMA product rescaled
      // by 2^(tmax - m) into the FP32 running sum (level 2, every tile) ------
      const bool live = tmax != -INFINITY;
      const float mb = live ? tmax : 0.0f;
      const float fb = live ? __builtin_amdgcn_exp2f(tmax - m_use) : 0.0f;
      float ps = -0.0f;                  // -0 + p is p: no add for the first term
      uint32_t pw[TP];
#pragma unroll
      for (int pg = 0; pg < TP; ++pg) {
        float pe[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pe[e] = __builtin_amdgcn_exp2f(x[pg][e] - mb);
        ps += (pe[0] + pe[1]) + (pe[2] + pe[3]);
        // e4m3 codes, round to nearest even (the hardware conversion agrees
        // with the cache codec on every input in [0, 1])
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(pe[0], pe[1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(pe[2], pe[3], w, true);
        pw[pg] = (uint32_t)w;
      }
      l_run += fb * ps;
      // every block's product first, then the folds: the MFMAs issue back to
      // back and each fold finds its result ready
      f32x4 tpv[NBLK];
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
        tpv[blk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int pp = 0; pp < TP / 2; ++pp) {
          const int i = blk / 4, ep = blk % 4;
          const uint4 wa = tl.v[2 * pp][i], wb = tl.v[2 * pp + 1][i];
          uint32_t da = ep == 0 ? wa.x : ep == 1 ? wa.y : ep == 2 ? wa.z : wa.w;
          uint32_t db = ep == 0 ? wb.x : ep == 1 ? wb.y : ep == 2 ? wb.z : wb.w;
          if (need_mask) {
            da &= vmask8[2 * pp];
            db &= vmask8[2 * pp + 1];
          }
          const long vop = (long)(((uint64_t)db << 32) | da);
          const long pop8 = (long)(((uint64_t)pw[2 * pp + 1] << 32) | pw[2 * pp]);
          if constexpr (FMT == kFmtE5M2)
            tpv[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf8_fp8(vop, pop8, tpv[blk], 0, 0, 0);
          else
            tpv[blk] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(vop, pop8, tpv[blk], 0, 0, 0);
        }
      }
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[blk][e] += fb * tpv[blk][e];
      return;
    }
    float psum_pg[TP];
    bf16x8 pop[TP / 2], pop_lo[TP / 2];    // pop_lo: wide mode only
#pragma unroll
    for (int pg = 0; pg < TP; ++pg) {
      float u[4], ulo[4], pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pe = __builtin_amdgcn_exp2f(x[pg][e] - m_use);
        pv[e] = pe;
        // dynamic scales: the row's V scale joins P (masked rows stay 0
        // whatever their pool entry holds)
        float pw = pe;
        if constexpr (DYN) pw = pe == 0.0f ? 0.0f : pe * tl.sv[pg][e];
        // P = hi + lo: hi is pw truncated to bf16 (query columns), lo the
        // exact residue, rounded to bf16 (duplicate columns)
        const float hi = __uint_as_float(__float_as_uint(pw) & 0xFFFF0000u);
        u[e] = lo_col ? pw - hi : hi;
        ulo[e] = pw - hi;
      }
      psum_pg[pg] = (pv[0] + pv[1]) + (pv[2] + pv[3]);
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const bf16x2 v2 = __builtin_convertvector((float2_t){u[e], u[e + 1]}, bf16x2);
        pop[pg / 2][4 * (pg % 2) + e] = v2[0];
        pop[pg / 2][4 * (pg % 2) + e + 1] = v2[1];
      }
      if constexpr (wide) {
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const bf16x2 v2 = __builtin_convertvector((float2_t){ulo[e], ulo[e + 1]}, bf16x2);
          pop_lo[pg / 2][4 * (pg % 2) + e] = v2[0];
          pop_lo[pg / 2][4 * (pg % 2) + e + 1] = v2[1];
        }
      }
    }
    float psum = psum_pg[0];
#pragma unroll
    for (int pg = 1; pg < TP; ++pg) psum += psum_pg[pg];
    l_run += psum;
    // ---- P*V: TP/2 chained k=32 MFMAs per 16-dim block into level 1 -------
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
#pragma unroll
      for (int pp = 0; pp < TP / 2; ++pp) {
        uint4 vb;
        if constexpr (FP8) {
          const int i = blk / 4, ep = blk % 4;
          const uint4 wa = tl.v[2 * pp][i], wb = tl.v[2 * pp + 1][i];
          const uint32_t da = ep == 0 ? wa.x : ep == 1 ? wa.y : ep == 2 ? wa.z : wa.w;
          const uint32_t db = ep == 0 ? wb.x : ep == 1 ? wb.y : ep == 2 ? wb.z : wb.w;
          vb = __builtin_bit_cast(uint4, cat(fp8x4_to_bf16x4<FMT>(da), fp8x4_to_bf16x4<FMT>(db)));
        } else {
          const int i = blk / 2, ep = blk % 2;
          const uint4 wa = tl.v[2 * pp][i], wb = tl.v[2 * pp + 1][i];
          vb = ep == 0 ? make_uint4(wa.x, wa.y, wb.x, wb.y) : make_uint4(wa.z, wa.w, wb.z, wb.w);
        }
        if (need_mask) {
          // zero the bf16 values of masked rows (poison codes are NaN)
          vb.x &= vmask[pp][0]; vb.y &= vmask[pp][1];
          vb.z &= vmask[pp][2]; vb.w &= vmask[pp][3];
        }
        lvl1[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bits_to_bf16x8(vb), pop[pp], lvl1[blk],
                                                            0, 0, 0);
        if constexpr (wide)
          lvl1[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bits_to_bf16x8(vb), pop_lo[pp],
                                                              lvl1[blk], 0, 0, 0);
      }
    }
    // ---- level 2: every kFoldTiles tiles ----------------------------------
    if (t % kFoldTiles == kFoldTiles - 1) fold();
  };

  const int ntiles = (npages + TP - 1) / TP;
  if constexpr (SLOTS > 0) {
    // ---- LDS ring: tile t lives in slot t % SLOTS ------------------------------
    // chunk q of a slot: page q / (2 NI), K (then V) chunk q % NI
    auto stage_tile = [&](int t, int slot) {
      uint8_t* dst = my_region + slot * TILE_BYTES;
      if constexpr (DYN) {
        // lane l < 8 TP: page l / 8, K (l % 8 < 4) or V scales, rows 4(l % 4)..+3;
        // issued first, so the tile's K/V wait covers it
        if (lane < 8 * TP) {
          static_assert(TP == 2, "the scale loads cover two pages");
          const int pid0 = __builtin_amdgcn_readlane(page_or0, (TP * t) & (kWave - 1));
          const int pid1 = __builtin_amdgcn_readlane(page_or0, (TP * t + 1) & (kWave - 1));
          const int pid = lane < 8 ? pid0 : pid1;
          const float* pool = (lane % 8) < 4 ? p.k_scale : p.v_scale;
          const float* src = pool + (int64_t)pid * p.num_kv_heads * kPage + (int64_t)h * kPage +
                             4 * (lane % 4);
          __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)(dst + KV_BYTES), 16, 0,
                                           0);
        }
      }
#pragma unroll
      for (int pg = 0; pg < TP; ++pg) {
        const int idx = TP * t + pg;
        const int pid = __builtin_amdgcn_readlane(page_or0, idx & (kWave - 1));
        const uint8_t* kp = kbase + (int64_t)pid * page_stride;
        const uint8_t* vp = vbase + (int64_t)pid * page_stride;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          dma_1k(kp + 1024 * i, lane, dst + 1024 * (2 * NI * pg + i));
          dma_1k(vp + 1024 * i, lane, dst + 1024 * (2 * NI * pg + NI + i));
        }
      }
    };
    // Reads slot `slot` into registers once at most `later` tiles issued after
    // it are still outstanding.
    auto read_tile = [&](int slot, int later, Tile& tl) {
      const uint32_t base =
          (uint32_t)(uintptr_t)(lds_void_t*)(my_region + slot * TILE_BYTES) + 16u * lane;
      uint4 ch[LPT];
#pragma unroll
      for (int j = 0; j < LPT / 4; ++j) {
        const uint32_t a = base + 4096u * j;
        if (later >= 2 && SLOTS >= 3)
          lds_read4<2 * VPT>(a, ch[4 * j], ch[4 * j + 1], ch[4 * j + 2], ch[4 * j + 3]);
        else if (later >= 1 && SLOTS >= 2)
          lds_read4<VPT>(a, ch[4 * j], ch[4 * j + 1], ch[4 * j + 2], ch[4 * j + 3]);
        else
          lds_read4<0>(a, ch[4 * j], ch[4 * j + 1], ch[4 * j + 2], ch[4 * j + 3]);
      }
#pragma unroll
      for (int pg = 0; pg < TP; ++pg)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          tl.k[pg][i] = ch[2 * NI * pg + i];
          tl.v[pg][i] = ch[2 * NI * pg + NI + i];
        }
      if constexpr (DYN) {
        static_assert(TP == 2, "the scale reads cover two pages");
        const uint32_t sb = (uint32_t)(uintptr_t)(lds_void_t*)(my_region + slot * TILE_BYTES +
                                                               KV_BYTES) + 16u * qd;
        lds_read4_s64(sb, tl.sk[0], tl.sv[0], tl.sk[1], tl.sv[1]);
      }
    };
    Tile t0;
    fused_prefetch();
#pragma unroll
    for (int sl = 0; sl < SLOTS; ++sl)
      if (sl < ntiles) stage_tile(sl, sl);
    if (t_new >= 0) fused_commit();
    quantize_q();
    c_log2 *= q_scale;
    for (int t = 0; t < ntiles; ++t) {
      // tiles issued after tile t (no store is outstanding in the loop)
      const int later = min(ntiles, t + SLOTS) - (t + 1);
      read_tile(t % SLOTS, later, t0);
      if (t + SLOTS < ntiles) stage_tile(t + SLOTS, t % SLOTS);
      if (FUSED && t == t_new) patch_tile(t0);
      compute_tile(t, t0);
    }
  } else if constexpr (RING == 2) {
    // ---- register ring of two tiles: one in flight while one is computed
    Tile t0, t1;
    fused_prefetch();
    if (ntiles > 0) load_tile(0, t0);
    if (t_new >= 0) fused_commit();
    quantize_q();
    c_log2 *= q_scale;
    for (int t = 0; t < ntiles; t += 2) {
      if (t + 1 < ntiles) load_tile(t + 1, t1);
      if (FUSED && t == t_new) patch_tile(t0);
      compute_tile(t, t0);
      if (t + 1 >= ntiles) break;
      if (t + 2 < ntiles) load_tile(t + 2, t0);
      if (FUSED && t + 1 == t_new) patch_tile(t1);
      compute_tile(t + 1, t1);
    }
  } else {
    Tile t0;
    fused_prefetch();
    if (ntiles > 0) load_tile(0, t0);
    if (t_new >= 0) fused_commit();
    quantize_q();
    c_log2 *= q_scale;
    for (int t = 0; t < ntiles; ++t) {
      if (t > 0) load_tile(t, t0);
      if (FUSED && t == t_new) patch_tile(t0);
      compute_tile(t, t0);
    }
  }

  if (FUSED && t_new >= 0) fused_store();
  if constexpr (!ATT8) fold();
  // ---- per-wave results: l over the row quads, lo columns into hi ----------
  l_run = wave_sum_col(l_run);
  // A NaN logit (a NaN query element or cache code) leaves l NaN but may
  // never raise the running max; carry it in m so the merges keep it.
  if (l_run != l_run) m_run = __builtin_nanf("");
  if constexpr (has_lo) {
    // column c + 8 (the low half of query c) into column c: DPP row_shl:8
    // within each 16-lane row (the MFMA column index is lane % 16)
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[blk][e] += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc[blk][e]),
                                                               0x108, 0xF, 0xF, true));
  }

  // The wave's unnormalised rows into LDS, 16 bytes at a time: lane (qd, c)
  // holds 4 consecutive dims for each (block group, e) (fp8 layout: dims
  // 64 i + 16 qd + 4 e + r from acc[4 i + r][e]; bf16 layout: dims
  // 32 i + 8 qd + 4 j + r' from acc[2 i + (r' % 2)][2 j + r' / 2]).
  if (c < G) {
    if (qd == 0) {
      sm_m[wave][c] = m_run;
      sm_l[wave][c] = l_run;
    }
    float* const orow = reinterpret_cast<float*>(my_region) + c * D;
    if constexpr (FP8) {
#pragma unroll
      for (int i = 0; i < NBLK / 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<f32x4*>(orow + 64 * i + 16 * qd + 4 * e) =
              f32x4{acc[4 * i][e], acc[4 * i + 1][e], acc[4 * i + 2][e], acc[4 * i + 3][e]};
    } else {
#pragma unroll
      for (int i = 0; i < NBLK / 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          *reinterpret_cast<f32x4*>(orow + 32 * i + 8 * qd + 4 * j) =
              f32x4{acc[2 * i][2 * j], acc[2 * i + 1][2 * j], acc[2 * i][2 * j + 1],
                    acc[2 * i + 1][2 * j + 1]};
    }
  }
  __syncthreads();

  // ---- merge the waves of this partition, 4 dims per thread ---------------
  for (int i = threadIdx.x; i < G * D / 4; i += NW * kWave) {
    const int gg = (4 * i) / D, d = (4 * i) % D;
    float M = -INFINITY;
    bool nan_m = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = sm_m[w][gg];
      nan_m |= mw != mw;
      M = fmaxf(M, mw);
    }
    f32x4 o = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float l = 0.0f;
    if (nan_m) {
      M = l = __builtin_nanf("");
      o = f32x4{M, M, M, M};
    } else if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float wt = __builtin_amdgcn_exp2f(sm_m[w][gg] - M);
        const f32x4 ow =
            *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(smem + w * REGION) +
                                            gg * D + d);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] += wt * ow[e];
        l += wt * sm_l[w][gg];
      }
    }
    const int hq = h * G + gg;
    const int64_t row = (int64_t)b * p.num_q_heads + hq;
    if (p.direct) {
      const bool live = l > 0.0f || l != l;                     // NaN stays NaN
      f32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = live ? o[e] / l * vs : 0.0f;
      if (p.out_bf16) {
        const bf16x2 lo2 = __builtin_convertvector((float2_t){r[0], r[1]}, bf16x2);
        const bf16x2 hi2 = __builtin_convertvector((float2_t){r[2], r[3]}, bf16x2);
        uint2 w2;
        w2.x = __builtin_bit_cast(uint32_t, lo2);
        w2.y = __builtin_bit_cast(uint32_t, hi2);
        *reinterpret_cast<uint2*>(reinterpret_cast<__bf16*>(p.out) + row * D + d) = w2;
      } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + row * D + d) = r;
      }
    } else {
      const int64_t slot = row * p.num_parts + part;
      *reinterpret_cast<f32x4*>(p.ws_o + slot * D + d) = o;
      if (d == 0) {
        p.ws_m[slot] = M;
        p.ws_l[slot] = l;
      }
    }
  }
}

// Merge the partitions of one (sequence, query head):
//   M = max_j m_j,  w_j = 2^(m_j - M),  out = s_v * sum_j w_j o_j / sum_j w_j l_j
// over every planned partition: the split kernel leaves an empty partial
// (m = -inf, l = 0) in the slots of partitions a sequence does not reach, so
// the merge needs neither the context length nor a second round trip. Each
// wave owns SW dims of one (sequence, query head) and needs no barrier. The
// partitions are taken NPC at a time (one chunk for up to 128 partitions):
// lane j reads m_j and l_j (two per lane past 64), and the partial outputs
// are read as 16-byte pieces: lane (pg, dq) = (lane / (SW/4), lane % (SW/4))
// holds dims 4 dq .. 4 dq + 3 of partitions pg, pg + PG, pg + 2 PG, ...
// (PG = 256 / SW partition groups), so a chunk is NPC / PG loads per lane,
// all issued before the first wait. The slice width shrinks as the
// partitions grow (64 dims up to 32 partitions, 32 for 64, 16 for 128), so
// a lane never holds more than 8 pieces and more work-groups share a row.
// The wave max and sum run on DPP row rotations and the gfx950 row swaps (no
// LDS round trip); the weights w_j reach the lanes through LDS. A partition
// of weight 0 adds nothing (its o may never have been written), and a later
// chunk with a larger max rescales what the earlier ones summed. The
// partition groups of a dim are summed at the end, inside rows with DPP
// rotations and across rows with the row swaps.
template <int NPC>
constexpr int reduce_slice_dims() {
  return NPC <= 32 ? 64 : (NPC <= 64 ? 32 : 16);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <bool MAX>
__device__ __forceinline__ float wave_all(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  x = op(x, dpp_mov<0x128>(x));           // row_ror:8
  x = op(x, dpp_mov<0x124>(x));           // row_ror:4
  x = op(x, dpp_mov<0x122>(x));           // row_ror:2
  x = op(x, dpp_mov<0x121>(x));           // row_ror:1 -> every lane holds its row's result
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = op(__uint_as_float(c[0]), __uint_as_float(c[1]));
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

template <int D, int NPC>
__global__ __launch_bounds__(kWave) void paged_decode_reduce_kernel(const DecodeParams p) {
  constexpr int SW = reduce_slice_dims<NPC>();        // dims per work-group
  constexpr int DQ = SW / 4;                           // lanes per partition group
  constexpr int PG = kWave / DQ;                       // partition groups
  static_assert(NPC % PG == 0 && (NPC <= kWave || NPC % kWave == 0) && NPC <= kReduceChunk &&
                    D % SW == 0,
                "a chunk is at most one wave of partitions, or whole waves of them");
  // One wave per work-group: work-group x merges dims SW*(x mod D/SW) ..
  // +SW-1 of query head x / (D/SW), so the partials of a row are read by
  // D/SW compute units at once rather than one.
  constexpr int kSlices = D / SW;
  constexpr int MPL = NPC > kWave ? NPC / kWave : 1;   // partitions per lane (m, l)
  constexpr int OPL = NPC / PG;                        // 16-byte partial loads per lane
  __shared__ __align__(16) float sw[NPC];
  const int lane = threadIdx.x;
  const int pg = lane / DQ, dq = lane % DQ;
  const int d0 = (int)(blockIdx.x % kSlices) * SW + 4 * dq;
  const int hq = (int)(blockIdx.x / kSlices);
  const int b = blockIdx.y;
  const int h = hq / p.group;
  const int np = p.num_parts;
  const int64_t row = (int64_t)b * p.num_q_heads + hq;
  const float* mrow = p.ws_m + row * np;
  const float* lrow = p.ws_l + row * np;
  const float* orow = p.ws_o + row * np * D + d0;
  const float vs = p.v_scale ? p.v_scale[p.scale_per_head ? h : 0] : 1.0f;

  float M = -INFINITY, L = 0.0f;
  f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  bool any_nan = false;                   // a NaN partial makes the row NaN
  for (int base = 0; base < np; base += NPC) {
    // Every load of the chunk, unconditionally: the workspace ends with a
    // chunk's worth of slack (and the m and l regions are followed by
    // others), and slots past this row's partitions (other rows' partials,
    // slack) get weight 0 below.
    float mv[MPL], lv[MPL];
#pragma unroll
    for (int k = 0; k < MPL; ++k) {
      mv[k] = mrow[base + k * kWave + lane];
      lv[k] = lrow[base + k * kWave + lane];
    }
    f32x4 ov[OPL];
#pragma unroll
    for (int u = 0; u < OPL; ++u)
      ov[u] = *reinterpret_cast<const f32x4*>(orow + (int64_t)(base + PG * u + pg) * D);
    float mj[MPL], lj[MPL], mloc = -INFINITY;
    bool nan_here = false;
#pragma unroll
    for (int k = 0; k < MPL; ++k) {
      const int j = k * kWave + lane;
      const bool in = j < NPC && base + j < np;
      mj[k] = in ? mv[k] : -INFINITY;
      lj[k] = in ? lv[k] : 0.0f;
      nan_here |= mj[k] != mj[k];
      mloc = fmaxf(mloc, mj[k]);
    }
    any_nan |= __builtin_amdgcn_ballot_w64(nan_here) != 0ull;
    const float Mn = fmaxf(M, wave_all<true>(mloc));
    // weights relative to Mn (to 0 while nothing is attended: all weights 0);
    // what earlier chunks summed is rescaled to it
    const float Mr = Mn == -INFINITY ? 0.0f : Mn;
    const float r = __builtin_amdgcn_exp2f(M - Mr);     // 0 while M = -inf
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= r;
    L *= r;
    M = Mn;
    float wl = 0.0f;
#pragma unroll
    for (int k = 0; k < MPL; ++k) {
      const int j = k * kWave + lane;
      const float wj = mj[k] != -INFINITY ? __builtin_amdgcn_exp2f(mj[k] - Mr) : 0.0f;
      wl += wj * lj[k];
      if (j < NPC) sw[j] = wj;
    }
    L += wave_all<false>(wl);
#pragma unroll
    for (int u = 0; u < OPL; ++u) {
      const float w = sw[PG * u + pg];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(w, w != 0.0f ? ov[u][e] : 0.0f, acc[e]);
    }
  }
  // the partition groups of each dim: lanes dq, dq + DQ, dq + 2 DQ, ...
  // (rotations by 8 and 4 inside each row of 16 lanes, then the row swaps)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (DQ <= 8) acc[e] += dpp_mov<0x128>(acc[e]);   // row_ror:8
    if constexpr (DQ <= 4) acc[e] += dpp_mov<0x124>(acc[e]);   // row_ror:4
    acc[e] = wave_sum_col(acc[e]);
  }
  // rows past the last row of a prefill merge write nothing (their loads
  // above stayed inside the workspace, which holds every grid row; the test
  // comes last so that its dependent load does not delay theirs)
  if (p.row_limit && b >= *p.row_limit) return;
  if (pg != 0) return;
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    r[e] = any_nan ? __builtin_nanf("") : (L > 0.0f ? acc[e] / L * vs : 0.0f);
  if (p.out_bf16) {
    const bf16x2 lo2 = __builtin_convertvector((float2_t){r[0], r[1]}, bf16x2);
    const bf16x2 hi2 = __builtin_convertvector((float2_t){r[2], r[3]}, bf16x2);
    uint2 w2;
    w2.x = __builtin_bit_cast(uint32_t, lo2);
    w2.y = __builtin_bit_cast(uint32_t, hi2);
    *reinterpret_cast<uint2*>(reinterpret_cast<__bf16*>(p.out) + row * D + d0) = w2;
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + row * D + d0) = r;
  }
}

template <int D, int NPC>
static void launch_reduce_chunk(const DecodeParams& pr, int num_seqs, hipStream_t stream) {
  const dim3 grid((unsigned)(pr.num_q_heads * (D / reduce_slice_dims<NPC>())),
                  (unsigned)num_seqs);
  hipLaunchKernelGGL((paged_decode_reduce_kernel<D, NPC>), grid, dim3(kWave), 0, stream, pr);
}

template <int D>
static void launch_reduce(const DecodeParams& pr, int num_seqs, hipStream_t stream) {
  static_assert(kReduceChunk == 128, "the largest chunk below is the workspace's slack");
  if (pr.num_parts <= 16) launch_reduce_chunk<D, 16>(pr, num_seqs, stream);
  else if (pr.num_parts <= 32) launch_reduce_chunk<D, 32>(pr, num_seqs, stream);
  else if (pr.num_parts <= 64) launch_reduce_chunk<D, 64>(pr, num_seqs, stream);
  else launch_reduce_chunk<D, 128>(pr, num_seqs, stream);
}

// Arithmetic modes of the split kernel.
constexpr int kModeBf16 = 0;   // codes expanded to bf16, static scales
constexpr int kModeFp8 = 1;    // all-FP8 attention
constexpr int kModeDyn = 2;    // codes expanded to bf16, dynamic per-token scales

template <int D, int FMT, int TP, int RING, int SLOTS, bool FUSED, int MODE, bool WIDE = false>
static hipError_t launch_variant(const DecodeParams& p, int num_seqs, hipStream_t stream,
                                 hipEvent_t ev_before, hipEvent_t ev_after) {
  constexpr int NW = kSplitWaves;
  constexpr bool ATT8 = MODE == kModeFp8, DYN = MODE == kModeDyn;
  const dim3 grid((unsigned)p.num_parts, (unsigned)p.num_kv_heads, (unsigned)num_seqs);
  if (ev_before && ev_after) {
    // the events take the kernel's own start and end timestamps
    hipExtLaunchKernelGGL((paged_decode_split_kernel<D, FMT, NW, TP, RING, SLOTS, FUSED, ATT8, DYN, WIDE>),
                          grid, dim3(NW * kWave), 0, stream, ev_before, ev_after, 0, p);
  } else {
    hipLaunchKernelGGL((paged_decode_split_kernel<D, FMT, NW, TP, RING, SLOTS, FUSED, ATT8, DYN, WIDE>),
                       grid, dim3(NW * kWave), 0, stream, p);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.direct) return err;
  DecodeParams pr = p;
  // the reduce kernel applies a static V scale only (dynamic ones are in P)
  if (FMT == kFmtBf16 || DYN) pr.v_scale = nullptr;
  launch_reduce<D>(pr, num_seqs, stream);
  return hipGetLastError();
}

// Tile shape of the split kernel: TP pages per tile, RING register buffers,
// SLOTS LDS buffers (SLOTS > 0: LDS-staged loads, one register tile).
// The plan picks 2x1 (2-page tiles, loaded and computed one at a time) or
// 2x1s1 (the same with the next tile staged in LDS), and 4x1s1 (4-page
// staged tiles) for fp8 caches at head_dim 64 in the bf16-arithmetic mode
// with static scales.
// The tuning override KVQ_TUNE_SPLIT_SHAPE (kvq_set_tuning) selects the other
// shapes (2x2, 4x1, 2x1s2, 4x1s1) for sweeps and tests; a shape whose LDS
// ring would pass 64 KiB is rejected. The all-FP8 and dynamic-scale modes, and groups above
// 8, are built for the two planned shapes only.
template <int D, int FMT, int TP, int RING, int SLOTS>
static hipError_t launch_shape(const DecodeParams& p, int num_seqs, bool fused, int mode,
                               hipStream_t stream, hipEvent_t ev_before, hipEvent_t ev_after) {
  constexpr int E = FMT == kFmtBf16 ? 2 : 1;
  constexpr int kv_ring = kSplitWaves * SLOTS * TP * 2 * kPage * D * E;
  constexpr bool planned = FMT != kFmtBf16 && TP == 2 && RING == 1 && SLOTS <= 1;
  if constexpr (kv_ring > kMaxLdsRing) {
    return hipErrorInvalidValue;
  } else {
    if (mode == kModeFp8) {
      if constexpr (planned) {
        return fused ? launch_variant<D, FMT, TP, RING, SLOTS, true, kModeFp8>(
                           p, num_seqs, stream, ev_before, ev_after)
                     : launch_variant<D, FMT, TP, RING, SLOTS, false, kModeFp8>(
                           p, num_seqs, stream, ev_before, ev_after);
      } else {
        return hipErrorInvalidValue;
      }
    }
    // G > 8 outside the all-FP8 mode: the WIDE instance (P*V once per half of
    // P), built for the plan's two shapes
    constexpr bool planned_any = TP == 2 && RING == 1 && SLOTS <= 1;
    const bool wide = p.group > 8;
    if (mode == kModeDyn) {
      if constexpr (planned &&
                    kv_ring + kSplitWaves * SLOTS * TP * kTileScaleBytesPerPage <= kMaxLdsRing) {
        if (wide)
          return fused ? launch_variant<D, FMT, TP, RING, SLOTS, true, kModeDyn, true>(
                             p, num_seqs, stream, ev_before, ev_after)
                       : launch_variant<D, FMT, TP, RING, SLOTS, false, kModeDyn, true>(
                             p, num_seqs, stream, ev_before, ev_after);
        return fused ? launch_variant<D, FMT, TP, RING, SLOTS, true, kModeDyn>(
                           p, num_seqs, stream, ev_before, ev_after)
                     : launch_variant<D, FMT, TP, RING, SLOTS, false, kModeDyn>(
                           p, num_seqs, stream, ev_before, ev_after);
      } else {
        return hipErrorInvalidValue;
      }
    }
    if (wide) {
      if constexpr (planned_any) {
        return fused ? launch_variant<D, FMT, TP, RING, SLOTS, true, kModeBf16, true>(
                           p, num_seqs, stream, ev_before, ev_after)
                     : launch_variant<D, FMT, TP, RING, SLOTS, false, kModeBf16, true>(
                           p, num_seqs, stream, ev_before, ev_after);
      } else {
        return hipErrorInvalidValue;
      }
    }
    return fused ? launch_variant<D, FMT, TP, RING, SLOTS, true, kModeBf16>(
                       p, num_seqs, stream, ev_before, ev_after)
                 : launch_variant<D, FMT, TP, RING, SLOTS, false, kModeBf16>(
                       p, num_seqs, stream, ev_before, ev_after);
  }
}

template <int D, int FMT>
static hipError_t launch_typed(const DecodeParams& p, int num_seqs, bool fused, int plan_slots,
                               int plan_tile_pages, int mode, hipStream_t stream,
                               hipEvent_t ev_before, hipEvent_t ev_after) {
  int tp = plan_tile_pages, ring = 1, slots = plan_slots;
  // an explicit shape override (kvq_set_tuning: 100 TP + 10 RING + SLOTS)
  if (const int v = tuning_override(KVQ_TUNE_SPLIT_SHAPE); v >= 0) {
    tp = v / 100;
    ring = (v / 10) % 10;
    slots = v % 10;
  }
#define KVFP8_SHAPE(TP_, RING_, SLOTS_)                                                 \
  if (tp == TP_ && ring == RING_ && slots == SLOTS_)                                    \
    return launch_shape<D, FMT, TP_, RING_, SLOTS_>(p, num_seqs, fused, mode, stream,   \
                                                    ev_before, ev_after);
  KVFP8_SHAPE(2, 1, 0)
  KVFP8_SHAPE(2, 2, 0)
  KVFP8_SHAPE(4, 1, 0)
  KVFP8_SHAPE(2, 1, 1)
  KVFP8_SHAPE(2, 1, 2)
  KVFP8_SHAPE(4, 1, 1)
#undef KVFP8_SHAPE
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t launch_dim(const DecodeParams& p, int fmt, int num_seqs, bool fused, int slots,
                             int tile_pages, int mode, hipStream_t stream, hipEvent_t ev_before,
                             hipEvent_t ev_after) {
  switch (fmt) {
    case kFmtBf16:
      return launch_typed<D, kFmtBf16>(p, num_seqs, fused, slots, tile_pages, mode, stream,
                                       ev_before, ev_after);
    case kFmtE4M3:
      return launch_typed<D, kFmtE4M3>(p, num_seqs, fused, slots, tile_pages, mode, stream,
                                       ev_before, ev_after);
    case kFmtE5M2:
      return launch_typed<D, kFmtE5M2>(p, num_seqs, fused, slots, tile_pages, mode, stream,
                                       ev_before, ev_after);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace kvfp8
