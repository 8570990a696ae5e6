// paged_decode.hip - GQA decode attention over the paged FP8 e4m3 (or bf16)
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
//    accurate to ~2^-17 at no extra MFMA cost;
//  * per 2-page tile the P*V MFMA result (level 1, FP32) is added to the FP32
//    running accumulator after the online-softmax rescale (level 2);
//  * the waves of a work-group merge their (m, l, o) through LDS; the reduce
//    kernel merges partitions in FP32 and applies the V head scale.
#include <hip/hip_ext.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

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

__device__ __forceinline__ float wave_max_col(float x) {
  // lanes c, c+16, c+32, c+48 hold the same MFMA column
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum_col(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

struct PartitionRange {
  int L, lo, first_page, end_page, num_parts_b;
};

// The partitions of one sequence: pages [first_page, end_page) cover the
// attended positions [lo, L); partition j holds part_pages pages of them.
__device__ __forceinline__ PartitionRange partition_range(const DecodeParams& p,
                                                          int b, int part_pages) {
  PartitionRange r;
  r.L = p.context_lens[b];
  if (r.L < 0) r.L = 0;
  r.lo = (p.window > 0 && r.L > p.window) ? r.L - p.window : 0;
  // Device-side values are never trusted to stay in bounds: positions past
  // the block-table row are ignored and partitions past the plan are dropped.
  if (r.L > p.max_pages_per_seq * kPage) r.L = p.max_pages_per_seq * kPage;
  if (r.lo > r.L) r.lo = r.L;
  r.first_page = r.lo / kPage;
  r.end_page = (r.L + kPage - 1) / kPage;
  const int n = r.end_page - r.first_page;
  r.num_parts_b = n > 0 ? (n + part_pages - 1) / part_pages : 0;
  if (r.num_parts_b > p.num_parts) r.num_parts_b = p.num_parts;
  return r;
}

template <int D, bool FP8, int NW, int TP, int RING, bool FUSED>
__global__ __launch_bounds__(NW * kWave) void paged_decode_split_kernel(
    const DecodeParams p) {
  constexpr int E = FP8 ? 1 : 2;
  constexpr int PB = kPage * D * E;     // bytes of one (page, head) block
  constexpr int NI = PB / 1024;         // 1 KiB wave loads per page per tensor
  constexpr int NK = D / 32;            // q k^T MFMAs per page
  constexpr int NBLK = D / 16;          // P*V output blocks of 16 dims
  constexpr int GMAX = 8;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int part = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int G = p.group;
  const int qd = lane >> 4;             // row quad of the MFMA layout
  const int c = lane & 15;              // MFMA column
  const int part_pages = NW * p.pages_per_wave;

  const PartitionRange pr = partition_range(p, b, part_pages);
  const float vs = FP8 ? p.v_scale[p.scale_per_head ? h : 0] : 1.0f;
  if (part >= pr.num_parts_b) {
    // Nothing to attend here. In direct mode the first partition still owns
    // the output rows (empty context -> zeros).
    if (p.direct && part == 0) {
      for (int i = threadIdx.x; i < G * D; i += NW * kWave) {
        const int64_t o = ((int64_t)b * p.num_q_heads + h * G + i / D) * D + i % D;
        if (p.out_bf16) reinterpret_cast<__bf16*>(p.out)[o] = (__bf16)0.0f;
        else reinterpret_cast<float*>(p.out)[o] = 0.0f;
      }
    }
    return;
  }

  const int wbeg = pr.first_page + part * part_pages + wave * p.pages_per_wave;
  const int wend = min(wbeg + p.pages_per_wave, pr.end_page);
  const int npages = wend > wbeg ? wend - wbeg : 0;

  // Column c < G: query c (high half of P); G <= c < 2G: query c - G (low
  // half of P); other columns idle.
  const int g = c < G ? c : (c < 2 * G ? c - G : -1);
  const bool lo_col = (c >= G) && (c < 2 * G);

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

  // Page ids of this wave's run, one per lane.
  int my_page = -1;
  if (lane < npages)
    my_page = p.block_tables[(int64_t)b * p.max_pages_per_seq + wbeg + lane];
  if (my_page < 0 || (int64_t)my_page >= p.num_pages) my_page = -1;   // empty page
  const uint64_t bad_pages = __ballot(my_page < 0 && lane < npages);

  const int64_t page_stride = (int64_t)p.num_kv_heads * PB;
  const uint8_t* kbase = p.k_cache + (int64_t)h * PB;
  const uint8_t* vbase = p.v_cache + (int64_t)h * PB;
  const float ks = FP8 ? p.k_scale[p.scale_per_head ? h : 0] : 1.0f;
  const float c_log2 = ks * p.sm_scale_log2;

  // ---- fused decode step: the cache write of position L-1 -----------------
  // Exactly one wave streams the page that holds the newest position of this
  // (sequence, KV head). That wave quantises the new K and V rows (the same
  // arithmetic as the cache-write kernel), stores them into the cache and
  // keeps the stored bytes in LDS; when it reaches that page it patches them
  // into its tile registers. No other wave reads that page, so no ordering
  // across waves is needed, and the page load never has to observe the store.
  __shared__ __align__(16) uint8_t new_rows[FUSED ? 2 * D * E : 16];
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
  // loads (lane j < D/8 holds dims 8j..8j+7 of K and of V) and quantises,
  // stores and stages them right after: memory operations retire in order,
  // so waiting for the rows does not wait for the tiles, and the conversion
  // overlaps their latency.
  uint4 kx_new = make_uint4(0u, 0u, 0u, 0u), vx_new = make_uint4(0u, 0u, 0u, 0u);
  auto fused_prefetch = [&]() {
    if constexpr (FUSED) {
      if (t_new < 0 || lane >= D / 8) return;
      const int64_t src = ((int64_t)b * p.num_kv_heads + h) * D + 8 * lane;
      kx_new = *reinterpret_cast<const uint4*>(p.k_new + src);
      vx_new = *reinterpret_cast<const uint4*>(p.v_new + src);
    }
  };
  auto fused_commit = [&]() {
    if constexpr (FUSED) {
      const int pid = __builtin_amdgcn_readlane(my_page, idx_new);
      uint8_t* kblk = const_cast<uint8_t*>(p.k_cache) + ((int64_t)pid * p.num_kv_heads + h) * PB;
      uint8_t* vblk = const_cast<uint8_t*>(p.v_cache) + ((int64_t)pid * p.num_kv_heads + h) * PB;
      const int j = lane;
      if (j < D / 8) {
        const uint4 kx = kx_new, vx = vx_new;
        if constexpr (FP8) {
          const float sk = p.k_scale[p.scale_per_head ? h : 0];
          const float sv = p.v_scale[p.scale_per_head ? h : 0];
          const uint32_t kw[4] = {kx.x, kx.y, kx.z, kx.w};
          const uint32_t vw[4] = {vx.x, vx.y, vx.z, vx.w};
          uint32_t kq[2] = {0u, 0u}, vq[2] = {0u, 0u};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t kb = (kw[e / 2] >> (16 * (e % 2))) & 0xFFFFu;
            const uint32_t vb = (vw[e / 2] >> (16 * (e % 2))) & 0xFFFFu;
            kq[e / 4] |= e4m3_encode_sat(bf16_bits_to_f32(kb) / sk) << (8 * (e % 4));
            vq[e / 4] |= e4m3_encode_sat(bf16_bits_to_f32(vb) / sv) << (8 * (e % 4));
          }
          *reinterpret_cast<uint2*>(new_rows + 8 * j) = make_uint2(kq[0], kq[1]);
          *reinterpret_cast<uint2*>(new_rows + D + 8 * j) = make_uint2(vq[0], vq[1]);
          *reinterpret_cast<uint2*>(kblk + k_byte<1>(r_new, 8 * j)) = make_uint2(kq[0], kq[1]);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            vblk[v_byte<1>(r_new, 8 * j + e)] = (uint8_t)(vq[e / 4] >> (8 * (e % 4)));
        } else {
          *reinterpret_cast<uint4*>(new_rows + 16 * j) = kx;
          *reinterpret_cast<uint4*>(new_rows + 2 * D + 16 * j) = vx;
          *reinterpret_cast<uint4*>(kblk + k_byte<2>(r_new, 8 * j)) = kx;
          const uint32_t vw[4] = {vx.x, vx.y, vx.z, vx.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            *reinterpret_cast<uint16_t*>(vblk + v_byte<2>(r_new, 8 * j + e)) =
                (uint16_t)(vw[e / 2] >> (16 * (e % 2)));
        }
      }
    }
  };

  float m_run = -INFINITY;
  float l_run = 0.0f;
  f32x4 acc[NBLK];
#pragma unroll
  for (int i = 0; i < NBLK; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // A tile is TP pages (an even number: the P*V MFMA contracts 32 positions,
  // two pages). Missing pages (past the run, an odd tail) and invalid ids
  // load pool page 0 instead: their positions are masked, so the values never
  // matter, and the registers never hold uninitialised data.
  struct Tile {
    uint4 k[TP][NI];
    uint4 v[TP][NI];
  };

  auto load_tile = [&](int t, Tile& tl) {
#pragma unroll
    for (int pg = 0; pg < TP; ++pg) {
      const int idx = TP * t + pg;
      const bool ok = idx < npages && !((bad_pages >> idx) & 1ull);
      const int pid = ok ? __builtin_amdgcn_readlane(my_page, idx) : 0;
      const uint4* kp = reinterpret_cast<const uint4*>(kbase + (int64_t)pid * page_stride);
      const uint4* vp = reinterpret_cast<const uint4*>(vbase + (int64_t)pid * page_stride);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        tl.k[pg][i] = load_stream(kp + i * kWave + lane);
        tl.v[pg][i] = load_stream(vp + i * kWave + lane);
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
        bf16x8 kop;
        if constexpr (FP8) {
          const uint4 w = tl.k[pg][s / 2];
          kop = (s % 2 == 0) ? e4m3x8_to_bf16x8(w.x, w.y) : e4m3x8_to_bf16x8(w.z, w.w);
        } else {
          kop = bits_to_bf16x8(tl.k[pg][s]);
        }
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[s], sacc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) x[pg][e] = sacc[e] * c_log2;
    }
    // ---- masking: positions outside [lo, L), past the run, invalid pages --
    const int pos0 = (wbeg + TP * t) * kPage;           // first position of the tile
    bool any_missing = false;
#pragma unroll
    for (int pg = 0; pg < TP; ++pg) {
      const int idx = TP * t + pg;
      any_missing |= idx >= npages || ((bad_pages >> idx) & 1ull);
    }
    const bool need_mask = (pos0 < pr.lo) || (pos0 + TP * kPage > pr.L) || any_missing;
    uint32_t vkeep = 0xFFFFFFFFu;                        // bit 4*pg+e: row 4qd+e of page pg
    if (need_mask) {
      vkeep = 0u;
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
    }
    if (g < 0) {
#pragma unroll
      for (int pg = 0; pg < TP; ++pg)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[pg][e] = -INFINITY;
    }
    // ---- online softmax (log2 domain) -------------------------------------
    float tmax = x[0][0];
#pragma unroll
    for (int pg = 0; pg < TP; ++pg)
#pragma unroll
      for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, x[pg][e]);
    tmax = wave_max_col(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.0f;
    bf16x8 pop[TP / 2];
#pragma unroll
    for (int pg = 0; pg < TP; ++pg) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pe = __builtin_amdgcn_exp2f(x[pg][e] - m_use);
        psum += pe;
        // P as bf16: the high part in the query columns, the rounding
        // residue in the duplicate columns.
        const __bf16 hi = (__bf16)pe;
        pop[pg / 2][4 * (pg % 2) + e] = lo_col ? (__bf16)(pe - (float)hi) : hi;
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // ---- P*V: TP/2 chained k=32 MFMAs per 16-dim block (level 1, FP32),
    // folded into the running accumulator after the rescale (level 2) -------
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      f32x4 part_o = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int pp = 0; pp < TP / 2; ++pp) {
        uint4 vb;
        if constexpr (FP8) {
          const int i = blk / 4, ep = blk % 4;
          const uint4 wa = tl.v[2 * pp][i], wb = tl.v[2 * pp + 1][i];
          const uint32_t da = ep == 0 ? wa.x : ep == 1 ? wa.y : ep == 2 ? wa.z : wa.w;
          const uint32_t db = ep == 0 ? wb.x : ep == 1 ? wb.y : ep == 2 ? wb.z : wb.w;
          vb = __builtin_bit_cast(uint4, cat(e4m3x4_to_bf16x4(da), e4m3x4_to_bf16x4(db)));
        } else {
          const int i = blk / 2, ep = blk % 2;
          const uint4 wa = tl.v[2 * pp][i], wb = tl.v[2 * pp + 1][i];
          vb = ep == 0 ? make_uint4(wa.x, wa.y, wb.x, wb.y) : make_uint4(wa.z, wa.w, wb.z, wb.w);
        }
        if (need_mask) {
          // zero the bf16 values of masked rows (poison codes are NaN)
          const uint32_t kk = vkeep >> (8 * pp);
          uint32_t mw[4];
#pragma unroll
          for (int k2 = 0; k2 < 4; ++k2)
            mw[k2] = (((kk >> (2 * k2)) & 1u) ? 0x0000FFFFu : 0u) |
                     (((kk >> (2 * k2 + 1)) & 1u) ? 0xFFFF0000u : 0u);
          vb.x &= mw[0]; vb.y &= mw[1]; vb.z &= mw[2]; vb.w &= mw[3];
        }
        part_o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bits_to_bf16x8(vb), pop[pp], part_o,
                                                         0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[blk][e] = acc[blk][e] * alpha + part_o[e];
    }
  };

  const int ntiles = (npages + TP - 1) / TP;
  // Register ring of RING tiles: RING - 1 tiles are in flight while one is
  // computed.
  if constexpr (RING == 3) {
    Tile t0, t1, t2;
    fused_prefetch();
    if (ntiles > 0) load_tile(0, t0);
    if (ntiles > 1) load_tile(1, t1);
    if (t_new >= 0) fused_commit();
    for (int t = 0; t < ntiles; t += 3) {
      if (t + 2 < ntiles) load_tile(t + 2, t2);
      if (FUSED && t == t_new) patch_tile(t0);
      compute_tile(t, t0);
      if (t + 1 >= ntiles) break;
      if (t + 3 < ntiles) load_tile(t + 3, t0);
      if (FUSED && t + 1 == t_new) patch_tile(t1);
      compute_tile(t + 1, t1);
      if (t + 2 >= ntiles) break;
      if (t + 4 < ntiles) load_tile(t + 4, t1);
      if (FUSED && t + 2 == t_new) patch_tile(t2);
      compute_tile(t + 2, t2);
    }
  } else if constexpr (RING == 2) {
    Tile t0, t1;
    fused_prefetch();
    if (ntiles > 0) load_tile(0, t0);
    if (t_new >= 0) fused_commit();
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
    for (int t = 0; t < ntiles; ++t) {
      if (t > 0) load_tile(t, t0);
      if (FUSED && t == t_new) patch_tile(t0);
      compute_tile(t, t0);
    }
  }

  // ---- per-wave results: l over the row quads, lo columns into hi ----------
  l_run = wave_sum_col(l_run);
#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[blk][e] += __shfl_down(acc[blk][e], G);

  __shared__ float sm_o[NW][GMAX][D];
  __shared__ float sm_m[NW][GMAX];
  __shared__ float sm_l[NW][GMAX];
  if (c < G) {
    if (qd == 0) {
      sm_m[wave][c] = m_run;
      sm_l[wave][c] = l_run;
    }
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int d;
        if constexpr (FP8) d = 64 * (blk / 4) + 16 * qd + 4 * e + (blk % 4);
        else d = 32 * (blk / 2) + 8 * qd + 2 * e + (blk % 2);
        sm_o[wave][c][d] = acc[blk][e];
      }
    }
  }
  __syncthreads();

  // ---- merge the waves of this partition ----------------------------------
  for (int i = threadIdx.x; i < G * D; i += NW * kWave) {
    const int gg = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][gg]);
    float o = 0.0f, l = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float wt = __builtin_amdgcn_exp2f(sm_m[w][gg] - M);
        o += wt * sm_o[w][gg][d];
        l += wt * sm_l[w][gg];
      }
    }
    const int hq = h * G + gg;
    const int64_t row = (int64_t)b * p.num_q_heads + hq;
    if (p.direct) {
      const float r = l > 0.0f ? o / l * vs : 0.0f;
      if (p.out_bf16) reinterpret_cast<__bf16*>(p.out)[row * D + d] = (__bf16)r;
      else reinterpret_cast<float*>(p.out)[row * D + d] = r;
    } else {
      const int64_t slot = row * p.num_parts + part;
      p.ws_o[slot * D + d] = o;
      if (d == 0) {
        p.ws_m[slot] = M;
        p.ws_l[slot] = l;
      }
    }
  }
}

// Merge the partitions of one (sequence, query head):
//   M = max_j m_j,  w_j = 2^(m_j - M),  out = s_v * sum_j w_j o_j / sum_j w_j l_j
// kReduceThreads threads, as (dim d, partition group) pairs. Every global load
// is issued up front - each thread's first kReducePer partial outputs into
// registers, the m and l rows into LDS - so the kernel costs one memory round
// trip plus two block reductions; partitions past the first
// kReduceThreads / D * kReducePer (very long contexts) are read in a second
// loop.
constexpr int kReduceThreads = 512;
constexpr int kReducePer = 8;             // partial outputs per thread held in registers
constexpr int kReduceLds = 4096;          // partitions whose m/l (then weight) sit in LDS

__device__ __forceinline__ float block_reduce(float v, bool is_max, float* red) {
  for (int off = kWave / 2; off > 0; off /= 2) {
    const float o = __shfl_xor(v, off);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  const int wid = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  __syncthreads();                       // red[] may still be read by a previous call
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < (int)(blockDim.x / kWave); ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

template <int D>
__global__ __launch_bounds__(kReduceThreads) void paged_decode_reduce_kernel(
    const DecodeParams p, int part_pages) {
  constexpr int NG = kReduceThreads / D;  // partition groups
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int h = hq / p.group;
  const PartitionRange pr = partition_range(p, b, part_pages);
  const int np = pr.num_parts_b;
  const int64_t row = (int64_t)b * p.num_q_heads + hq;
  const float* ms = p.ws_m + row * p.num_parts;
  const float* ls = p.ws_l + row * p.num_parts;
  const float* os = p.ws_o + row * p.num_parts * D;

  __shared__ float red[kReduceThreads / kWave];
  __shared__ float m_s[kReduceLds];       // m_j, then the weight w_j
  __shared__ float l_s[kReduceLds];
  __shared__ float o_s[NG][D];

  const int d = tid % D, grp = tid / D;
  // ---- every load first -----------------------------------------------------
  float ov[kReducePer];
#pragma unroll
  for (int u = 0; u < kReducePer; ++u) {
    const int jj = grp + u * NG;
    ov[u] = jj < np ? os[(int64_t)jj * D + d] : 0.0f;
  }
  for (int jj = tid; jj < np && jj < kReduceLds; jj += kReduceThreads) {
    m_s[jj] = ms[jj];
    l_s[jj] = ls[jj];
  }
  // ---- M, weights, normaliser (each thread touches the LDS entries it wrote)
  float m = -INFINITY;
  for (int jj = tid; jj < np; jj += kReduceThreads)
    m = fmaxf(m, jj < kReduceLds ? m_s[jj] : ms[jj]);
  const float M = block_reduce(m, true, red);
  float lsum = 0.0f;
  for (int jj = tid; jj < np; jj += kReduceThreads) {
    const float mj = jj < kReduceLds ? m_s[jj] : ms[jj];
    const float lj = jj < kReduceLds ? l_s[jj] : ls[jj];
    const float w = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mj - M);
    if (jj < kReduceLds) m_s[jj] = w;
    lsum += w * lj;
  }
  const float L = block_reduce(lsum, false, red);   // its barriers publish the weights
  auto weight = [&](int jj) {
    return jj < kReduceLds ? m_s[jj] : __builtin_amdgcn_exp2f(ms[jj] - M);
  };
  // ---- weighted sum of the partial outputs ---------------------------------
  float acc = 0.0f;
#pragma unroll
  for (int u = 0; u < kReducePer; ++u) {
    const int jj = grp + u * NG;
    if (jj < np) acc += weight(jj) * ov[u];
  }
  for (int jj = grp + kReducePer * NG; jj < np; jj += NG) acc += weight(jj) * os[(int64_t)jj * D + d];
  o_s[grp][d] = acc;
  __syncthreads();
  if (grp == 0) {
    float o = 0.0f;
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) o += o_s[g2][d];
    const float vs = p.v_scale ? p.v_scale[p.scale_per_head ? h : 0] : 1.0f;
    const float r = L > 0.0f ? o / L * vs : 0.0f;
    if (p.out_bf16) reinterpret_cast<__bf16*>(p.out)[row * D + d] = (__bf16)r;
    else reinterpret_cast<float*>(p.out)[row * D + d] = r;
  }
}

template <int D, bool FP8, int TP, int RING, bool FUSED>
static hipError_t launch_variant(const DecodeParams& p, int num_seqs, hipStream_t stream,
                                 hipEvent_t ev_before, hipEvent_t ev_after) {
  constexpr int NW = kSplitWaves;
  const dim3 grid((unsigned)p.num_parts, (unsigned)p.num_kv_heads, (unsigned)num_seqs);
  if (ev_before && ev_after) {
    // the events take the kernel's own start and end timestamps
    hipExtLaunchKernelGGL((paged_decode_split_kernel<D, FP8, NW, TP, RING, FUSED>), grid,
                          dim3(NW * kWave), 0, stream, ev_before, ev_after, 0, p);
  } else {
    hipLaunchKernelGGL((paged_decode_split_kernel<D, FP8, NW, TP, RING, FUSED>), grid,
                       dim3(NW * kWave), 0, stream, p);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.direct) return err;
  DecodeParams pr = p;
  if (!FP8) pr.v_scale = nullptr;
  hipLaunchKernelGGL((paged_decode_reduce_kernel<D>),
                     dim3((unsigned)p.num_q_heads, (unsigned)num_seqs), dim3(kReduceThreads), 0,
                     stream, pr, NW * p.pages_per_wave);
  return hipGetLastError();
}

// Tile shape of the split kernel: TP pages per tile, RING register buffers.
// Default 2x1: 2-page tiles, loaded and computed one at a time, which keeps
// the register count low enough for 3 waves per SIMD; with about 1.5 waves
// per SIMD it was the fastest shape measured on MI355X for the 8B layer at
// 131072 positions (70.5 % of peak) and for 8 ragged sequences of ~20k
// (71.4 %), ahead of the prefetching shapes. KVFP8_SPLIT_VARIANT=TPxRING
// (2x1, 2x2, 2x3, 4x1, 4x2) overrides it for tuning sweeps.
template <int D, bool FP8>
static hipError_t launch_typed(const DecodeParams& p, int num_seqs, bool fused,
                               hipStream_t stream, hipEvent_t ev_before, hipEvent_t ev_after) {
  int tp = 2, ring = 1;
  if (const char* env = getenv("KVFP8_SPLIT_VARIANT")) {
    int a = 0, c = 0;
    if (sscanf(env, "%dx%d", &a, &c) == 2) { tp = a; ring = c; }
  }
#define KVFP8_VARIANT(TP_, RING_)                                                       \
  if (tp == TP_ && ring == RING_)                                                       \
    return fused ? launch_variant<D, FP8, TP_, RING_, true>(p, num_seqs, stream, ev_before,   \
                                                             ev_after)                       \
                 : launch_variant<D, FP8, TP_, RING_, false>(p, num_seqs, stream, ev_before,  \
                                                              ev_after);
  KVFP8_VARIANT(2, 1)
  KVFP8_VARIANT(2, 2)
  KVFP8_VARIANT(2, 3)
  KVFP8_VARIANT(4, 1)
  KVFP8_VARIANT(4, 2)
#undef KVFP8_VARIANT
  return hipErrorInvalidValue;
}

hipError_t launch_paged_decode(const DecodeParams& p, int head_dim, bool fp8,
                               int num_seqs, bool fused, hipStream_t stream,
                               hipEvent_t ev_before, hipEvent_t ev_after) {
  switch (head_dim) {
    case 64:
      return fp8 ? launch_typed<64, true>(p, num_seqs, fused, stream, ev_before, ev_after)
                 : launch_typed<64, false>(p, num_seqs, fused, stream, ev_before, ev_after);
    case 128:
      return fp8 ? launch_typed<128, true>(p, num_seqs, fused, stream, ev_before, ev_after)
                 : launch_typed<128, false>(p, num_seqs, fused, stream, ev_before, ev_after);
    case 256:
      return fp8 ? launch_typed<256, true>(p, num_seqs, fused, stream, ev_before, ev_after)
                 : launch_typed<256, false>(p, num_seqs, fused, stream, ev_before, ev_after);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace kvfp8
