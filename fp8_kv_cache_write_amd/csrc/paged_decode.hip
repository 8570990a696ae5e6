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

template <int D, bool FP8, int NW, int TP, int RING>
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
        tl.k[pg][i] = kp[i * kWave + lane];
        tl.v[pg][i] = vp[i * kWave + lane];
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
    if (ntiles > 0) load_tile(0, t0);
    if (ntiles > 1) load_tile(1, t1);
    for (int t = 0; t < ntiles; t += 3) {
      if (t + 2 < ntiles) load_tile(t + 2, t2);
      compute_tile(t, t0);
      if (t + 1 >= ntiles) break;
      if (t + 3 < ntiles) load_tile(t + 3, t0);
      compute_tile(t + 1, t1);
      if (t + 2 >= ntiles) break;
      if (t + 4 < ntiles) load_tile(t + 4, t1);
      compute_tile(t + 2, t2);
    }
  } else if constexpr (RING == 2) {
    Tile t0, t1;
    if (ntiles > 0) load_tile(0, t0);
    for (int t = 0; t < ntiles; t += 2) {
      if (t + 1 < ntiles) load_tile(t + 1, t1);
      compute_tile(t, t0);
      if (t + 1 >= ntiles) break;
      if (t + 2 < ntiles) load_tile(t + 2, t0);
      compute_tile(t + 1, t1);
    }
  } else {
    Tile t0;
    for (int t = 0; t < ntiles; ++t) {
      load_tile(t, t0);
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
// kReduceThreads threads: the maxima, weights and the normaliser are reduced
// over partitions cooperatively; the weighted sum of the partial outputs runs
// as (dim, partition group) pairs so that every partial row is read once, in
// parallel, and the groups are added through LDS.
constexpr int kReduceThreads = 512;
constexpr int kReduceWeightsLds = 4096;   // partitions whose weight is cached in LDS

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
  __shared__ float w_s[kReduceWeightsLds];
  __shared__ float o_s[NG][D];

  float m = -INFINITY;
  for (int j = tid; j < np; j += kReduceThreads) m = fmaxf(m, ms[j]);
  const float M = block_reduce(m, true, red);
  float lsum = 0.0f;
  for (int j = tid; j < np; j += kReduceThreads) {
    const float w = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ms[j] - M);
    if (j < kReduceWeightsLds) w_s[j] = w;
    lsum += w * ls[j];
  }
  const float L = block_reduce(lsum, false, red);   // its barriers publish w_s

  const int d = tid % D, grp = tid / D;
  float acc = 0.0f;
  int j = grp;
  for (; j + 3 * NG < np; j += 4 * NG) {
    float w[4], o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int jj = j + u * NG;
      w[u] = jj < kReduceWeightsLds ? w_s[jj] : __builtin_amdgcn_exp2f(ms[jj] - M);
      o[u] = os[(int64_t)jj * D + d];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += w[u] * o[u];
  }
  for (; j < np; j += NG) {
    const float w = j < kReduceWeightsLds ? w_s[j] : __builtin_amdgcn_exp2f(ms[j] - M);
    acc += w * os[(int64_t)j * D + d];
  }
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

template <int D, bool FP8, int TP, int RING>
static hipError_t launch_variant(const DecodeParams& p, int num_seqs, hipStream_t stream,
                                 hipEvent_t ev_before, hipEvent_t ev_after) {
  constexpr int NW = kSplitWaves;
  const dim3 grid((unsigned)p.num_parts, (unsigned)p.num_kv_heads, (unsigned)num_seqs);
  if (ev_before && ev_after) {
    // the events take the kernel's own start and end timestamps
    hipExtLaunchKernelGGL((paged_decode_split_kernel<D, FP8, NW, TP, RING>), grid,
                          dim3(NW * kWave), 0, stream, ev_before, ev_after, 0, p);
  } else {
    hipLaunchKernelGGL((paged_decode_split_kernel<D, FP8, NW, TP, RING>), grid,
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
// Default: 2-page tiles with one tile in flight (fp8 D <= 128, bf16 D = 64;
// the fastest shape measured on MI355X at 32k-128k), one buffer for the large
// tiles of bf16 D >= 128 and fp8 D = 256. KVFP8_SPLIT_VARIANT=TPxRING (2x1,
// 2x2, 2x3, 4x1, 4x2) overrides it for tuning sweeps.
template <int D, bool FP8>
static hipError_t launch_typed(const DecodeParams& p, int num_seqs, hipStream_t stream,
                               hipEvent_t ev_before, hipEvent_t ev_after) {
  int tp = 2, ring = (FP8 ? D <= 128 : D <= 64) ? 2 : 1;
  if (const char* env = getenv("KVFP8_SPLIT_VARIANT")) {
    int a = 0, c = 0;
    if (sscanf(env, "%dx%d", &a, &c) == 2) { tp = a; ring = c; }
  }
#define KVFP8_VARIANT(TP_, RING_)                                                    \
  if (tp == TP_ && ring == RING_)                                                    \
    return launch_variant<D, FP8, TP_, RING_>(p, num_seqs, stream, ev_before, ev_after);
  KVFP8_VARIANT(2, 1)
  KVFP8_VARIANT(2, 2)
  KVFP8_VARIANT(2, 3)
  KVFP8_VARIANT(4, 1)
  KVFP8_VARIANT(4, 2)
#undef KVFP8_VARIANT
  return hipErrorInvalidValue;
}

hipError_t launch_paged_decode(const DecodeParams& p, int head_dim, bool fp8,
                               int num_seqs, hipStream_t stream, hipEvent_t ev_before,
                               hipEvent_t ev_after) {
  switch (head_dim) {
    case 64:
      return fp8 ? launch_typed<64, true>(p, num_seqs, stream, ev_before, ev_after)
                 : launch_typed<64, false>(p, num_seqs, stream, ev_before, ev_after);
    case 128:
      return fp8 ? launch_typed<128, true>(p, num_seqs, stream, ev_before, ev_after)
                 : launch_typed<128, false>(p, num_seqs, stream, ev_before, ev_after);
    case 256:
      return fp8 ? launch_typed<256, true>(p, num_seqs, stream, ev_before, ev_after)
                 : launch_typed<256, false>(p, num_seqs, stream, ev_before, ev_after);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace kvfp8
