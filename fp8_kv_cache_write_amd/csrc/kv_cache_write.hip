// kv_cache_write.hip - quantise new tokens' K/V into the paged cache (gfx950),
// plus the static amax/fmax scale calibration and the flat fp8 quantiser, for
// the e4m3 and e5m2 formats.
//
// The write is the cache-write kernel of "State of FP8 KV cache and attention
// quantization in vLLM" (section "Kernel and vLLM improvements", paragraph
// "Per-head scales": one FP32 scale per KV head instead of a scalar); the
// conversion is "FP8量化与长上下文推理" section 1.1 (q = round(x / s)) with the
// saturating mode of "cooking-agi: FP8 and the KV cache" (section "dynamic vs
// static scale"); e5m2 is the same page's second fp8 cache dtype (section "how
// to enable it in the engine").
#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

namespace kvfp8 {

// Quantise 16 bf16 values (two 16-byte words) to 16 codes: 4 words, byte b of
// word j the code of element 4j + b.
template <int FMT>
__device__ __forceinline__ void quantize16(const uint32_t* w, float s, uint32_t (&q)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t o = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int e = j * 4 + b;
      const uint32_t bits = (w[e / 2] >> (16 * (e % 2))) & 0xFFFFu;
      o |= fp8_encode_sat<FMT>(bf16_bits_to_f32(bits) / s) << (8 * b);
    }
    q[j] = o;
  }
}

// Lanes of one wave exchange words through LDS: the fences and the wave
// barrier keep the compiler from moving the LDS accesses across it; the LDS
// itself serves one wave's accesses in order.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kWriteThreads = 256;

// Four lanes per (quad of tokens, kv head, 16-dim chunk): lane j of a quad
// handles token 4*tq + j. Each lane reads 16 bf16 of K and of V (two 16-byte
// loads each) and writes
//   fp8 : K as one 16-byte store (one layout chunk). V: when the quad's four
//         tokens go to four consecutive slots starting at a multiple of 4 (a
//         row quad of one page, as a prefill writes them), the lanes swap
//         their codes through LDS and lane j stores the 16 bytes of dims
//         4j .. 4j+3 of the chunk for all four rows; otherwise 16 byte stores
//         (the V layout interleaves 4 rows per dim, so a row's dims are 4
//         bytes apart);
//   bf16: K as two 16-byte stores, V as 16 two-byte stores.
template <int FMT>
__global__ __launch_bounds__(kWriteThreads) void kv_cache_write_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int64_t* __restrict__ slots, int64_t num_tokens, int num_kv_heads,
    int head_dim, uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    int64_t num_pages, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, int scale_per_head) {
  constexpr bool FP8 = FMT != kFmtBf16;
  constexpr int E = FP8 ? 1 : 2;
  const int chunks = head_dim / 16;
  const int64_t quads = (num_tokens + 3) / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = quads * 4 * num_kv_heads * chunks;
  const int j = (int)(gid & 3);
  const int64_t rest = gid >> 2;
  const int c = (int)(rest % chunks);
  const int64_t th = rest / chunks;
  const int h = (int)(th % num_kv_heads);
  const int64_t t = (th / num_kv_heads) * 4 + j;
  // no lane returns before the quad's ballot: every lane of a wave takes part
  const bool live = gid < total && t < num_tokens;
  const int64_t slot = live ? slots[t] : -1;
  const bool ok = slot >= 0 && slot < num_pages * kPage;   // else skipped / outside the pool
  const int64_t page = ok ? slot / kPage : 0;
  const int r = (int)(slot & (kPage - 1));
  const int64_t pb = (int64_t)kPage * head_dim * E;
  uint8_t* kb = k_cache + (page * num_kv_heads + h) * pb;
  uint8_t* vb = v_cache + (page * num_kv_heads + h) * pb;
  const int d0 = c * 16;

  uint4 kx[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
  uint4 vx[2] = {kx[0], kx[1]};
  if (ok) {
    const int64_t src = (t * num_kv_heads + h) * head_dim + (int64_t)c * 16;
    const uint4* ks = reinterpret_cast<const uint4*>(k + src);
    const uint4* vs = reinterpret_cast<const uint4*>(v + src);
    kx[0] = ks[0];
    kx[1] = ks[1];
    vx[0] = vs[0];
    vx[1] = vs[1];
  }
  const uint32_t* kw = reinterpret_cast<const uint32_t*>(kx);
  const uint32_t* vw = reinterpret_cast<const uint32_t*>(vx);

  if constexpr (FP8) {
    const float sk = k_scale[scale_per_head ? h : 0];
    const float sv = v_scale[scale_per_head ? h : 0];
    // lane j's slot must be the quad's first slot + j, that slot a multiple of 4
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t slot0 = __shfl(slot, lane & ~3);
    const bool run = ok && slot == slot0 + j && (slot0 & 3) == 0;
    const uint64_t bal = __ballot(run);
    const bool quad = ((bal >> (lane & ~3)) & 0xFull) == 0xFull;
    uint32_t kq[4], vq[4];
    quantize16<FMT>(kw, sk, kq);
    quantize16<FMT>(vw, sv, vq);
    if (ok)
      *reinterpret_cast<uint4*>(kb + k_byte<1>(r, d0)) = make_uint4(kq[0], kq[1], kq[2], kq[3]);
    // [lane / 4][row j][word]: the quad's codes, four words per row
    __shared__ uint32_t xchg[kWriteThreads / 4][4][4];
    const int qi = threadIdx.x >> 2;
#pragma unroll
    for (int w = 0; w < 4; ++w) xchg[qi][j][w] = vq[w];
    wave_lds_sync();
    if (quad) {
      // lane j: dims 4j .. 4j+3 of the chunk, rows r-j .. r-j+3 (one 16-byte span)
      uint32_t W[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) W[i] = xchg[qi][i][j];
      uint32_t o[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        o[b] = ((W[0] >> (8 * b)) & 0xFFu) | (((W[1] >> (8 * b)) & 0xFFu) << 8) |
               (((W[2] >> (8 * b)) & 0xFFu) << 16) | (((W[3] >> (8 * b)) & 0xFFu) << 24);
      *reinterpret_cast<uint4*>(vb + v_byte<1>(r - j, d0 + 4 * j)) =
          make_uint4(o[0], o[1], o[2], o[3]);
    } else if (ok) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        vb[v_byte<1>(r, d0 + e)] = (uint8_t)(vq[e / 4] >> (8 * (e % 4)));
    }
  } else {
    if (!ok) return;
    // bf16 layers keep the bits: the skip-layer path.
    *reinterpret_cast<uint4*>(kb + k_byte<2>(r, d0)) = kx[0];
    *reinterpret_cast<uint4*>(kb + k_byte<2>(r, d0 + 8)) = kx[1];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t bits = (vw[e / 2] >> (16 * (e % 2))) & 0xFFFFu;
      *reinterpret_cast<uint16_t*>(vb + v_byte<2>(r, d0 + e)) = (uint16_t)bits;
    }
  }
}

// Largest |x| of 16 bf16 values (two 16-byte words each of K and V) as bf16
// magnitude bits: the integer order of those bits is the order of the
// magnitudes with NaN above Inf above every finite value.
__device__ __forceinline__ uint32_t max_mag_bits(const uint32_t* w) {
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  return m;
}

// Cache write with dynamic per-token scales ("FP8量化与长上下文推理" section
// 2.2: every new token gets its own scale): one work-group per token. Pass 1
// takes the token's largest |x| of K and of V - over each KV head, or over
// all of them (ALL_HEADS) - as an LDS integer max of magnitude bits; pass 2
// sets s = amax / fmax (1 when amax is 0, NaN when a NaN is present: the
// static calibration's rule), stores it beside the page for the slot
// (pool[page][head][row]) and writes the codes as the static write does.
constexpr int kMaxDynHeads = 256;
template <int FMT, bool ALL_HEADS>
__global__ __launch_bounds__(kWriteThreads) void kv_cache_write_dyn_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int64_t* __restrict__ slots, int64_t num_tokens, int num_kv_heads, int head_dim,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, int64_t num_pages,
    float* __restrict__ k_pool, float* __restrict__ v_pool) {
  // One work-group per quad of tokens; item it = 4 * (head, chunk) + j is
  // token 4 * blockIdx.x + j, so the four tokens of a quad sit in adjacent
  // lanes as in the static write.
  constexpr float fmax = FMT == kFmtE5M2 ? 57344.0f : 448.0f;
  const int64_t t0 = (int64_t)blockIdx.x * 4;
  const int chunks = head_dim / 16;
  const int items4 = 4 * num_kv_heads * chunks;
  __shared__ uint32_t km[4][kMaxDynHeads], vm[4][kMaxDynHeads];
  __shared__ uint32_t xchg[kWriteThreads / 4][4][4];
  for (int i = threadIdx.x; i < 4 * num_kv_heads; i += blockDim.x)
    km[i / num_kv_heads][i % num_kv_heads] = vm[i / num_kv_heads][i % num_kv_heads] = 0u;
  __syncthreads();
  // pass 1: the largest magnitude of each token's K and V (per head, or over
  // all heads), as integer maxima of bf16 magnitude bits
  for (int it = threadIdx.x; it < items4; it += blockDim.x) {
    const int j = it & 3, item = it >> 2;
    const int64_t t = t0 + j;
    if (t >= num_tokens) continue;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_pages * kPage) continue;   // the token is skipped
    const int h = item / chunks;
    const int64_t src = (t * num_kv_heads + h) * head_dim + (int64_t)(item % chunks) * 16;
    const uint4* ks = reinterpret_cast<const uint4*>(k + src);
    const uint4* vs = reinterpret_cast<const uint4*>(v + src);
    const uint4 kx[2] = {ks[0], ks[1]}, vx[2] = {vs[0], vs[1]};
    atomicMax(&km[j][ALL_HEADS ? 0 : h], max_mag_bits(reinterpret_cast<const uint32_t*>(kx)));
    atomicMax(&vm[j][ALL_HEADS ? 0 : h], max_mag_bits(reinterpret_cast<const uint32_t*>(vx)));
  }
  __syncthreads();
  // pass 2: s = amax / fmax (1 for zero, NaN for NaN), the pools, the codes
  const int64_t pb = (int64_t)kPage * head_dim;
  const int lane = threadIdx.x & (kWave - 1);
  const int qi = threadIdx.x >> 2;
  for (int it = threadIdx.x; it < items4; it += blockDim.x) {
    const int j = it & 3, item = it >> 2;
    const int h = item / chunks, c = item % chunks;
    const int64_t t = t0 + j;
    const int64_t slot = t < num_tokens ? slots[t] : -1;
    const bool ok = slot >= 0 && slot < num_pages * kPage;
    const int64_t page = ok ? slot / kPage : 0;
    const int r = (int)(slot & (kPage - 1));
    const float ak = bf16_bits_to_f32(km[j][ALL_HEADS ? 0 : h]);
    const float av = bf16_bits_to_f32(vm[j][ALL_HEADS ? 0 : h]);
    const float sk = ak == 0.0f ? 1.0f : ak / fmax;
    const float sv = av == 0.0f ? 1.0f : av / fmax;
    uint4 kx[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
    uint4 vx[2] = {kx[0], kx[1]};
    if (ok) {
      const int64_t src = (t * num_kv_heads + h) * head_dim + (int64_t)c * 16;
      const uint4* ks = reinterpret_cast<const uint4*>(k + src);
      const uint4* vs = reinterpret_cast<const uint4*>(v + src);
      kx[0] = ks[0];
      kx[1] = ks[1];
      vx[0] = vs[0];
      vx[1] = vs[1];
    }
    uint32_t kq[4], vq[4];
    quantize16<FMT>(reinterpret_cast<const uint32_t*>(kx), sk, kq);
    quantize16<FMT>(reinterpret_cast<const uint32_t*>(vx), sv, vq);
    uint8_t* kb = k_cache + (page * num_kv_heads + h) * pb;
    uint8_t* vb = v_cache + (page * num_kv_heads + h) * pb;
    const int d0 = c * 16;
    if (ok) {
      *reinterpret_cast<uint4*>(kb + k_byte<1>(r, d0)) = make_uint4(kq[0], kq[1], kq[2], kq[3]);
      if (c == 0) {
        k_pool[(page * num_kv_heads + h) * kPage + r] = sk;
        v_pool[(page * num_kv_heads + h) * kPage + r] = sv;
      }
    }
    // V: 16-byte spans when the quad's tokens fill one row quad (see the
    // static write), else byte stores
    const int64_t slot0 = __shfl(slot, lane & ~3);
    const bool run = ok && slot == slot0 + j && (slot0 & 3) == 0;
    const uint64_t bal = __ballot(run);
    const bool quad = ((bal >> (lane & ~3)) & 0xFull) == 0xFull;
#pragma unroll
    for (int w = 0; w < 4; ++w) xchg[qi][j][w] = vq[w];
    wave_lds_sync();
    if (quad) {
      uint32_t W[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) W[i] = xchg[qi][i][j];
      uint32_t o[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        o[b] = ((W[0] >> (8 * b)) & 0xFFu) | (((W[1] >> (8 * b)) & 0xFFu) << 8) |
               (((W[2] >> (8 * b)) & 0xFFu) << 16) | (((W[3] >> (8 * b)) & 0xFFu) << 24);
      *reinterpret_cast<uint4*>(vb + v_byte<1>(r - j, d0 + 4 * j)) =
          make_uint4(o[0], o[1], o[2], o[3]);
    } else if (ok) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        vb[v_byte<1>(r, d0 + e)] = (uint8_t)(vq[e / 4] >> (8 * (e % 4)));
    }
    wave_lds_sync();   // this round's reads before the next round's writes
  }
}

// Static scale calibration: s[o] = fp32(amax) / fmax over the bf16 tensor
// x [T][Hkv][D], per KV head (o = head) or per tensor (one o over every
// head); fmax = 448 (e4m3) or 57344 (e5m2). NaN anywhere gives NaN, amax ==
// 0 gives 1. Three launches, no workspace: the output words are cleared,
// then many work-groups per output fold the largest bf16 magnitude bits of
// their share into them with an integer atomicMax (as integers those bits
// order NaN above Inf above every finite value), then the bits become the
// scale.
constexpr int kAmaxThreads = 256;

__global__ void amax_clear_kernel(uint32_t* __restrict__ bits, int n_out) {
  const int o = blockIdx.x * blockDim.x + threadIdx.x;
  if (o < n_out) bits[o] = 0u;
}

// Work-group (s, o) folds tokens [s * tps, (s + 1) * tps) of output o.
__global__ __launch_bounds__(kAmaxThreads) void amax_bits_kernel(
    const uint16_t* __restrict__ x, int64_t num_tokens, int num_kv_heads, int head_dim,
    int per_head, int64_t tps, uint32_t* __restrict__ bits) {
  const int o = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * tps;
  const int64_t t1 = t0 + tps < num_tokens ? t0 + tps : num_tokens;
  // 16-byte chunks of one token that belong to output o, and where they start
  const int chunks = (per_head ? 1 : num_kv_heads) * (head_dim / 8);
  const int64_t row = (int64_t)num_kv_heads * head_dim;            // bf16 per token
  const int64_t first = per_head ? (int64_t)o * head_dim : 0;
  uint32_t m = 0u;
  if (t1 > t0) {
    const int64_t n = (t1 - t0) * chunks;
    for (int64_t i = threadIdx.x; i < n; i += kAmaxThreads) {
      const int64_t t = t0 + i / chunks;
      const int c = (int)(i % chunks);
      const uint4 w = *reinterpret_cast<const uint4*>(x + t * row + first + (int64_t)c * 8);
      m = max(m, max_mag_bits8(w));
    }
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t red[kAmaxThreads / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kAmaxThreads / kWave; ++w) m = max(m, red[w]);
    if (m != 0u) atomicMax(&bits[o], m);
  }
}

__global__ void amax_finish_kernel(uint32_t* __restrict__ bits, int n_out, float fmax) {
  const int o = blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= n_out) return;
  const uint32_t b = bits[o];
  float s;
  if (b > 0x7F80u) s = __builtin_nanf("");        // a NaN was present
  else if (b == 0u) s = 1.0f;                     // all zero
  else s = bf16_bits_to_f32(b) / fmax;            // Inf gives Inf
  reinterpret_cast<float*>(bits)[o] = s;
}

// Flat quantiser: out[i] = fp8(x[i] / s), 4 elements per thread.
template <int FMT>
__global__ __launch_bounds__(256) void quantize_kernel(
    const float* __restrict__ x, int64_t n, const float* __restrict__ scale,
    uint8_t* __restrict__ out) {
  const float s = scale[0];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i * 4 < n;
       i += stride) {
    const int64_t base = i * 4;
    if (base + 4 <= n) {
      const float4 f = *reinterpret_cast<const float4*>(x + base);
      const uint32_t w = fp8_encode_sat<FMT>(f.x / s) | (fp8_encode_sat<FMT>(f.y / s) << 8) |
                         (fp8_encode_sat<FMT>(f.z / s) << 16) |
                         (fp8_encode_sat<FMT>(f.w / s) << 24);
      *reinterpret_cast<uint32_t*>(out + base) = w;
    } else {
      for (int64_t j = base; j < n; ++j) out[j] = (uint8_t)fp8_encode_sat<FMT>(x[j] / s);
    }
  }
}

hipError_t launch_kv_cache_write(int fmt, const uint16_t* k, const uint16_t* v,
                                 const int64_t* slots, int64_t num_tokens,
                                 int num_kv_heads, int head_dim, uint8_t* k_cache,
                                 uint8_t* v_cache, int64_t num_pages,
                                 const float* k_scale, const float* v_scale,
                                 int scale_per_head, hipStream_t stream) {
  // four lanes per quad of tokens (the last quad may be partial)
  const int64_t total = (num_tokens + 3) / 4 * 4 * num_kv_heads * (head_dim / 16);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + kWriteThreads - 1) / kWriteThreads;
  if (fmt == kFmtE4M3)
    hipLaunchKernelGGL(kv_cache_write_kernel<kFmtE4M3>, dim3((unsigned)blocks), dim3(kWriteThreads),
                       0, stream, k, v, slots, num_tokens, num_kv_heads, head_dim,
                       k_cache, v_cache, num_pages, k_scale, v_scale, scale_per_head);
  else if (fmt == kFmtE5M2)
    hipLaunchKernelGGL(kv_cache_write_kernel<kFmtE5M2>, dim3((unsigned)blocks), dim3(kWriteThreads),
                       0, stream, k, v, slots, num_tokens, num_kv_heads, head_dim,
                       k_cache, v_cache, num_pages, k_scale, v_scale, scale_per_head);
  else if (fmt == kFmtBf16)
    hipLaunchKernelGGL(kv_cache_write_kernel<kFmtBf16>, dim3((unsigned)blocks), dim3(kWriteThreads),
                       0, stream, k, v, slots, num_tokens, num_kv_heads, head_dim,
                       k_cache, v_cache, num_pages, k_scale, v_scale, scale_per_head);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_scale_from_amax(const uint16_t* x, int64_t num_tokens,
                                  int num_kv_heads, int head_dim, int per_head,
                                  float fmax, float* scale_out, hipStream_t stream) {
  const int n_out = per_head ? num_kv_heads : 1;
  const dim3 small((unsigned)((n_out + 255) / 256)), small_block(256);
  uint32_t* bits = reinterpret_cast<uint32_t*>(scale_out);   // holds magnitude bits meanwhile
  hipLaunchKernelGGL(amax_clear_kernel, small, small_block, 0, stream, bits, n_out);
  if (num_tokens > 0) {
    // about 1024 work-groups in all, each a contiguous run of tokens
    const int64_t slices = std::max<int64_t>(1, std::min<int64_t>(num_tokens, 1024 / n_out));
    const int64_t tps = (num_tokens + slices - 1) / slices;
    const int64_t used = (num_tokens + tps - 1) / tps;
    hipLaunchKernelGGL(amax_bits_kernel, dim3((unsigned)used, (unsigned)n_out),
                       dim3(kAmaxThreads), 0, stream, x, num_tokens, num_kv_heads, head_dim,
                       per_head, tps, bits);
  }
  hipLaunchKernelGGL(amax_finish_kernel, small, small_block, 0, stream, bits, n_out, fmax);
  return hipGetLastError();
}

hipError_t launch_quantize(int fmt, const float* x, int64_t n, const float* scale,
                           uint8_t* out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  int64_t groups = (n + 3) / 4;
  int64_t blocks = (groups + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (fmt == kFmtE5M2)
    hipLaunchKernelGGL(quantize_kernel<kFmtE5M2>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       x, n, scale, out);
  else
    hipLaunchKernelGGL(quantize_kernel<kFmtE4M3>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       x, n, scale, out);
  return hipGetLastError();
}

hipError_t launch_kv_cache_write_dyn(int fmt, const uint16_t* k, const uint16_t* v,
                                     const int64_t* slots, int64_t num_tokens, int num_kv_heads,
                                     int head_dim, uint8_t* k_cache, uint8_t* v_cache,
                                     int64_t num_pages, float* k_pool, float* v_pool,
                                     int all_heads, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  if (num_kv_heads > kMaxDynHeads || num_tokens > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  // one work-group per quad of tokens, four lanes per (head, 16-dim chunk)
  const int items4 = 4 * num_kv_heads * (head_dim / 16);
  const int threads = std::min(kWriteThreads, (items4 + kWave - 1) / kWave * kWave);
  const dim3 grid((unsigned)((num_tokens + 3) / 4)), block((unsigned)threads);
#define KVFP8_DYN(F, A)                                                                      \
  hipLaunchKernelGGL((kv_cache_write_dyn_kernel<F, A>), grid, block, 0, stream, k, v, slots, \
                     num_tokens, num_kv_heads, head_dim, k_cache, v_cache, num_pages,         \
                     k_pool, v_pool)
  if (fmt == kFmtE4M3) {
    if (all_heads) KVFP8_DYN(kFmtE4M3, true); else KVFP8_DYN(kFmtE4M3, false);
  } else if (fmt == kFmtE5M2) {
    if (all_heads) KVFP8_DYN(kFmtE5M2, true); else KVFP8_DYN(kFmtE5M2, false);
  } else {
    return hipErrorInvalidValue;
  }
#undef KVFP8_DYN
  return hipGetLastError();
}

}  // namespace kvfp8
