// device_common.hpp - gfx950 device helpers shared by the kvfp8 kernels:
// vector types, the paged-cache layout, the e4m3 and e5m2 encoders and the
// exact fp8 -> bf16 expansions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvfp8 {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPage = 16;     // positions per page
constexpr int kWave = 64;     // CDNA wavefront

// Cache element formats (the values of the C ABI's kvq_dtype).
constexpr int kFmtBf16 = 0;
constexpr int kFmtE4M3 = 1;
constexpr int kFmtE5M2 = 2;

// ---------------------------------------------------------------------------
// Paged layout of one (page, kv head) block, e = element bytes (1 fp8, 2 bf16).
// K: 16-byte chunks of CE = 16/e consecutive dims of one row, chunk-major:
//      byte((r, d)) = ((d / CE) * 16 + r) * 16 + (d % CE) * e
// V: 1 KiB groups of DB = 64/e dims; inside a group 4 quads of rows, each
//    holding, for every dim, its 4 rows side by side:
//      byte((r, d)) = (d / DB) * 1024 + (r / 4) * 256 + (d % DB) * 4e + (r % 4) * e
// With these, lane l of a wave loading 16 bytes at 1024 * i + 16 * l gets
//   K: row l % 16, dims of chunk 4i + l / 16;
//   V: rows 4 * (l/16) .. +3, dims DB*i + (16/(4e)) * (l % 16) .. (4 or 2 dims)
// which is exactly what one lane feeds to a 16x16x32 MFMA (see the decode
// kernel), and every load instruction reads one contiguous 1 KiB span.
// ---------------------------------------------------------------------------
template <int E>
__device__ __forceinline__ uint32_t k_byte(int r, int d) {
  constexpr int CE = 16 / E;
  return ((uint32_t)(d / CE) * 16u + (uint32_t)r) * 16u + (uint32_t)(d % CE) * E;
}
template <int E>
__device__ __forceinline__ uint32_t v_byte(int r, int d) {
  constexpr int DB = 64 / E;
  return (uint32_t)(d / DB) * 1024u + (uint32_t)(r / 4) * 256u +
         (uint32_t)(d % DB) * (4u * E) + (uint32_t)(r % 4) * E;
}

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}

// ---------------------------------------------------------------------------
// fp32 -> e4m3 (OCP), saturating, round to nearest even.
// |y| >= 448 (and +-Inf) -> +-448; NaN -> 0x7F with the sign of y; the sign
// of zero is kept. Normal range: y = 2^E * f with f in [1, 2); f * 8 is
// rounded to an integer in [8, 16] by rintf (ties to even) and a result of 16
// moves to the next binade. Below 2^-6 the representable values are the
// multiples of 2^-9, so y * 2^9 is rounded directly. All scalings are by
// powers of two and exact.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_encode_sat(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __uint_as_float(u & 0x7FFFFFFFu);
  uint32_t mag;
  if (!(a == a)) {
    mag = 0x7Fu;                                   // NaN
  } else if (a >= 448.0f) {
    mag = 0x7Eu;                                   // saturate (Inf too)
  } else if (a < 0.015625f) {                      // 2^-6
    mag = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 9));   // 0..8
  } else {
    int ex = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // -6 .. 8
    uint32_t m8 = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - ex)); // 8..16
    if (m8 == 16u) { m8 = 8u; ex += 1; }
    mag = ((uint32_t)(ex + 7) << 3) | (m8 - 8u);   // ex + 7 in 1..15
    if (mag > 0x7Eu) mag = 0x7Eu;                  // 448 < a < 448 rounds up
  }
  return sign | mag;
}

// ---------------------------------------------------------------------------
// fp32 -> e5m2 (OCP), saturating, round to nearest even: the same scheme with
// 2 mantissa bits and bias 15. |y| >= 57344 (and +-Inf) -> +-57344 (0x7B,
// saturation as for e4m3); NaN -> 0x7F with the sign of y; below 2^-14 the
// representable values are the multiples of 2^-16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e5m2_encode_sat(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __uint_as_float(u & 0x7FFFFFFFu);
  uint32_t mag;
  if (!(a == a)) {
    mag = 0x7Fu;                                   // NaN
  } else if (a >= 57344.0f) {
    mag = 0x7Bu;                                   // saturate (Inf too)
  } else if (a < 6.103515625e-05f) {               // 2^-14
    mag = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 16));  // 0..4
  } else {
    int ex = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // -14 .. 15
    uint32_t m4 = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 2 - ex)); // 4..8
    if (m4 == 8u) { m4 = 4u; ex += 1; }
    mag = ((uint32_t)(ex + 15) << 2) | (m4 - 4u);  // ex + 15 in 1..30
    if (mag > 0x7Bu) mag = 0x7Bu;
  }
  return sign | mag;
}

// ---------------------------------------------------------------------------
// The same e4m3 conversion on the hardware converter: NaN keeps its sign
// (0x7F | sign), everything else is clamped to [-448, 448] (so +-Inf and
// finite overflow saturate) and converted by v_cvt_pk_fp8_f32, which rounds
// to nearest even and keeps the sign of zero. A GPU probe matched it with
// e4m3_encode_sat on every fp32 value in [-448.0005, 448.0005]; only the
// NaN codes differ, hence the NaN case first. About a third of the software
// encoder's instructions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_encode_sat_hw(float y) {
  if (!(y == y)) return ((__float_as_uint(y) >> 24) & 0x80u) | 0x7Fu;
  const float c = __builtin_fminf(__builtin_fmaxf(y, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}

// The same for e5m2 on v_cvt_pk_bf8_f32: NaN first, then a clamp to
// [-57344, 57344] (finite and infinite overflow saturate; the write never
// stores an infinity). Checked against e5m2_encode_sat on every fp32 value
// by the flat e5m2 quantiser's test.
__device__ __forceinline__ uint32_t e5m2_encode_sat_hw(float y) {
  if (!(y == y)) return ((__float_as_uint(y) >> 24) & 0x80u) | 0x7Fu;
  const float c = __builtin_fminf(__builtin_fmaxf(y, -57344.0f), 57344.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c, c, 0, false) & 0xFFu;
}

template <int FMT>
__device__ __forceinline__ uint32_t fp8_encode_sat(float y) {
  if constexpr (FMT == kFmtE5M2) return e5m2_encode_sat_hw(y);
  else return e4m3_encode_sat_hw(y);
}

// ---------------------------------------------------------------------------
// e4m3 -> bf16, exact (every e4m3 value, subnormals included, is a bf16
// value). gfx950 converts two codes of a dword per instruction; the scale
// operand 1.0 leaves the values unchanged. NaN codes give NaN.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x2 e4m3x2_to_bf16x2(uint32_t w, bool high_pair) {
  return high_pair ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                   : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
}

__device__ __forceinline__ bf16x4 e4m3x4_to_bf16x4(uint32_t w) {
  bf16x2 lo = e4m3x2_to_bf16x2(w, false);
  bf16x2 hi = e4m3x2_to_bf16x2(w, true);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
}

__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  bf16x4 a = e4m3x4_to_bf16x4(w0);
  bf16x4 b = e4m3x4_to_bf16x4(w1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// e5m2 -> bf16, exact likewise (bf16 has the wider exponent; e5m2 infinities
// and NaNs stay infinities and NaNs).
__device__ __forceinline__ bf16x2 e5m2x2_to_bf16x2(uint32_t w, bool high_pair) {
  return high_pair ? __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, true)
                   : __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, false);
}

// Four / eight codes of either fp8 format to bf16.
template <int FMT>
__device__ __forceinline__ bf16x4 fp8x4_to_bf16x4(uint32_t w) {
  bf16x2 lo, hi;
  if constexpr (FMT == kFmtE5M2) {
    lo = e5m2x2_to_bf16x2(w, false);
    hi = e5m2x2_to_bf16x2(w, true);
  } else {
    lo = e4m3x2_to_bf16x2(w, false);
    hi = e4m3x2_to_bf16x2(w, true);
  }
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
}

template <int FMT>
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  bf16x4 a = fp8x4_to_bf16x4<FMT>(w0);
  bf16x4 b = fp8x4_to_bf16x4<FMT>(w1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------------------
// Max over the four lanes c, c+16, c+32, c+48 that hold one column of a
// 16x16 MFMA tile, with the gfx950 row swaps (VALU, no LDS round trip).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float mfma_col_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Largest magnitude of 8 bf16 values (one 16-byte word) as bf16 bits: each
// half-word is masked and compared on its own, so as integers NaN > Inf >
// every finite value.
__device__ __forceinline__ uint32_t max_mag_bits8(uint4 w) {
  const uint32_t a = max(max(w.x & 0x7FFFu, (w.x >> 16) & 0x7FFFu),
                         max(w.y & 0x7FFFu, (w.y >> 16) & 0x7FFFu));
  const uint32_t b = max(max(w.z & 0x7FFFu, (w.z >> 16) & 0x7FFFu),
                         max(w.w & 0x7FFFu, (w.w >> 16) & 0x7FFFu));
  return max(a, b);
}

// ---------------------------------------------------------------------------
// All-FP8 attention: one query row as e4m3 codes with s_q = amax / 448 (the
// 4 lanes of an MFMA column hold the row, NK pieces of 8 values each; the
// codes go out as 8-byte fp8 MFMA operands in the same order). Returns s_q.
//   The codes are those of the IEEE quotient x / s_q. With r = 1 / s_q
// (correctly rounded), q0 = x r, e = fma(-q0, s_q, x), fma(e, r, q0) is that
// quotient by Markstein's theorem when nothing underflows; checked
// exhaustively over every bf16 amax and every bf16 x with |x| <= amax, the
// e4m3 codes of the two agree for all s_q >= 2^-100 (and the quotients
// themselves wherever they reach 2^-12). A row with a smaller or non-finite
// scale, or a NaN element, takes the division (the wave as a whole). The
// hardware conversion (round to nearest even) gives the saturating encoder's
// codes on [-448, 448] and just beyond, where the quotients lie (checked for
// every fp32 value there); only the NaN codes differ, hence NaN rows divide.
// ---------------------------------------------------------------------------
template <int NK>
__device__ __forceinline__ float quantize_q_e4m3(const bf16x8 (&q)[NK], uint64_t (&q8)[NK]) {
  float am = 0.0f;
  uint32_t mag = 0u;                               // largest |x| bits: NaN > Inf > finite
#pragma unroll
  for (int s = 0; s < NK; ++s) {
#pragma unroll
    for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf((float)q[s][j]));
    mag = max(mag, max_mag_bits8(__builtin_bit_cast(uint4, q[s])));
  }
  am = mfma_col_max(am);
  const float q_scale = am == 0.0f ? 1.0f : am / 448.0f;
  const bool fast = q_scale >= 0x1p-100f && q_scale <= 0x1p+120f && mag <= 0x7F80u;
  if (__builtin_amdgcn_ballot_w64(!fast) == 0ull) {
    const float r = 1.0f / q_scale;
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      float qq[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = (float)q[s][j];
        const float q0 = x * r;
        qq[j] = __builtin_fmaf(__builtin_fmaf(-q0, q_scale, x), r, q0);
      }
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(qq[0], qq[1], 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(qq[2], qq[3], lo, true);
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(qq[4], qq[5], 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(qq[6], qq[7], hi, true);
      q8[s] = ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
    }
  } else {
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      uint64_t w = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        w |= (uint64_t)e4m3_encode_sat((float)q[s][j] / q_scale) << (8 * j);
      q8[s] = w;
    }
  }
  return q_scale;
}

__device__ __forceinline__ bf16x8 bits_to_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x4 bits_to_bf16x4(uint32_t a, uint32_t b) {
  uint2 t = make_uint2(a, b);
  return __builtin_bit_cast(bf16x4, t);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace kvfp8
