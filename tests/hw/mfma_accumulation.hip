// Accumulation precision of the gfx950 matrix instructions the kernels use.
//
// One wave forms C = A * B over 128 products per output (16 x 16 outputs)
// from random e4m3 codes, three ways: four chained bf16 16x16x32 MFMAs on
// the codes' exact bf16 values (the bf16-arithmetic paths), four chained
// fp8 16x16x32 MFMAs on the codes (the all-FP8 mode), and one fp8
// 16x16x128 MFMA (f8f6f4, neutral scales). Every product of two e4m3 values
// is exact in FP32, so any error is the instruction's summation. The host
// sums the same products in double (the reference) and in FP32 one by one.
// Printed: for each form, the largest |result - reference| divided by the
// sum of |products| of that output, over three code mixes (normal codes;
// normal times subnormal; both mixed); and, for the fp8 chain, the largest
// difference (same scale) between chaining the accumulator through the four
// MFMAs and adding each MFMA's own result in FP32. Two-level accumulation
// ("vLLM FP8 KV-Cache and Attention Quantization Update", section "Two-Level
// Accumulation for Accuracy"; the inference-research card
// "kv-cache-quantization-fp8-scale-granularity": Hopper's FP8 tensor cores
// keep intermediate sums at reduced precision) answers a short accumulator
// inside the matrix unit: this measures where these instructions round.
//
// Operand map: rows of A and columns of B are lane % 16; a lane's 32 bytes
// (16x16x128) are its k-group's codes, and chained step s takes bytes
// 8s .. 8s+7 of each lane: A and B use the same (lane, byte) -> k map, so the
// contraction covers all 128 pairs whatever the hardware's order. Outputs:
// lane l holds C[4 (l / 16) + i][l % 16], i = 0..3. One wave of 64 lanes;
// every buffer holds exactly 64 lanes' operands or results.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(64) void contract(const v8i* a, const v8i* b, v4f* c_k128,
                                               v4f* c_bf16, v4f* c_fp8, v4f* c_fold) {
  const int l = threadIdx.x;
  const v8i x = a[l], y = b[l];
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, acc, 0, 0, 0, 127, 0, 127);
  c_k128[l] = acc;
  // a8 chains the accumulator through the four fp8 MFMAs; f8 runs each
  // from zero and adds the four results in FP32
  v4f a16 = {0.f, 0.f, 0.f, 0.f}, a8 = {0.f, 0.f, 0.f, 0.f}, f8 = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < 4; ++s) {
    const unsigned xa = x[2 * s], xb = x[2 * s + 1], ya = y[2 * s], yb = y[2 * s + 1];
    bf16x8 A, B;
    for (int j = 0; j < 8; ++j) {
      const unsigned bx = ((j < 4 ? xa : xb) >> (8 * (j % 4))) & 0xffu;
      const unsigned by = ((j < 4 ? ya : yb) >> (8 * (j % 4))) & 0xffu;
      // exact: every e4m3 value is a bf16 value
      A[j] = (__bf16)__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(bx, 1.0f, false)[0];
      B[j] = (__bf16)__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(by, 1.0f, false)[0];
    }
    a16 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, a16, 0, 0, 0);
    a8 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)(((uint64_t)xb << 32) | xa),
                                                    (long)(((uint64_t)yb << 32) | ya), a8, 0, 0, 0);
    const v4f step = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
        (long)(((uint64_t)xb << 32) | xa), (long)(((uint64_t)yb << 32) | ya),
        v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    for (int e = 0; e < 4; ++e) f8[e] += step[e];
  }
  c_bf16[l] = a16;
  c_fp8[l] = a8;
  c_fold[l] = f8;
}

// e4m3 (OCP): bias 7, subnormals 2^-6 * m/8; the NaN codes are never drawn
static double e4m3(uint8_t v) {
  const int E = (v >> 3) & 15, M = v & 7;
  const double mag = E == 0 ? std::ldexp(M / 8.0, -6) : std::ldexp(1.0 + M / 8.0, E - 7);
  return (v & 0x80) ? -mag : mag;
}

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

int main() {
  std::mt19937 rng(2026);
  v8i *da, *db;
  v4f *dk, *d16, *d8, *df;
  CHECK(hipMalloc(&da, 64 * sizeof(v8i)));
  CHECK(hipMalloc(&db, 64 * sizeof(v8i)));
  CHECK(hipMalloc(&dk, 64 * sizeof(v4f)));
  CHECK(hipMalloc(&d16, 64 * sizeof(v4f)));
  CHECK(hipMalloc(&d8, 64 * sizeof(v4f)));
  CHECK(hipMalloc(&df, 64 * sizeof(v4f)));
  double worst[4] = {0, 0, 0, 0};   // f8f6f4 k128, fp8 4x k32, bf16 4x k32, FP32 sequential
  double chain_vs_fold = 0.0;       // fp8: accumulator chained vs each step added in FP32
  for (int mix = 0; mix < 3; ++mix) {
    // mix 0: normal codes; 1: A normal, B subnormal; 2: any non-NaN code
    auto draw = [&](bool subnormal_only) {
      for (;;) {
        const uint8_t v = (uint8_t)(rng() & 0xffu);
        const int E = (v >> 3) & 15;
        if ((v & 0x7f) == 0x7f) continue;
        if (subnormal_only && E != 0) continue;
        if (!subnormal_only && mix < 2 && E == 0) continue;
        return v;
      }
    };
    std::vector<uint8_t> A(64 * 32), B(64 * 32);
    for (auto& v : A) v = draw(false);
    for (auto& v : B) v = draw(mix == 1);
    CHECK(hipMemcpy(da, A.data(), A.size(), hipMemcpyHostToDevice));
    CHECK(hipMemcpy(db, B.data(), B.size(), hipMemcpyHostToDevice));
    contract<<<1, 64>>>(da, db, dk, d16, d8, df);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    std::vector<float> ck(256), c16(256), c8(256), cf(256);
    CHECK(hipMemcpy(ck.data(), dk, 1024, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(c16.data(), d16, 1024, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(c8.data(), d8, 1024, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(cf.data(), df, 1024, hipMemcpyDeviceToHost));
    for (int l = 0; l < 64; ++l)
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * (l / 16) + i, c = l % 16;
        double ref = 0.0, mag = 0.0;
        float seq = 0.0f;
        for (int g = 0; g < 4; ++g)
          for (int j = 0; j < 32; ++j) {
            const double p = e4m3(A[(16 * g + r) * 32 + j]) * e4m3(B[(16 * g + c) * 32 + j]);
            ref += p;
            mag += std::fabs(p);
            seq += (float)p;
          }
        if (mag == 0.0) continue;
        const double got[4] = {ck[l * 4 + i], c8[l * 4 + i], c16[l * 4 + i], seq};
        for (int f = 0; f < 4; ++f) worst[f] = std::fmax(worst[f], std::fabs(got[f] - ref) / mag);
        chain_vs_fold = std::fmax(chain_vs_fold, std::fabs((double)c8[l * 4 + i] - cf[l * 4 + i]) / mag);
      }
  }
  std::printf("{\"products_per_output\": 128, \"fp8_16x16x128\": %.4e, \"fp8_16x16x32_chain\": %.4e, "
              "\"bf16_16x16x32_chain\": %.4e, \"fp32_sequential\": %.4e, "
              "\"fp8_chain_minus_fp32_fold\": %.4e}\n",
              worst[0], worst[1], worst[2], worst[3], chain_vs_fold);
  return 0;
}
