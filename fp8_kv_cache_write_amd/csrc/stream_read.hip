// stream_read.hip - a plain streaming read, the reference point for the
// split-decode kernel's bandwidth: every 16-byte chunk of a buffer is read
// once with a non-temporal load (as the split kernel reads pages) and folded
// into an XOR checksum, one 32-bit word per work-group. There is no other
// work, so its rate is what the chip's memory system gives a read-only
// stream.
#include <hip/hip_ext.h>

#include "launch.hpp"

namespace kvfp8 {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;   // 16-byte loads in flight per thread

__device__ inline uint32_t fold(u32x4 a) { return a.x ^ a.y ^ a.z ^ a.w; }

// Work-group w reads the contiguous chunks [w*per, min((w+1)*per, n16)) of
// the buffer, per = ceil(n16 / gridDim.x); consecutive threads read
// consecutive chunks, so each wave load covers 1 KiB.
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(
    const u32x4* __restrict__ src, int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t beg = (int64_t)blockIdx.x * per;
  const int64_t end = beg + per < n16 ? beg + per : n16;
  uint32_t acc = 0;
  int64_t i = beg + threadIdx.x;
  constexpr int64_t kStride = (int64_t)kStreamThreads * kStreamUnroll;
  for (; i + (kStreamUnroll - 1) * kStreamThreads < end; i += kStride) {
    u32x4 a[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u)
      a[u] = __builtin_nontemporal_load(src + i + u * kStreamThreads);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= fold(a[u]);
  }
  for (; i < end; i += kStreamThreads) acc ^= fold(__builtin_nontemporal_load(src + i));
  // XOR over the work-group: waves by shuffles, then one LDS word per wave
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t part[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x / 64] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kStreamThreads / 64; ++w) s ^= part[w];
    sink[blockIdx.x] = s;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t n_bytes, uint32_t* sink,
                              int num_blocks, hipStream_t stream, hipEvent_t ev_before,
                              hipEvent_t ev_after) {
  if (ev_before && ev_after) {
    // the events take the kernel's own start and end timestamps, as for the
    // split-decode kernel, so the two are timed alike
    hipExtLaunchKernelGGL(stream_read_kernel, dim3((unsigned)num_blocks), dim3(kStreamThreads),
                          0, stream, ev_before, ev_after, 0, static_cast<const u32x4*>(src),
                          n_bytes / 16, sink);
  } else {
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)num_blocks), dim3(kStreamThreads), 0,
                       stream, static_cast<const u32x4*>(src), n_bytes / 16, sink);
  }
  return hipGetLastError();
}

}  // namespace kvfp8
