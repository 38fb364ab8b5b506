// Reference kernels for the achieved peaks of one MI355X (include/qlin_peaks.h):
// an HBM streaming read and a matrix-core-only loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qlin_peaks.h"

namespace {

constexpr int kReadGroups = 16384;
constexpr int kReadInFlight = 16;          // 16-byte loads in flight per thread
constexpr int kMfmaGroups = 512;           // 2 per CU
constexpr int kMfmaThreads = 256;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Each work-group reads one contiguous chunk of n16 / gridDim.x words (the
// last one also the remainder): sequential addresses per work-group keep
// every HBM page busy with fewer row switches than a grid-stride sweep.
__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ src, int64_t n16,
                                                     uint32_t* __restrict__ sink) {
  const int64_t per = n16 / gridDim.x;
  const int64_t begin = (int64_t)blockIdx.x * per;
  const int64_t end = blockIdx.x + 1 == gridDim.x ? n16 : begin + per;
  const uint4* p = src + begin;
  const int64_t len = end - begin;
  uint32_t acc = 0;
  int64_t i = threadIdx.x;
  for (; i + (kReadInFlight - 1) * 256 < len; i += kReadInFlight * 256) {
    uint4 v[kReadInFlight];
#pragma unroll
    for (int l = 0; l < kReadInFlight; ++l) v[l] = p[i + l * 256];
#pragma unroll
    for (int l = 0; l < kReadInFlight; ++l) acc ^= v[l].x ^ v[l].y ^ v[l].z ^ v[l].w;
  }
  for (; i < len; i += 256) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < 256; ++t) r ^= red[t];
    sink[blockIdx.x] = r;
  }
}

__global__ __launch_bounds__(kMfmaThreads) void k_mfma_loop(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (float)(lane + i));
    b[i] = (_Float16)(0.002f * (float)(lane - i));
  }
  f32x16 acc[8];
  for (int t = 0; t < 8; ++t)
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[t], 0, 0, 0);
  }
  float s = 0.f;
  for (int t = 0; t < 8; ++t) s += acc[t][lane & 15];
  if (lane == 0) sink[blockIdx.x * (kMfmaThreads / 64) + (threadIdx.x >> 6)] = s;
}

}  // namespace

extern "C" {

int64_t qlin_peak_read_groups(void) { return kReadGroups; }

int qlin_peak_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (src == nullptr || sink == nullptr || bytes <= 0 || (bytes & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0 || bytes / 16 < kReadGroups)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_stream_read, dim3(kReadGroups), dim3(256), 0, stream,
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return (int)hipGetLastError();
}

int64_t qlin_peak_mfma_waves(void) { return (int64_t)kMfmaGroups * (kMfmaThreads / 64); }

int qlin_peak_mfma(int32_t iters, float* sink, hipStream_t stream) {
  if (sink == nullptr || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mfma_loop, dim3(kMfmaGroups), dim3(kMfmaThreads), 0, stream, iters, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
