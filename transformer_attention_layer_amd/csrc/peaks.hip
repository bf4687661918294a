// Measurement microkernels for gfx950: a bf16 MFMA-only loop and a
// streaming read, the measured counterparts of the published bf16 matrix
// and HBM peaks that the layer's kernels are reported against.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gqa_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;  // independent accumulators per wave

// Each wave: `iters` rounds of kChains independent 32x32x16 bf16 MFMAs on
// register operands.  The operands depend on the lane so the compiler can
// fold nothing; the accumulators are summed and stored at the end.
__global__ __launch_bounds__(256) void peak_mfma_kernel(int iters, float* sink) {
  const int tid = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f + 1e-3f * (float)((tid + i) & 7));
    b[i] = (__bf16)(1.0f - 1e-3f * (float)((tid * 3 + i) & 7));
  }
  floatx16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[(size_t)blockIdx.x * 256 + tid] = s;
}

constexpr int kUnroll = 8;  // 16-byte loads in flight per lane and trip

// Grid-stride streaming read: trip j of lane g reads the kUnroll 16-byte
// pieces g + (j * kUnroll + u) * stride, stride = all lanes of the grid, so
// every load instruction of a wave covers 1 KiB of consecutive bytes.
__global__ __launch_bounds__(256) void peak_read_kernel(const u32x4* buf, size_t n16,
                                                        uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  const size_t g = (size_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 x = {0u, 0u, 0u, 0u};
  for (size_t base = g; base < n16; base += stride * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + (size_t)u * stride;
      v[u] = i < n16 ? __builtin_nontemporal_load(buf + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= v[u];
  }
  sink[g] = x.x ^ x.y ^ x.z ^ x.w;
}

}  // namespace

extern "C" {

int gqa_peak_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream) {
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24) || !sink)
    return 1;
  hipLaunchKernelGGL(peak_mfma_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                     iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int gqa_peak_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink,
                         void* stream) {
  if (!buf || !sink || workgroups < 1 || workgroups > (1 << 20) || bytes == 0 ||
      bytes % 32768 != 0 || ((uintptr_t)buf & 15) != 0)
    return 1;
  hipLaunchKernelGGL(peak_read_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
