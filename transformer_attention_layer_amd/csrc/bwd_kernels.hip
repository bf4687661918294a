// Memory-bound helpers of the layer's backward pass on gfx950: the sum of
// split-K partial products, and a bf16 transpose that lays a token-major
// matrix out feature-major in token chunks (the K-contiguous operands of
// the weight-gradient GEMMs).
#include "common.h"
#include "kernels.h"

namespace gqa {
namespace {

// 64 x 64 tiles through LDS: 16-byte loads along the input rows, 16-byte
// stores along the output rows.  Output rows are written 8 input rows at a
// time; Rc is a multiple of 8, so such a group never straddles two chunks.
// Rows R .. S Rc - 1 (the last chunk's tail) are written as zeros.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16* __restrict__ in, int R,
                                                             int C, int Rc, int rows_out,
                                                             bf16* __restrict__ out) {
  __shared__ unsigned short tile[64][64 + 8];
  poison_lds(tile);
  const int c0 = blockIdx.x * 64;
  const int r0 = blockIdx.y * 64;
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = t / 8 + 32 * p;
    const int cg = (t % 8) * 8;
    const int r = r0 + row, c = c0 + cg;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < R && c < C) v = ld16(in + (size_t)r * C + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[row][cg + 2 * i] = (unsigned short)(v[i] & 0xffffu);
      tile[row][cg + 2 * i + 1] = (unsigned short)(v[i] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int col = t / 8 + 32 * p;
    const int rg = (t % 8) * 8;
    const int c = c0 + col;
    const int r = r0 + rg;
    if (c >= C || r >= rows_out) continue;
    const int s = r / Rc, rp = r - s * Rc;
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = (unsigned)tile[rg + 2 * i][col] | ((unsigned)tile[rg + 2 * i + 1][col] << 16);
    st16(out + ((size_t)s * C + c) * Rc + rp, v);
  }
}

__global__ __launch_bounds__(256) void sum_partials_kernel(const float* __restrict__ part, int S,
                                                           long long n, float* __restrict__ out) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  floatx4 acc = *reinterpret_cast<const floatx4*>(part + i);
  for (int s = 1; s < S; ++s) acc += *reinterpret_cast<const floatx4*>(part + (size_t)s * n + i);
  *reinterpret_cast<floatx4*>(out + i) = acc;
}

}  // namespace

hipError_t launch_transpose_bf16(const __bf16* in, int R, int C, int Rc, __bf16* out,
                                 hipStream_t stream) {
  if (Rc <= 0 || Rc % 8 != 0 || C % 8 != 0 || R < 0) return hipErrorInvalidValue;
  if (R == 0 || C == 0) return hipSuccess;
  const long long rows_out = (long long)((R + Rc - 1) / Rc) * Rc;
  const long long gy = (rows_out + 63) / 64;
  if (gy > 65535 || rows_out > 0x7fffffffLL) return hipErrorInvalidValue;
  dim3 grid((C + 63) / 64, (unsigned)gy);
  transpose_bf16_kernel<<<grid, 256, 0, stream>>>(in, R, C, Rc, (int)rows_out, out);
  return hipGetLastError();
}

hipError_t launch_sum_partials(const float* part, int S, long long n, float* out,
                               hipStream_t stream) {
  if (n % 4 != 0) return hipErrorInvalidValue;
  const long long blocks = (n / 4 + 255) / 256;
  sum_partials_kernel<<<(unsigned)blocks, 256, 0, stream>>>(part, S, n, out);
  return hipGetLastError();
}

}  // namespace gqa
