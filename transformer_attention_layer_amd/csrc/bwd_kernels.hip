// Memory-bound kernels of the layer's backward pass on gfx950:
//   * the backward through RoPE and the per-head QK-norm (tutorial "Multi-Head
//     and Grouped-Query Attention (Full Layer)", section 4 steps 2-3; section 3
//     for the per-head norm), producing the gradient of the fused projection
//     output and per-block partial sums of the two norm-weight gradients;
//   * the sum of those partials, the sum of split-K partial products, and a
//     bf16 transpose that lays a token-major matrix out feature-major in
//     token chunks (the K-contiguous operands of the weight-gradient GEMMs).
#include "common.h"
#include "kernels.h"

namespace gqa {
namespace {

GQA_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// A block of 4 waves takes kNormRopeBwdTokens tokens; wave w handles the
// rows (token, head) with head = w, w + 4, ... of the fused projection's
// Hq + 2 Hkv heads.  Lane l holds features l + 64 i (d <= 256).
//
// With g the gradient of a head's rotated output:
//   RoPE: pair (e, e + r/2) was turned by [[c, -s], [s, c]], so the
//         gradient of the normalised value is [[c, s], [-s, c]] g
//         (features past the rotary width r pass through);
//   norm: out_e = y_e r w_e with r = (mean(y^2) + eps)^(-1/2), so
//         dy_e = r (w_e dn_e - y_e r^2 mean(w dn y)) and the weight gets
//         dn_e y_e r, summed over every token and head.
// V heads pass their gradient through.  The partner of a rotary pair may
// sit in another lane, so a wave's gradient row goes through its own LDS
// row (a wave's LDS accesses complete in order).
__global__ __launch_bounds__(256) void normrope_bwd_kernel(NormRopeBwdArgs a) {
  __shared__ float xs[4][256];
  __shared__ float red[4][2][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d = a.d, rh = a.rot >> 1;
  const int nh = a.Hq + 2 * a.Hkv;
  const int T = a.B * a.L;
  const size_t n_qkv = (size_t)nh * d;
  float gw[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const int m0 = blockIdx.x * kNormRopeBwdTokens;
  for (int tt = 0; tt < kNormRopeBwdTokens; ++tt) {
    const int m = m0 + tt;
    if (m >= T) break;
    const int b = m / a.L, tok = m - b * a.L;
    for (int head = wave; head < nh; head += 4) {
      int kind, h;
      if (head < a.Hq) { kind = 0; h = head; }
      else if (head < a.Hq + a.Hkv) { kind = 1; h = head - a.Hq; }
      else { kind = 2; h = head - a.Hq - a.Hkv; }
      const float* g = kind == 0   ? a.dq + (((size_t)b * a.Hq + h) * a.L + tok) * d
                       : kind == 1 ? a.dk + (((size_t)b * a.Hkv + h) * a.L + tok) * d
                                   : a.dv + (((size_t)b * a.Hkv + h) * a.L + tok) * d;
      bf16* dst = a.dy + (size_t)m * n_qkv + (size_t)head * d;
      float gv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        gv[i] = e < d ? g[e] : 0.f;
      }
      if (kind == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = lane + 64 * i;
          if (e < d) dst[e] = (bf16)gv[i];
        }
        continue;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        if (e < d) xs[wave][e] = gv[i];
      }
      float dn[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        dn[i] = gv[i];
        if (e < a.rot) {
          const int j = e < rh ? e : e - rh;
          const float2 cs = a.rope[(size_t)tok * rh + j];
          dn[i] = e < rh ? gv[i] * cs.x + xs[wave][e + rh] * cs.y
                         : gv[i] * cs.x - xs[wave][e - rh] * cs.y;
        }
      }
      if (a.qk_norm) {
        const float* y = a.y + (size_t)m * n_qkv + (size_t)head * d;
        const bf16* w = kind == 0 ? a.q_norm_w : a.k_norm_w;
        float yv[4], wd[4], ss = 0.f, c = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = lane + 64 * i;
          yv[i] = e < d ? y[e] : 0.f;
          wd[i] = e < d ? (float)w[e] * dn[i] : 0.f;
          ss += yv[i] * yv[i];
          c += wd[i] * yv[i];
        }
        ss = wave_sum(ss);
        c = wave_sum(c);
        const float r = 1.0f / sqrtf(ss / (float)d + a.eps);
        const float k = r * r * c / (float)d;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = lane + 64 * i;
          if (e >= d) continue;
          dst[e] = (bf16)(r * (wd[i] - yv[i] * k));
          gw[kind][i] += dn[i] * yv[i] * r;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = lane + 64 * i;
          if (e < d) dst[e] = (bf16)dn[i];
        }
      }
    }
  }
  if (!a.qk_norm) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    if (e < d) {
      red[wave][0][e] = gw[0][i];
      red[wave][1][e] = gw[1][i];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 2 * d; idx += 256) {
    const int kk = idx / d, e = idx - kk * d;
    const float s = red[0][kk][e] + red[1][kk][e] + red[2][kk][e] + red[3][kk][e];
    a.dgamma_part[((size_t)blockIdx.x * 2 + kk) * d + e] = s;
  }
}

// Block kk (0 = q, 1 = k) sums feature j of every block's partial.
__global__ __launch_bounds__(256) void dgamma_reduce_kernel(const float* __restrict__ part,
                                                            int blocks, int d, float* dq_w,
                                                            float* dk_w) {
  const int kk = blockIdx.x;
  float* out = kk == 0 ? dq_w : dk_w;
  for (int j = threadIdx.x; j < d; j += 256) {
    float s = 0.f;
    for (int i = 0; i < blocks; ++i) s += part[((size_t)i * 2 + kk) * d + j];
    out[j] = s;
  }
}

// 64 x 64 tiles through LDS: 16-byte loads along the input rows, 16-byte
// stores along the output rows.  Output rows are written 8 input rows at a
// time; Rc is a multiple of 8, so such a group never straddles two chunks.
// Rows R .. S Rc - 1 (the last chunk's tail) are written as zeros.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16* __restrict__ in, int R,
                                                             int C, int Rc, int rows_out,
                                                             bf16* __restrict__ out) {
  __shared__ unsigned short tile[64][64 + 8];
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

hipError_t launch_normrope_bwd(const NormRopeBwdArgs& a, hipStream_t stream) {
  const int T = a.B * a.L;
  if (T == 0) return hipSuccess;
  const int blocks = (T + kNormRopeBwdTokens - 1) / kNormRopeBwdTokens;
  normrope_bwd_kernel<<<blocks, 256, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_dgamma_reduce(const float* part, int blocks, int d, float* dq_w, float* dk_w,
                                hipStream_t stream) {
  dgamma_reduce_kernel<<<2, 256, 0, stream>>>(part, blocks, d, dq_w, dk_w);
  return hipGetLastError();
}

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
