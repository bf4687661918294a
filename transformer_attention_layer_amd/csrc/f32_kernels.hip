// fp32 path of the layer (any even head_dim from 2 to 256), and the pieces
// the bf16 path uses for head sizes other than 128.  Plain VALU kernels: a
// tiled GEMM, a per-(token, head) QK-norm + RoPE + scatter, and a
// one-wave-per-query attention with an online softmax.  Same steps as the
// bf16 path (tutorial "Multi-Head and Grouped-Query Attention (Full Layer)",
// section 4 steps 1-7), in float throughout.
#include "common.h"
#include "kernels.h"

namespace gqa {
namespace {

constexpr int kT = 64;   // output tile (tokens and features)
constexpr int kKT = 16;  // K step

// y[m, n] = sum_k x[m, k] w[n, k]; 256 threads, 4 x 4 outputs each.
__global__ __launch_bounds__(256) void gemm_f32_kernel(F32Args a) {
  __shared__ float sx[kKT][kT + 1];
  __shared__ float sw[kKT][kT + 1];
  poison_lds(sx, sw);
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * kT, n0 = blockIdx.x * kT;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < a.K; k0 += kKT) {
    for (int i = tid; i < kT * kKT; i += 256) {
      const int r = i / kKT, c = i % kKT;
      const int gm = m0 + r, gn = n0 + r, gk = k0 + c;
      sx[c][r] = (gm < a.M && gk < a.K) ? a.x[(size_t)gm * a.K + gk] : 0.f;
      sw[c][r] = (gn < a.N && gk < a.K) ? a.w[(size_t)gn * a.K + gk] : 0.f;
    }
    __syncthreads();
    for (int c = 0; c < kKT; ++c) {
      float xv[4], wv[4];
      for (int i = 0; i < 4; ++i) xv[i] = sx[c][ty + 16 * i];
      for (int j = 0; j < 4; ++j) wv[j] = sw[c][tx + 16 * j];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty + 16 * i;
    if (m >= a.M) continue;
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n < a.N) a.y[(size_t)m * a.N + n] = acc[i][j];
    }
  }
}

// One workgroup per (token, head of the fused projection); thread j < d/2
// holds features j and j + d/2.  The normalised head goes through shared
// memory so that any rotary width r works: output feature e < r/2 pairs with
// e + r/2; features r .. d-1 pass through.  T is the element type of the
// norm weights and of q / the caches (float, or bf16 for the bf16 path).
template <typename T>
__global__ __launch_bounds__(128) void normrope_kernel(NormRopeArgs a) {
  __shared__ float red[128];
  __shared__ float xs[256];
  poison_lds(red, xs);
  const int m = blockIdx.x;       // token
  const int head = blockIdx.y;    // 0 .. Hq + 2 Hkv - 1
  const int j = threadIdx.x;
  const int d = a.d, half = d >> 1, rh = a.rot >> 1;
  const int b = m / a.L, tok = m - b * a.L;
  const int n_qkv = (a.Hq + 2 * a.Hkv) * d;
  const float* y = a.y + (size_t)m * n_qkv + (size_t)head * d;
  int kind, h;
  if (head < a.Hq) { kind = 0; h = head; }
  else if (head < a.Hq + a.Hkv) { kind = 1; h = head - a.Hq; }
  else { kind = 2; h = head - a.Hq - a.Hkv; }
  const bool act = j < half;
  float x1 = act ? y[j] : 0.f;
  float x2 = act ? y[j + half] : 0.f;
  const long pos = (long)(a.start_pos ? a.start_pos[b] : 0) + tok;
  if (kind != 2) {
    if (a.qk_norm) {
      red[j] = x1 * x1 + x2 * x2;
      __syncthreads();
      for (int s = 64; s > 0; s >>= 1) {
        if (j < s) red[j] += red[j + s];
        __syncthreads();
      }
      const float inv = 1.0f / sqrtf(red[0] / (float)d + a.eps);
      const T* w = static_cast<const T*>(kind == 0 ? a.q_norm_w : a.k_norm_w);
      if (act) {
        x1 = x1 * inv * (float)w[j];
        x2 = x2 * inv * (float)w[j + half];
      }
    }
    if (act) {
      xs[j] = x1;
      xs[j + half] = x2;
    }
    __syncthreads();
    // rotated value of feature e (the pair's angle uses its lower index)
    auto rot_of = [&](int e) {
      if (e >= a.rot) return xs[e];
      const int i = e < rh ? e : e - rh;
      const double ang = (double)pos * pow(a.theta, -2.0 * (double)i / (double)a.rot);
      double sd, cd;
      sincos(ang, &sd, &cd);
      const float c = (float)cd, s = (float)sd;
      return e < rh ? xs[e] * c - xs[e + rh] * s : xs[e] * c + xs[e - rh] * s;
    };
    if (act) {
      x1 = rot_of(j);
      x2 = rot_of(j + half);
    }
  }
  if (!act) return;
  if (kind != 0 && a.kv_fp8) {
    // E4M3 code of x / scale: the conversion rounds to nearest even but
    // turns magnitudes past the largest finite value into NaN, so they are
    // clamped to 448 first
    if (pos < 0 || pos >= a.cap) return;
    const float inv = kind == 1 ? a.inv_k_scale : a.inv_v_scale;
    const float y1 = fminf(fmaxf(x1 * inv, -448.0f), 448.0f);
    const float y2 = fminf(fmaxf(x2 * inv, -448.0f), 448.0f);
    const int codes = __builtin_amdgcn_cvt_pk_fp8_f32(y1, y2, 0, false);
    unsigned char* dst = static_cast<unsigned char*>(kind == 1 ? a.k_cache : a.v_cache) +
                         (((size_t)b * a.Hkv + h) * a.cap + pos) * d;
    dst[j] = (unsigned char)(codes & 0xff);
    dst[j + half] = (unsigned char)((codes >> 8) & 0xff);
    return;
  }
  T* dst;
  if (kind == 0) {
    dst = static_cast<T*>(a.q) + (((size_t)b * a.Hq + h) * a.L + tok) * d;
  } else {
    if (pos < 0 || pos >= a.cap) return;
    dst = static_cast<T*>(kind == 1 ? a.k_cache : a.v_cache) +
          (((size_t)b * a.Hkv + h) * a.cap + pos) * d;
  }
  dst[j] = (T)x1;
  dst[j + half] = (T)x2;
}

// One wave per (query, head, sequence); lane e owns features e, e+64, ...
// T is the element type of q, the caches and o (float, or bf16 for head
// sizes the bf16 matrix-core kernels do not cover); with bf16 and o_split
// the output is the bf16 value followed, Hq * d further on, by its rounding
// residual; with bf16 and o_f16 it is the fp16 value.
template <typename T>
__global__ __launch_bounds__(64) void attn_vec_kernel(F32AttnArgs a) {
  const int i = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int d = a.d;
  const int G = a.Hq / a.Hkv;
  const int kvh = hq / G;
  int kvl = (a.kv_base ? a.kv_base[b] : 0) + a.kv_add;
  kvl = kvl < 0 ? 0 : (kvl > a.cap ? a.cap : kvl);
  const int qpos = kvl - a.Lq + i;
  const int kend = a.causal ? min(kvl, qpos + 1) : kvl;
  const T* q = static_cast<const T*>(a.q) + (((size_t)b * a.Hq + hq) * a.Lq + i) * d;
  const T* kb = static_cast<const T*>(a.k) + ((size_t)b * a.Hkv + kvh) * a.cap * d;
  const T* vb = static_cast<const T*>(a.v) + ((size_t)b * a.Hkv + kvh) * a.cap * d;
  float qv[4], ov[4];
  for (int u = 0; u < 4; ++u) {
    const int e = lane + 64 * u;
    qv[u] = e < d ? (float)q[e] : 0.f;
    ov[u] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j < kend; ++j) {
    const T* kr = kb + (size_t)j * d;
    float part = 0.f;
    for (int u = 0; u < 4; ++u) {
      const int e = lane + 64 * u;
      if (e < d) part = fmaf(qv[u], (float)kr[e], part);
    }
    for (int s = 32; s > 0; s >>= 1) part += __shfl_xor(part, s, 64);
    const float x = part * a.scale;
    const float m_new = fmaxf(m, x);
    const float alpha = expf(m - m_new);
    const float p = expf(x - m_new);
    l = l * alpha + p;
    const T* vr = vb + (size_t)j * d;
    for (int u = 0; u < 4; ++u) {
      const int e = lane + 64 * u;
      ov[u] = ov[u] * alpha + (e < d ? p * (float)vr[e] : 0.f);
    }
    m = m_new;
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  const size_t width = (size_t)a.Hq * d;
  T* o = static_cast<T*>(a.o) + ((size_t)b * a.Lq + i) * width * (a.o_split ? 2 : 1) +
         (size_t)hq * d;
  for (int u = 0; u < 4; ++u) {
    const int e = lane + 64 * u;
    if (e >= d) continue;
    const float val = ov[u] * inv;
    if constexpr (sizeof(T) == 2) {
      if (a.o_f16) {  // fp16 bits in the 16-bit slot
        reinterpret_cast<_Float16*>(o)[e] = (_Float16)val;
        continue;
      }
    }
    const T hi = (T)val;
    o[e] = hi;
    if (a.o_split) o[width + e] = (T)(val - (float)hi);
  }
}

}  // namespace

hipError_t launch_gemm_f32(const F32Args& a, hipStream_t stream) {
  dim3 grid((a.N + kT - 1) / kT, (a.M + kT - 1) / kT);
  gemm_f32_kernel<<<grid, 256, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_normrope(const NormRopeArgs& a, hipStream_t stream) {
  dim3 grid(a.B * a.L, a.Hq + 2 * a.Hkv);
  if (a.bf16)
    normrope_kernel<bf16><<<grid, 128, 0, stream>>>(a);
  else
    normrope_kernel<float><<<grid, 128, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_attn_vec(const F32AttnArgs& a, hipStream_t stream) {
  dim3 grid(a.Lq, a.Hq, a.B);
  if (a.bf16)
    attn_vec_kernel<bf16><<<grid, 64, 0, stream>>>(a);
  else
    attn_vec_kernel<float><<<grid, 64, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace gqa
