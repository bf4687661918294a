// bf16 MFMA GEMMs of the layer on gfx950:
//   * the fused QKV projection with the QK-norm + RoPE epilogue and the
//     head-major scatter into q and the K/V cache (GPT-NeoX issue "Fused QKV
//     projection"; tutorial "Multi-Head and Grouped-Query Attention (Full
//     Layer)", section 4 steps 1-4 and section 3 for the per-head norm);
//   * the output projection (GPT-NeoX issue "Output projection"; tutorial
//     section 4 step 7).
//
// Both compute a tile of C^T: rows are output features n (rows of the weight
// W [N, K]), columns are tokens m (rows of the activation X [M, K]); both
// operands are K-contiguous.  With this orientation one lane of the MFMA
// accumulator holds, for one token, 64 of the 128 features of a head and the
// other 64 sit in lane l^32: the per-head RMS needs one cross-lane exchange,
// and the RoPE partners (feature i and i + 64) sit in the same lane.
#include "common.h"
#include "kernels.h"

namespace gqa {

namespace {

constexpr int kBK = 64;          // K elements per LDS stage (8 chunks of 16 B)
constexpr int kThreads = 256;    // 4 waves, 2 x 2 over the C^T tile

// LDS row of one tile: kBK bf16 = 128 B = 8 chunks of 16 B.  Chunk c of row r
// lives at slot c ^ (r & 7): eight consecutive rows read at one chunk index
// hit eight distinct 16-byte bank groups.
__device__ __forceinline__ int swz8(int row, int chunk) { return (row << 3) + (chunk ^ (row & 7)); }

template <int ROWS>
struct TileRegs {
  static constexpr int kPer = ROWS * 8 / kThreads;  // 16-byte chunks per thread
  u32x4 v[kPer];
};

template <int ROWS>
__device__ __forceinline__ void load_tile(TileRegs<ROWS>& r, const bf16* __restrict__ base,
                                          int row0, int nrows, int k0, int K, int tid) {
#pragma unroll
  for (int i = 0; i < TileRegs<ROWS>::kPer; ++i) {
    const int idx = tid + i * kThreads;
    const int row = idx >> 3;
    const int ch = idx & 7;
    const int gr = row0 + row;
    const int gk = k0 + ch * 8;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (gr < nrows && gk < K) val = ld16(base + (size_t)gr * K + gk);
    r.v[i] = val;
  }
}

template <int ROWS>
__device__ __forceinline__ void store_tile(const TileRegs<ROWS>& r, u32x4* lds, int tid) {
#pragma unroll
  for (int i = 0; i < TileRegs<ROWS>::kPer; ++i) {
    const int idx = tid + i * kThreads;
    lds[swz8(idx >> 3, idx & 7)] = r.v[i];
  }
}

template <int BN, int BM, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int WN = BN / 2, WM = BM / 2;
  constexpr int FB = WN / 32, TB = WM / 32;
  static_assert(EPI != kEpiQKV || WN == 128, "QKV epilogue needs one head (128 features) per wave");
  __shared__ u32x4 lds[2][(BN + BM) * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int l32 = lane & 31, hh = lane >> 5;

  // Tiles along N are the fast grid dimension so that the activation tile
  // (tokens) of neighbouring workgroups is shared through L2.
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int N = a.N, M = a.M, K = a.K;

  floatx16 acc[FB][TB];
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[f][t][r] = 0.f;

  TileRegs<BN> ra;
  TileRegs<BM> rb;
  const int nk = (K + kBK - 1) / kBK;
  // W may be narrower than X along K (w_kmod): X = [hi | lo] reads W twice
  const int Kw = a.w_kmod > 0 ? a.w_kmod : K;
  load_tile<BN>(ra, a.W, n0, N, 0, Kw, tid);
  load_tile<BM>(rb, a.X, m0, M, 0, K, tid);
  store_tile<BN>(ra, &lds[0][0], tid);
  store_tile<BM>(rb, &lds[0][BN * 8], tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      load_tile<BN>(ra, a.W, n0, N, ((kt + 1) * kBK) % Kw, Kw, tid);
      load_tile<BM>(rb, a.X, m0, M, (kt + 1) * kBK, K, tid);
    }
    const u32x4* sa = &lds[buf][0];
    const u32x4* sb = &lds[buf][BN * 8];
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int ch = 2 * s + hh;
      u32x4 fa[FB], fb[TB];
#pragma unroll
      for (int f = 0; f < FB; ++f) fa[f] = sa[swz8(wn * WN + 32 * f + l32, ch)];
#pragma unroll
      for (int t = 0; t < TB; ++t) fb[t] = sb[swz8(wm * WM + 32 * t + l32, ch)];
#pragma unroll
      for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int t = 0; t < TB; ++t) acc[f][t] = mfma32x32x16(fa[f], fb[t], acc[f][t]);
    }
    if (kt + 1 < nk) {
      store_tile<BN>(ra, &lds[buf ^ 1][0], tid);
      store_tile<BM>(rb, &lds[buf ^ 1][BN * 8], tid);
    }
    __syncthreads();
  }

  const int nw = n0 + wn * WN;  // first feature of this wave
  if (EPI == kEpiPlain) {
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const int m = m0 + wm * WM + 32 * t + l32;
      if (m >= M) continue;
#pragma unroll
      for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = nw + 32 * f + 8 * j + 4 * hh;
          if (n >= N) continue;
          if (a.out_f32) {
            floatx4 w = {acc[f][t][4 * j + 0], acc[f][t][4 * j + 1], acc[f][t][4 * j + 2],
                         acc[f][t][4 * j + 3]};
            *reinterpret_cast<floatx4*>(static_cast<float*>(a.out) + (size_t)m * N + n) = w;
          } else {
            u32x2 w;
            w.x = pack_bf16x2(acc[f][t][4 * j + 0], acc[f][t][4 * j + 1]);
            w.y = pack_bf16x2(acc[f][t][4 * j + 2], acc[f][t][4 * j + 3]);
            st8(static_cast<bf16*>(a.out) + (size_t)m * N + n, w);
          }
        }
    }
    return;
  }

  // ---- QKV epilogue: one head of 128 features per wave ----
  if (nw >= N) return;  // wave-uniform
  const int head = nw >> 7;
  const int Hq = a.Hq, Hkv = a.Hkv;
  int kind;       // 0 = q, 1 = k, 2 = v
  int h;
  if (head < Hq) { kind = 0; h = head; }
  else if (head < Hq + Hkv) { kind = 1; h = head - Hq; }
  else { kind = 2; h = head - Hq - Hkv; }

  const bool do_norm = (kind != 2) && a.qk_norm;
  const bf16* wsrc = kind == 0 ? a.q_norm_w : a.k_norm_w;

#pragma unroll
  for (int t = 0; t < TB; ++t) {
    const int m = m0 + wm * WM + 32 * t + l32;
    const bool valid = m < M;
    const int mm = valid ? m : 0;
    const int b = mm / a.L;
    const int tok = mm - b * a.L;
    float v[4][16];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) v[f][r] = acc[f][t][r];

    if (do_norm) {
      float ss = 0.f;
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) ss += v[f][r] * v[f][r];
      ss += wave_xor32(ss);
      const float inv = 1.0f / __builtin_sqrtf(ss * (1.0f / 128.0f) + a.eps);
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          v[f][r] = v[f][r] * inv * (float)wsrc[32 * f + 8 * (r >> 2) + 4 * hh + (r & 3)];
    }
    const int pos = (a.start_pos ? a.start_pos[b] : 0) + tok;
    if (kind != 2) {
      // rotate-half RoPE: feature i (< 64) pairs with i + 64, same lane, f+2
      const float2* cs = a.rope + (size_t)(a.start_pos ? mm : tok) * 64;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = 32 * f + 8 * (r >> 2) + 4 * hh + (r & 3);
          const float2 c = valid ? cs[i] : make_float2(1.f, 0.f);
          const float x1 = v[f][r], x2 = v[f + 2][r];
          v[f][r] = x1 * c.x - x2 * c.y;
          v[f + 2][r] = x2 * c.x + x1 * c.y;
        }
    }
    if (!valid) continue;
    bf16* dst;
    if (kind == 0) {
      dst = a.q + (((size_t)b * Hq + h) * a.L + tok) * 128;
    } else {
      if (pos < 0 || pos >= a.cap) continue;
      bf16* cache = kind == 1 ? a.k_cache : a.v_cache;
      dst = cache + (((size_t)b * Hkv + h) * a.cap + pos) * 128;
    }
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w;
        w.x = pack_bf16x2(v[f][4 * j + 0], v[f][4 * j + 1]);
        w.y = pack_bf16x2(v[f][4 * j + 2], v[f][4 * j + 3]);
        st8(dst + 32 * f + 8 * j + 4 * hh, w);
      }
  }
}

// cos/sin of position * theta^(-2i/d) for i < d/2, angles in double.
__global__ void rope_table_kernel(float2* __restrict__ table, const int* __restrict__ start_pos,
                                  int rows, int L, int half, double theta) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * half) return;
  const int row = idx / half;
  const int i = idx - row * half;
  long pos;
  if (start_pos) {
    const int b = row / L;
    pos = (long)start_pos[b] + (row - b * L);
  } else {
    pos = row;
  }
  const double inv = pow(theta, -2.0 * (double)i / (double)(2 * half));
  const double ang = (double)pos * inv;
  double s, c;
  sincos(ang, &s, &c);
  table[idx] = make_float2((float)c, (float)s);
}

}  // namespace

hipError_t launch_rope_table(float2* table, const int* start_pos, int rows, int L, int half,
                             double theta, hipStream_t stream) {
  const int n = rows * half;
  if (n == 0) return hipSuccess;
  rope_table_kernel<<<(n + 255) / 256, 256, 0, stream>>>(table, start_pos, rows, L, half, theta);
  return hipGetLastError();
}

hipError_t launch_gemm_qkv_bf16(const GemmArgs& args, hipStream_t stream) {
  constexpr int BN = 256, BM = 128;
  dim3 grid((args.N + BN - 1) / BN, (args.M + BM - 1) / BM);
  gemm_bf16_kernel<BN, BM, kEpiQKV><<<grid, kThreads, 0, stream>>>(args);
  return hipGetLastError();
}

hipError_t launch_gemm_plain_bf16(const GemmArgs& args, hipStream_t stream) {
  constexpr int BN = 256, BM = 128;
  dim3 grid((args.N + BN - 1) / BN, (args.M + BM - 1) / BM);
  gemm_bf16_kernel<BN, BM, kEpiPlain><<<grid, kThreads, 0, stream>>>(args);
  return hipGetLastError();
}

}  // namespace gqa
