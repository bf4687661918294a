// Per-head QK-norm + RoPE of the fused projection output, forward and
// backward, for bf16 outputs and head_dim 64, 128 or 256 on gfx950 (tutorial
// "Multi-Head and Grouped-Query Attention (Full Layer)", section 4 steps 2-4;
// section 3: the norm has dim = head_dim and works within each head).
//
// Layout: a row is one (token, head of the fused projection) pair of D
// features; R = D / 4 lanes hold a row, 4 consecutive features per lane
// (16-byte fp32 loads), so a wave holds 64 / R rows.  Row reductions are
// shuffles within the lane group; the RoPE partner of feature e (e +- r/2)
// is 4 features away per r/8 lanes in the same group (r % 8 == 0), fetched
// by shuffle.  cos / sin come from a table [positions][r/2] built in double.
//
//   forward : out_e = rot(y_e * rs * w_e),   rs = (mean(y^2) + eps)^-1/2
//   backward: dn = rot^T(g);  dy_e = rs (w_e dn_e - y_e rs^2 mean(w dn y));
//             dw_e += dn_e y_e rs  (partial sums per block)
// where rot turns pair (e, e + r/2) by [[c, -s], [s, c]] and passes
// features r .. D-1 through.
#include "common.h"
#include "kernels.h"

namespace gqa {
namespace {

constexpr int kRowsNT = 256;
constexpr int kRowsIter = 8;  // most rows per lane group per block

template <int R>
GQA_DEV float group_sum(float v) {
#pragma unroll
  for (int o = R / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

GQA_DEV floatx4 ld_f4(const float* p) { return *reinterpret_cast<const floatx4*>(p); }

GQA_DEV floatx4 bf16x4_to_f4(u32x2 w) {
  return floatx4{lo_bf16(w.x), hi_bf16(w.x), lo_bf16(w.y), hi_bf16(w.y)};
}

GQA_DEV u32x2 f4_to_bf16x4(floatx4 v) {
  return u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// Partner values of this lane's 4 features (feature e -> e + rh for e < rh,
// e - rh for rh <= e < rot); lanes of other features get their own values.
template <int R>
GQA_DEV floatx4 partner4(floatx4 v, int sub, int rh4, int rot4) {
  const int base = threadIdx.x & 63 & ~(R - 1);
  int src = sub;
  if (sub < rh4) src = sub + rh4;
  else if (sub < rot4) src = sub - rh4;
  floatx4 p;
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __shfl(v[i], base + src, 64);
  return p;
}

// (cos, sin) of this lane's 4 features at table row `pos`
GQA_DEV void cossin4(const float2* rope, int rh, int pos, int e0, floatx4& c, floatx4& s) {
  const int j0 = e0 < rh ? e0 : e0 - rh;
  const floatx4 a = ld_f4(reinterpret_cast<const float*>(rope + (size_t)pos * rh + j0));
  const floatx4 b = ld_f4(reinterpret_cast<const float*>(rope + (size_t)pos * rh + j0 + 2));
  c = floatx4{a[0], a[2], b[0], b[2]};
  s = floatx4{a[1], a[3], b[1], b[3]};
}

// Rows are numbered below 2^31 (the launch checks), so the row -> (token,
// head) and token -> (sequence, position) splits are 32-bit divisions.
template <int D>
__global__ __launch_bounds__(kRowsNT) void normrope_fwd_rows_kernel(NormRopeRowsArgs a, int iters) {
  constexpr int R = D / 4, RPW = 64 / R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % R, e0 = 4 * sub;
  const int nh = a.Hq + 2 * a.Hkv;
  const unsigned rows = (unsigned)a.B * (unsigned)a.L * (unsigned)nh;
  const int rh = a.rot >> 1, rh4 = rh / 4, rot4 = a.rot / 4;
  const size_t n_qkv = (size_t)nh * D;
  const unsigned r0 = ((blockIdx.x * (unsigned)iters) * (kRowsNT / 64) + wave) * RPW + lane / R;
#pragma unroll 2
  for (int it = 0; it < iters; ++it) {
    const unsigned r = r0 + (unsigned)it * (kRowsNT / 64) * RPW;
    const bool live = r < rows;  // uniform within a lane group
    const unsigned m = live ? r / (unsigned)nh : 0u;
    const int head = live ? (int)(r - m * (unsigned)nh) : 0;
    const unsigned bu = m / (unsigned)a.L;
    const int b = (int)bu, tok = (int)(m - bu * (unsigned)a.L);
    int kind, h;
    if (head < a.Hq) { kind = 0; h = head; }
    else if (head < a.Hq + a.Hkv) { kind = 1; h = head - a.Hq; }
    else { kind = 2; h = head - a.Hq - a.Hkv; }
    floatx4 y;
    if (a.part) {
      // the split K's partial products, summed in split order; the loads
      // of four splits go out together
      const size_t o = (size_t)m * n_qkv + (size_t)head * D + e0;
      const size_t plane = (size_t)a.B * a.L * n_qkv;
      y = floatx4{0.f, 0.f, 0.f, 0.f};
      for (int z0 = 0; z0 < a.parts; z0 += 4) {
        floatx4 pz[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pz[i] = z0 + i < a.parts ? ld_f4(a.part + (size_t)(z0 + i) * plane + o) : floatx4{};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (z0 + i < a.parts) y = z0 + i == 0 ? pz[i] : y + pz[i];
      }
    } else {
      y = ld_f4(a.y + (size_t)m * n_qkv + (size_t)head * D + e0);
    }
    const int pos = (a.start_pos ? a.start_pos[b] : 0) + tok;
    if (kind != 2) {
      if (a.qk_norm) {
        const float ss = group_sum<R>(y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3]);
        const float rs = 1.0f / sqrtf(ss / (float)D + a.eps);
        const floatx4 w = bf16x4_to_f4(ld8((kind == 0 ? a.q_norm_w : a.k_norm_w) + e0));
        y = y * rs * w;
      }
      const floatx4 p = partner4<R>(y, sub, rh4, rot4);
      if (e0 < a.rot) {
        floatx4 c, s;
        cossin4(a.rope, rh, a.start_pos ? (int)m : tok, e0, c, s);
        y = e0 < rh ? y * c - p * s : y * c + p * s;
      }
    }
    if (!live) continue;
    bf16* dst;
    if (kind == 0) {
      dst = a.q + (((size_t)b * a.Hq + h) * a.L + tok) * D;
    } else {
      if (pos < 0 || pos >= a.cap) continue;
      dst = (kind == 1 ? a.k_cache : a.v_cache) + (((size_t)b * a.Hkv + h) * a.cap + pos) * D;
    }
    st8(dst + e0, f4_to_bf16x4(y));
  }
}

// Backward: a block takes one head of the fused projection (the grid's y)
// over kBwdTokens consecutive tokens (x).  Each row's gradient goes to dy
// [T, n_qkv] (token-major, for dx = dy W_qkv) and, through an LDS tile, to
// dyT (token chunks [s][n_qkv][Rc], for dW_qkv = dy^T x): the tile's
// kBwdTokens tokens lie in one chunk (Rc is a multiple of 64), so every
// feature's run of tokens is written in one piece.
constexpr int kBwdTokens = 64;

template <int D>
__global__ __launch_bounds__(kRowsNT) void normrope_bwd_rows_kernel(NormRopeBwdArgs a) {
  constexpr int R = D / 4, RPW = 64 / R;
  constexpr int PASSES = kBwdTokens / (kRowsNT / 64) / RPW;  // rows per lane group
  static_assert(PASSES * RPW * (kRowsNT / 64) == kBwdTokens, "a block covers kBwdTokens tokens");
  __shared__ floatx4 red[kRowsNT / 64][RPW][R];
  __shared__ u32x2 tile[kBwdTokens][R];  // bf16 dy of the block's tokens
  poison_lds(red, tile);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % R, e0 = 4 * sub, grp = lane / R;
  const int head = blockIdx.y;
  const int kind = head < a.Hq ? 0 : head < a.Hq + a.Hkv ? 1 : 2;  // block-uniform
  const int h = kind == 0 ? head : kind == 1 ? head - a.Hq : head - a.Hq - a.Hkv;
  const long long T = (long long)a.B * a.L;
  const long long m0 = (long long)blockIdx.x * kBwdTokens;
  const int rh = a.rot >> 1, rh4 = rh / 4, rot4 = a.rot / 4;
  const size_t n_qkv = (size_t)(a.Hq + 2 * a.Hkv) * D;
  floatx4 gw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int it = 0; it < PASSES; ++it) {
    const int t = (it * (kRowsNT / 64) + wave) * RPW + grp;  // token within the block
    const long long m = m0 + t;
    const bool live = m < T;  // uniform within a lane group
    const long long mm = live ? m : 0;
    const unsigned bu = (unsigned)mm / (unsigned)a.L;  // T < 2^31 (the launch checks)
    const int b = (int)bu, tok = (int)((unsigned)mm - bu * (unsigned)a.L);
    const bf16* g = kind == 0   ? a.dq + (((size_t)b * a.Hq + h) * a.L + tok) * D
                    : kind == 1 ? a.dk + (((size_t)b * a.Hkv + h) * a.L + tok) * D
                                : a.dv + (((size_t)b * a.Hkv + h) * a.L + tok) * D;
    floatx4 v = bf16x4_to_f4(ld8(g + e0));
    if (kind != 2) {
      // RoPE backward: the transpose of the rotation
      const floatx4 p = partner4<R>(v, sub, rh4, rot4);
      if (e0 < a.rot) {
        floatx4 c, s;
        cossin4(a.rope, rh, tok, e0, c, s);
        v = e0 < rh ? v * c + p * s : v * c - p * s;
      }
      if (a.qk_norm) {
        const floatx4 y = ld_f4(a.y + (size_t)mm * n_qkv + (size_t)head * D + e0);
        const floatx4 w = bf16x4_to_f4(ld8((kind == 0 ? a.q_norm_w : a.k_norm_w) + e0));
        const floatx4 wd = w * v;
        const float ss = group_sum<R>(y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3]);
        const float c = group_sum<R>(wd[0] * y[0] + wd[1] * y[1] + wd[2] * y[2] + wd[3] * y[3]);
        const float rs = 1.0f / sqrtf(ss / (float)D + a.eps);
        const float k = rs * rs * c / (float)D;
        if (live) gw += v * y * rs;
        v = rs * (wd - y * k);
      }
    }
    const u32x2 packed = f4_to_bf16x4(v);
    tile[t][sub] = live ? packed : u32x2{0u, 0u};  // tokens past T: zeros in dyT's padding
    if (live) st8(a.dy + (size_t)m * n_qkv + (size_t)head * D + e0, packed);
  }
  // the transposed copy: feature f's kBwdTokens tokens, 16 bytes per thread
  const int s_chunk = (int)(m0 / a.Rc);
  const long long t0 = m0 - (long long)s_chunk * a.Rc;
  __syncthreads();
  for (int idx = threadIdx.x; idx < D * (kBwdTokens / 8); idx += kRowsNT) {
    const int f = idx / (kBwdTokens / 8), tg = (idx - f * (kBwdTokens / 8)) * 8;
    const unsigned short* col = reinterpret_cast<const unsigned short*>(&tile[0][0]) + f;
    constexpr int RS = R * 4;  // ushorts per tile row
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (unsigned)col[(tg + 2 * i) * RS] | ((unsigned)col[(tg + 2 * i + 1) * RS] << 16);
    st16(a.dyT + ((size_t)s_chunk * n_qkv + (size_t)head * D + f) * a.Rc + t0 + tg, w);
  }
  if (!a.qk_norm) return;
  // block partial sums of this head kind's weight gradient (the other kind: 0)
  red[wave][grp][sub] = gw;
  __syncthreads();
  for (int idx = threadIdx.x; idx < 2 * R; idx += kRowsNT) {
    const int kk = idx / R, sb = idx - kk * R;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (kk == kind) {
#pragma unroll
      for (int w = 0; w < kRowsNT / 64; ++w)
#pragma unroll
        for (int gq = 0; gq < RPW; ++gq) acc += red[w][gq][sb];
    }
    const size_t blk = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
    *reinterpret_cast<floatx4*>(a.dgamma_part + (blk * 2 + kk) * D + 4 * sb) = acc;
  }
}

// Sum of the per-block partials [blocks][2][d] in two fixed-order stages:
// stage 1 block j sums partial rows j, j + S1, j + 2 S1, ... (one thread per
// column, eight loads in flight); stage 2 (one block of 1024 threads) gives
// each column 1024 / (2 d) threads, thread u summing stage rows u, u + TPC,
// ... (sixteen loads in flight), and adds their sums in u order.  Both
// orders are fixed, so the result does not depend on the schedule.
constexpr int kReduceS1 = 256;
constexpr int kReduceS2NT = 1024;

__global__ __launch_bounds__(256) void dgamma_stage1_kernel(const float* __restrict__ part,
                                                            int blocks, int d,
                                                            float* __restrict__ stage) {
  const int j = blockIdx.x;
  for (int col = threadIdx.x; col < 2 * d; col += 256) {
    float s = 0.f;
#pragma unroll 8
    for (int i = j; i < blocks; i += kReduceS1) s += part[(size_t)i * 2 * d + col];
    stage[(size_t)j * 2 * d + col] = s;
  }
}

__global__ __launch_bounds__(kReduceS2NT) void dgamma_stage2_kernel(const float* __restrict__ stage,
                                                                   int d, float* dq_w,
                                                                   float* dk_w) {
  __shared__ float red[kReduceS2NT];
  poison_lds(red);
  const int cols = 2 * d;  // 128, 256 or 512: divides kReduceS2NT
  const int tpc = kReduceS2NT / cols;
  const int col = threadIdx.x % cols, u = threadIdx.x / cols;
  float s = 0.f;
#pragma unroll 16
  for (int j = u; j < kReduceS1; j += tpc) s += stage[(size_t)j * cols + col];
  red[threadIdx.x] = s;
  __syncthreads();
  if (u != 0) return;
  float t = 0.f;
  for (int v = 0; v < tpc; ++v) t += red[v * cols + col];
  if (col < d) dq_w[col] = t;
  else dk_w[col - d] = t;
}

// Rows per lane group and block: kRowsIter for large row counts, fewer
// when that would leave fewer than about 1024 blocks (a decode step has a
// few thousand rows, which then spread over many CUs instead of queueing in
// a few lane groups).
template <int D>
int rows_iters(long long rows) {
  const long long per_iter = (long long)(kRowsNT / 64) * (64 / (D / 4));
  long long it = rows / (per_iter * 1024);
  if (it > kRowsIter) it = kRowsIter;
  if (it < 1) it = 1;
  return (int)it;
}

template <int D>
hipError_t launch_rows(const NormRopeRowsArgs& a, long long rows, hipStream_t stream) {
  const int iters = rows_iters<D>(rows);
  const long long per = (long long)iters * (kRowsNT / 64) * (64 / (D / 4));
  const long long blocks = (rows + per - 1) / per;
  normrope_fwd_rows_kernel<D><<<(unsigned)blocks, kRowsNT, 0, stream>>>(a, iters);
  return hipGetLastError();
}

}  // namespace

bool normrope_rows_ok(int d, int rot) {
  return (d == 64 || d == 128 || d == 256) && rot % 8 == 0 && rot > 0;
}

// The grid covers every token chunk in full (tiles past T write zeros into
// dyT's padding, which the weight-gradient GEMM reads).
long long normrope_bwd_tiles(long long T, int Rc) {
  return (T + Rc - 1) / Rc * Rc / kBwdTokens;
}

int normrope_bwd_blocks(long long T, int Rc, int nh) {
  return (int)(normrope_bwd_tiles(T, Rc) * nh);
}

hipError_t launch_normrope_fwd_rows(const NormRopeRowsArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.L * (a.Hq + 2 * a.Hkv);
  if (rows == 0) return hipSuccess;
  if (!normrope_rows_ok(a.d, a.rot) || rows > 0x7fffffffLL) return hipErrorInvalidValue;
  switch (a.d) {
    case 64: return launch_rows<64>(a, rows, stream);
    case 128: return launch_rows<128>(a, rows, stream);
    default: return launch_rows<256>(a, rows, stream);
  }
}

hipError_t launch_normrope_bwd(const NormRopeBwdArgs& a, hipStream_t stream) {
  const long long T = (long long)a.B * a.L;
  if (T == 0) return hipSuccess;
  if (!normrope_rows_ok(a.d, a.rot) || a.Rc % kBwdTokens != 0 || T > 0x7fffffffLL)
    return hipErrorInvalidValue;
  const long long gx = normrope_bwd_tiles(T, a.Rc);
  if (gx > 0x7fffffffLL || a.Hq + 2 * a.Hkv > 65535) return hipErrorInvalidValue;
  dim3 grid((unsigned)gx, a.Hq + 2 * a.Hkv);
  switch (a.d) {
    case 64: normrope_bwd_rows_kernel<64><<<grid, kRowsNT, 0, stream>>>(a); break;
    case 128: normrope_bwd_rows_kernel<128><<<grid, kRowsNT, 0, stream>>>(a); break;
    default: normrope_bwd_rows_kernel<256><<<grid, kRowsNT, 0, stream>>>(a); break;
  }
  return hipGetLastError();
}

size_t dgamma_stage_floats(int d) { return (size_t)kReduceS1 * 2 * d; }

hipError_t launch_dgamma_reduce(const float* part, int blocks, int d, float* stage, float* dq_w,
                                float* dk_w, hipStream_t stream) {
  dgamma_stage1_kernel<<<kReduceS1, 256, 0, stream>>>(part, blocks, d, stage);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (kReduceS2NT % (2 * d) != 0) return hipErrorInvalidValue;
  dgamma_stage2_kernel<<<1, kReduceS2NT, 0, stream>>>(stage, d, dq_w, dk_w);
  return hipGetLastError();
}

}  // namespace gqa
