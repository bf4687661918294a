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
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;
constexpr int kThreads = 256;    // 4 waves, 2 x 2 over the C^T tile

// LDS row of one tile: kBK bf16 = 128 B = 8 chunks of 16 B.  Chunk c of row r
// lives at slot c ^ (r & 7): eight consecutive rows read at one chunk index
// hit eight distinct 16-byte bank groups.
__device__ __forceinline__ int swz8(int row, int chunk) { return (row << 3) + (chunk ^ (row & 7)); }

// Raw buffer descriptor over rows [row0, nrows) of a row-major bf16 matrix
// with `ld` elements per row.  Loads past the end of the range return zero
// (hardware bounds check), which zero-fills ragged row and K tails.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const bf16* base, int row0, int nrows,
                                                            int ld) {
  long long bytes = (long long)(nrows - row0) * ld * 2;
  if (bytes < 0) bytes = 0;
  if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
  return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)row0 * ld), 0, (int)bytes,
                                           0x00020000);
}

// Stage one kBK-wide tile of ROWS rows straight from global memory into LDS
// (buffer_load ... lds, no register staging).  One instruction fills 64
// consecutive 16-byte LDS slots = 8 rows; lane i writes slot i, so it loads
// the global chunk that the XOR swizzle places there: chunk (i & 7) ^ (i >> 3)
// of row i >> 3.  Chunks at or past column `kcols` read as zero.
template <int ROWS>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rsrc, u32x4* lds, int ld, int k0,
                                         int kcols, int wave, int lane) {
  constexpr int kInstr = ROWS / 8 / 4;  // per wave
  const int r_in = lane >> 3;
  const int c = (lane & 7) ^ r_in;
  const int k = k0 + c * 8;
#pragma unroll
  for (int j = 0; j < kInstr; ++j) {
    const int r0 = (wave * kInstr + j) * 8;
    const unsigned voff = k < kcols ? (unsigned)(((r0 + r_in) * ld + k) * 2) : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(lds + r0 * 8), 16, voff, 0, 0, 0);
  }
}

// Workgroup -> output tile.  The grid is 1-D and padded to a multiple of the
// 8 XCDs; workgroup i runs on XCD i % 8, so each XCD is handed one
// contiguous run of the tile order below.  That order walks groups of
// kGroupM token tiles and, inside a group, the feature tiles token tile by
// token tile, so the tiles an XCD works on at one time share activations
// and weights through its L2.
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

__device__ __forceinline__ bool tile_of(const GemmArgs& a, int BN, int BM, int& tn, int& tm) {
  const int ntn = (a.N + BN - 1) / BN;
  const int ntm = (a.M + BM - 1) / BM;
  const int total = ntn * ntm;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int id = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
  if (id >= total) return false;
  const int group = id / (kGroupM * ntn);
  const int first_m = group * kGroupM;
  const int gm = min(ntm - first_m, kGroupM);
  const int in = id - group * kGroupM * ntn;
  tm = first_m + in % gm;
  tn = in / gm;
  return true;
}

__host__ __device__ constexpr int gemm_grid(int N, int M, int BN, int BM) {
  return ((((N + BN - 1) / BN) * ((M + BM - 1) / BM) + kXcds - 1) / kXcds) * kXcds;
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

  const int N = a.N, M = a.M, K = a.K;
  int tn, tm;
  if (!tile_of(a, BN, BM, tn, tm)) return;  // padding workgroup
  const int n0 = tn * BN;
  const int m0 = tm * BM;

  floatx16 acc[FB][TB];
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[f][t][r] = 0.f;

  const int nk = (K + kBK - 1) / kBK;
  // W may be narrower than X along K (w_kmod): X = [hi | lo] reads W twice
  const int Kw = a.w_kmod > 0 ? a.w_kmod : K;
  const __amdgpu_buffer_rsrc_t rw = rows_rsrc(a.W, n0, N, Kw);
  const __amdgpu_buffer_rsrc_t rx = rows_rsrc(a.X, m0, M, K);
  dma_tile<BN>(rw, &lds[0][0], Kw, 0, Kw, wave, lane);
  dma_tile<BM>(rx, &lds[0][BN * 8], K, 0, K, wave, lane);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      // the other buffer was last read before the barrier that ended the
      // previous iteration
      dma_tile<BN>(rw, &lds[buf ^ 1][0], Kw, ((kt + 1) * kBK) % Kw, Kw, wave, lane);
      dma_tile<BM>(rx, &lds[buf ^ 1][BN * 8], K, (kt + 1) * kBK, K, wave, lane);
    }
    const u32x4* sa = &lds[buf][0];
    const u32x4* sb = &lds[buf][BN * 8];
    // fragments of k-substep s+1 are read from LDS while the MFMAs of
    // substep s run
    u32x4 fa[2][FB], fb[2][TB];
#pragma unroll
    for (int f = 0; f < FB; ++f) fa[0][f] = sa[swz8(wn * WN + 32 * f + l32, hh)];
#pragma unroll
    for (int t = 0; t < TB; ++t) fb[0][t] = sb[swz8(wm * WM + 32 * t + l32, hh)];
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int cur = s & 1;
      if (s + 1 < kBK / 16) {
        const int ch = 2 * (s + 1) + hh;
#pragma unroll
        for (int f = 0; f < FB; ++f) fa[cur ^ 1][f] = sa[swz8(wn * WN + 32 * f + l32, ch)];
#pragma unroll
        for (int t = 0; t < TB; ++t) fb[cur ^ 1][t] = sb[swz8(wm * WM + 32 * t + l32, ch)];
      }
      // Fence the scheduler: substep s+1's reads stay ahead of substep s's
      // MFMAs, so the wait before each substep only covers reads issued a
      // whole substep (16 MFMAs) earlier.
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int t = 0; t < TB; ++t) acc[f][t] = mfma32x32x16(fa[cur][f], fb[cur][t], acc[f][t]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();  // the next tile's loads are complete and visible
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
  // norm weights of this lane's features 32f + 8j + 4hh + (0..3), kept packed
  u32x2 wpk[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 z = {0x3f803f80u, 0x3f803f80u};  // bf16 1.0
      wpk[f][j] = do_norm ? ld8(wsrc + 32 * f + 8 * j + 4 * hh) : z;
    }

  // One token block (32 tokens) at a time; within it, a lane handles four
  // consecutive features i..i+3 of the first half together with their RoPE
  // partners i+64..i+67, so only a few values are live at once.
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    const int m = m0 + wm * WM + 32 * t + l32;
    const bool valid = m < M;
    const int mm = valid ? m : 0;
    const int b = mm / a.L;
    const int tok = mm - b * a.L;
    float inv = 1.0f;
    if (do_norm) {
      float ss = 0.f;
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) ss += acc[f][t][r] * acc[f][t][r];
      ss += wave_xor32(ss);
      inv = 1.0f / __builtin_sqrtf(ss * (1.0f / 128.0f) + a.eps);
    }
    if (!valid) continue;
    const int pos = (a.start_pos ? a.start_pos[b] : 0) + tok;
    bf16* dst;
    if (kind == 0) {
      dst = a.q + (((size_t)b * Hq + h) * a.L + tok) * 128;
    } else {
      if (pos < 0 || pos >= a.cap) continue;
      bf16* cache = kind == 1 ? a.k_cache : a.v_cache;
      dst = cache + (((size_t)b * Hkv + h) * a.cap + pos) * 128;
    }
    if (kind == 2) {
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 w;
          w.x = pack_bf16x2(acc[f][t][4 * j + 0], acc[f][t][4 * j + 1]);
          w.y = pack_bf16x2(acc[f][t][4 * j + 2], acc[f][t][4 * j + 3]);
          st8(dst + 32 * f + 8 * j + 4 * hh, w);
        }
      continue;
    }
    // rotate-half RoPE: feature i (< 64) pairs with i + 64 (block f + 2)
    const float2* cs = a.rope + (size_t)(a.start_pos ? mm : tok) * 64;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i0 = 32 * f + 8 * j + 4 * hh;
        // (cos, sin) of features i0 .. i0+3: two 16-byte loads
        const floatx4 c01 = *reinterpret_cast<const floatx4*>(cs + i0);
        const floatx4 c23 = *reinterpret_cast<const floatx4*>(cs + i0 + 2);
        const float cc[4] = {c01[0], c01[2], c23[0], c23[2]};
        const float sn[4] = {c01[1], c01[3], c23[1], c23[3]};
        const u32x2 w1 = wpk[f][j], w2 = wpk[f + 2][j];
        const float g1[4] = {lo_bf16(w1.x), hi_bf16(w1.x), lo_bf16(w1.y), hi_bf16(w1.y)};
        const float g2[4] = {lo_bf16(w2.x), hi_bf16(w2.x), lo_bf16(w2.y), hi_bf16(w2.y)};
        float y1[4], y2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x1 = acc[f][t][4 * j + e] * inv * g1[e];
          const float x2 = acc[f + 2][t][4 * j + e] * inv * g2[e];
          y1[e] = x1 * cc[e] - x2 * sn[e];
          y2[e] = x2 * cc[e] + x1 * sn[e];
        }
        u32x2 o1, o2;
        o1.x = pack_bf16x2(y1[0], y1[1]);
        o1.y = pack_bf16x2(y1[2], y1[3]);
        o2.x = pack_bf16x2(y2[0], y2[1]);
        o2.y = pack_bf16x2(y2[2], y2[3]);
        st8(dst + i0, o1);
        st8(dst + i0 + 64, o2);
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

// Few-token projection (decode): weight streaming.  A workgroup computes a
// C^T tile of 32 features x 64 tokens; its 8 waves each take one eighth of
// K, reading the MFMA fragments straight from global memory (the weights
// are read once; the activations stay in L2), and the partial tiles are
// summed through LDS.  Out-of-range rows and K tails read as zero.
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyUnroll = 4;

__global__ __launch_bounds__(64 * kSkinnyWaves) void gemm_skinny_kernel(GemmArgs a) {
  __shared__ floatx16 red[kSkinnyWaves - 1][2][64];
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int N = a.N, M = a.M, K = a.K;
  const int f0 = blockIdx.x * 32;
  const int m0 = blockIdx.y * 64;
  const int Kw = a.w_kmod > 0 ? a.w_kmod : K;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.W + (size_t)f0 * Kw, (long long)(N - f0) * Kw * 2);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.X + (size_t)m0 * K, (long long)(M - m0) * K * 2);
  const int ksteps = (K + 15) / 16;
  const int per = (ksteps + kSkinnyWaves - 1) / kSkinnyWaves;
  const int kb = wave * per * 16;
  const int ke = min(K, kb + per * 16);
  constexpr unsigned kOob = 0x80000000u;

  floatx16 acc0 = {}, acc1 = {};
  auto step = [&](int k) {
    const int kwc = k % Kw + 8 * hh;
    const int kxc = k + 8 * hh;
    const u32x4 fa = buf_ld16(rw, kwc < Kw ? (unsigned)((l32 * Kw + kwc) * 2) : kOob);
    const u32x4 fb0 = buf_ld16(rx, kxc < K ? (unsigned)((l32 * K + kxc) * 2) : kOob);
    const u32x4 fb1 = buf_ld16(rx, kxc < K ? (unsigned)(((32 + l32) * K + kxc) * 2) : kOob);
    acc0 = mfma32x32x16(fa, fb0, acc0);
    acc1 = mfma32x32x16(fa, fb1, acc1);
  };
  int k = kb;
  for (; k + 16 * kSkinnyUnroll <= ke; k += 16 * kSkinnyUnroll) {
#pragma unroll
    for (int u = 0; u < kSkinnyUnroll; ++u) step(k + 16 * u);
  }
  for (; k < ke; k += 16) step(k);

  if (wave > 0) {
    red[wave - 1][0][lane] = acc0;
    red[wave - 1][1][lane] = acc1;
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kSkinnyWaves - 1; ++w) {
    acc0 += red[w][0][lane];
    acc1 += red[w][1][lane];
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const floatx16& c = t == 0 ? acc0 : acc1;
    const int m = m0 + 32 * t + l32;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = f0 + 8 * j + 4 * hh;
      if (n >= N) continue;
      if (a.out_f32) {
        floatx4 w = {c[4 * j + 0], c[4 * j + 1], c[4 * j + 2], c[4 * j + 3]};
        *reinterpret_cast<floatx4*>(static_cast<float*>(a.out) + (size_t)m * N + n) = w;
      } else {
        u32x2 w;
        w.x = pack_bf16x2(c[4 * j + 0], c[4 * j + 1]);
        w.y = pack_bf16x2(c[4 * j + 2], c[4 * j + 3]);
        st8(static_cast<bf16*>(a.out) + (size_t)m * N + n, w);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_skinny_bf16(const GemmArgs& args, hipStream_t stream) {
  dim3 grid((args.N + 31) / 32, (args.M + 63) / 64);
  gemm_skinny_kernel<<<grid, 64 * kSkinnyWaves, 0, stream>>>(args);
  return hipGetLastError();
}

hipError_t launch_rope_table(float2* table, const int* start_pos, int rows, int L, int half,
                             double theta, hipStream_t stream) {
  const int n = rows * half;
  if (n == 0) return hipSuccess;
  rope_table_kernel<<<(n + 255) / 256, 256, 0, stream>>>(table, start_pos, rows, L, half, theta);
  return hipGetLastError();
}

hipError_t launch_gemm_qkv_bf16(const GemmArgs& args, hipStream_t stream) {
  constexpr int BN = 256, BM = 256;
  gemm_bf16_kernel<BN, BM, kEpiQKV><<<gemm_grid(args.N, args.M, BN, BM), kThreads, 0, stream>>>(args);
  return hipGetLastError();
}

hipError_t launch_gemm_plain_bf16(const GemmArgs& args, hipStream_t stream) {
  constexpr int BN = 256, BM = 256;
  gemm_bf16_kernel<BN, BM, kEpiPlain><<<gemm_grid(args.N, args.M, BN, BM), kThreads, 0, stream>>>(args);
  return hipGetLastError();
}

}  // namespace gqa
