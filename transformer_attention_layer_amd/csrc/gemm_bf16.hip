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
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gqa {

namespace {

constexpr int kBK = 32;          // K elements per LDS stage
constexpr int kStages = 4;       // LDS ring: loads run kStages - 1 stages ahead
constexpr int kCPR = kBK / 8;    // 16-byte chunks per LDS row
constexpr int kThreads = 256;    // 4 waves, 2 x 2 over the C^T tile

// LDS row of one tile: kBK bf16 = kCPR chunks of 16 B.  gfx950's LDS serves a
// 16-byte read 16 lanes at a time over 64 banks (256 B), and a fragment read
// has 16 lanes on 16 consecutive rows at one chunk index.  kRPW rows share
// one 256-byte bank window, so chunk c of row r lives at slot
// c ^ ((r / kRPW) % kCPR): the rows of a 16-row run that fall on the same
// window offset take kCPR distinct slots.
constexpr int kRPW = 256 / (kBK * 2);
static_assert(kRPW * kCPR == 16, "16 rows must cover every bank once");
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kCPR + (chunk ^ ((row / kRPW) & (kCPR - 1)));
}

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

// One operand's share of a K stage, staged straight from global memory into
// LDS (buffer_load ... lds, no register staging).  One instruction fills 64
// consecutive 16-byte LDS slots = kRowsPerDma rows; lane i writes slot i, so
// it loads the global chunk that the swizzle places there.  A wave issues
// kInstr of them per stage; the per-lane byte offsets at K = 0 are computed
// once, and chunks at or past column `kcols` read as zero.
constexpr int kRowsPerDma = 64 / kCPR;
static_assert(kRowsPerDma % (kRPW * kCPR) == 0, "one swizzle term per lane for all instructions");

template <int ROWS>
struct DmaPlan {
  static constexpr int kInstr = ROWS / kRowsPerDma / (kThreads / 64);
  unsigned voff[kInstr];  // byte offset of this lane's chunk at K = 0
  int kc;                 // K offset (elements) of this lane's chunk
  int slot0;              // first LDS slot of this wave's rows

  __device__ __forceinline__ void init(int ld, int wave, int lane) {
    const int r_in = lane / kCPR;
    // the swizzle term depends on row / kRPW, which is the same for every
    // instruction of the wave (rows advance in multiples of kRowsPerDma,
    // a multiple of kRPW * kCPR)
    const int c = (lane % kCPR) ^ ((r_in / kRPW) & (kCPR - 1));
#pragma unroll
    for (int j = 0; j < kInstr; ++j) {
      const int row = (wave * kInstr + j) * kRowsPerDma + r_in;
      voff[j] = (unsigned)((row * ld + c * 8) * 2);
    }
    kc = c * 8;
    slot0 = wave * kInstr * kRowsPerDma * kCPR;
  }

  // instruction j of the stage whose K offset is k0, into `stage` (the
  // operand's first slot in that LDS stage)
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rsrc, u32x4* stage, int j, int k0,
                                        int kcols) const {
    const unsigned v = k0 + kc < kcols ? voff[j] + (unsigned)(k0 * 2) : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(stage + slot0 + j * kRowsPerDma * kCPR), 16,
        v, 0, 0, 0);
  }
};

// s_waitcnt with the vector-memory counter limited to N (0..63): the oldest
// loads of this wave, all but its N most recent, have completed.  LDS: also
// wait for all of this wave's LDS reads.
template <int N, bool LDS = false>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | ((LDS ? 0 : 15) << 8));
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
  static_assert(kBK == 32 && kStages == 4, "the pipeline below is written for 2 substeps x 4 stages");
  static_assert(FB == 4 && TB == 4, "16 MFMAs per substep");
  __shared__ u32x4 lds[kStages][(BN + BM) * kCPR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
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
  DmaPlan<BN> pw;
  DmaPlan<BM> px;
  pw.init(Kw, wave, lane);
  px.init(K, wave, lane);
  constexpr int kLw = DmaPlan<BN>::kInstr, kLx = DmaPlan<BM>::kInstr;
  static_assert(kLw == 4 && kLx == 4, "one load per two MFMAs in each substep's second half");
  // K offset into W of stage kt (K <= 2 Kw: X = [hi | lo] reads W at most twice)
  auto w_k0 = [&](int kt) { const int k0 = kt * kBK; return k0 >= Kw ? k0 - Kw : k0; };
  auto stage_w = [&](int kt) { return &lds[kt % kStages][0]; };
  auto stage_x = [&](int kt) { return &lds[kt % kStages][BN * kCPR]; };

  // LDS offsets (16-byte slots) of this lane's fragments: row-major
  // fragments of W (features) and X (tokens), chunk = 2 * substep + hh
  int oa[2][FB], ob[2][TB];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
    for (int f = 0; f < FB; ++f) oa[sub][f] = swz(wn * WN + 32 * f + l32, 2 * sub + hh);
#pragma unroll
    for (int t = 0; t < TB; ++t) ob[sub][t] = BN * kCPR + swz(wm * WM + 32 * t + l32, 2 * sub + hh);
  }

  // Prologue: stages 0 .. kStages - 2 in flight, stage 0 landed and visible.
#pragma unroll
  for (int p = 0; p < kStages - 1; ++p) {
    if (p < nk) {
#pragma unroll
      for (int j = 0; j < kLw; ++j) pw.issue(rw, stage_w(p), j, w_k0(p), Kw);
#pragma unroll
      for (int j = 0; j < kLx; ++j) px.issue(rx, stage_x(p), j, p * kBK, K);
    }
  }
  if (nk >= 3) wait_vmem<2 * (kLw + kLx)>();
  else if (nk == 2) wait_vmem<kLw + kLx>();
  else wait_vmem<0>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  u32x4 fa[2][FB], fb[2][TB];
  {
    const u32x4* st = &lds[0][0];
#pragma unroll
    for (int f = 0; f < FB; ++f) fa[0][f] = st[oa[0][f]];
#pragma unroll
    for (int t = 0; t < TB; ++t) fb[0][t] = st[ob[0][t]];
  }

  // Main loop, one K stage (two 16-wide substeps) per trip.  Each substep
  // issues its 16 MFMAs interleaved with the 8 LDS reads of the next
  // substep's fragments (first half) and 4 of the loads of stage kt + 3
  // (second half), so that no wave stalls for long on a queue of loads.
  // Stage kt + 3 goes to the LDS stage of kt - 1.  Every wave's reads of
  // that stage had completed (s_waitcnt lgkmcnt(0)) before it reached the
  // barrier in the middle of trip kt - 1, which in turn makes stage kt
  // visible.  LOAD: stage kt + 3 exists; NEXT: stage kt + 1 exists.
  auto trip = [&](int kt, auto LOAD, auto NEXT) {
    const int kn = kt + kStages - 1;
    const int kwn = w_k0(kn);
    const u32x4* st = &lds[kt % kStages][0];
    const u32x4* st1 = &lds[(kt + 1) % kStages][0];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      if (sub == 1) {
        if constexpr (NEXT) {
          // stage kt + 1 landed: at most stage kt + 2 (8 loads) and the
          // first half of stage kt + 3 (4 loads) may still be in flight;
          // this wave's reads of stage kt are done
          if constexpr (LOAD) wait_vmem<kLw + kLx + kLw, true>();
          else if (kt + 2 < nk) wait_vmem<kLw + kLx, true>();
          else wait_vmem<0, true>();
          __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      const bool reads = sub == 0 || NEXT;
      const u32x4* rs = sub == 0 ? st : st1;
      const int(&ra)[FB] = oa[sub ^ 1];
      const int(&rb)[TB] = ob[sub ^ 1];
#pragma unroll
      for (int i = 0; i < FB * TB; ++i) {
        const int f = i / TB, t = i % TB;
        acc[f][t] = mfma32x32x16(fa[sub][f], fb[sub][t], acc[f][t]);
        if (i < 8) {
          // next substep's fragments in the order its MFMAs use them
          if (reads) {
            if (i == 0) fa[sub ^ 1][0] = rs[ra[0]];
            else if (i <= 4) fb[sub ^ 1][i - 1] = rs[rb[i - 1]];
            else fa[sub ^ 1][i - 4] = rs[ra[i - 4]];
          }
        } else if ((i & 1) == 0) {
          if constexpr (LOAD) {
            const int j = (i - 8) / 2;
            if (sub == 0) pw.issue(rw, stage_w(kn), j, kwn, Kw);
            else px.issue(rx, stage_x(kn), j, kn * kBK, K);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  using True = std::integral_constant<bool, true>;
  using False = std::integral_constant<bool, false>;
  int kt = 0;
  for (; kt < nk - (kStages - 1); ++kt) trip(kt, True(), True());
  for (; kt < nk - 1; ++kt) trip(kt, False(), True());
  trip(kt, False(), False());

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
  // Per 32-token block the lane's values are normalised and rotated in
  // registers and written to this wave's 32 KB of LDS as rows of 128 bf16
  // per token; the rows are then stored 16 bytes per lane, 4 whole rows per
  // instruction (a head's rows are contiguous in q and in the caches).
  // Row r's 16-byte chunk c sits at slot c ^ (r & 15).
  __syncthreads();  // every wave is done reading the last K stages
  if (nw >= N) return;  // wave-uniform
  const int head = nw >> 7;
  const int Hq = a.Hq, Hkv = a.Hkv;
  int kind;       // 0 = q, 1 = k, 2 = v
  int h;
  if (head < Hq) { kind = 0; h = head; }
  else if (head < Hq + Hkv) { kind = 1; h = head - Hq; }
  else { kind = 2; h = head - Hq - Hkv; }
  u32x4* const stage = &lds[wave][0];   // 128 rows x 16 chunks
  u32x2* const stage8 = reinterpret_cast<u32x2*>(stage);
  auto put8 = [&](int row, int feat, u32x2 v) {  // 4 features at feat (multiple of 4)
    stage8[(row * 16 + ((feat >> 3) ^ (row & 15))) * 2 + ((feat >> 2) & 1)] = v;
  };

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
  // consecutive features i..i+3 together with their RoPE partners
  // i+rot/2..i+rot/2+3, so only a few values are live at once.
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    const int row = 32 * t + l32;
    const int m = m0 + wm * WM + row;
    const int mm = m < M ? m : 0;
    const int tok = mm % a.L;
    float inv = 1.0f;
    if (do_norm) {
      float ss = 0.f;
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) ss += acc[f][t][r] * acc[f][t][r];
      ss = sum_xor32(ss);
      inv = 1.0f / __builtin_sqrtf(ss * (1.0f / 128.0f) + a.eps);
    }
    if (kind == 2) {
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 w;
          w.x = pack_bf16x2(acc[f][t][4 * j + 0], acc[f][t][4 * j + 1]);
          w.y = pack_bf16x2(acc[f][t][4 * j + 2], acc[f][t][4 * j + 3]);
          put8(row, 32 * f + 8 * j + 4 * hh, w);
        }
      continue;
    }
    // rotate-half RoPE over the first `rot` features: feature i < rot/2
    // pairs with i + rot/2 (rot 128: block f with f + 2; rot 64: block 0
    // with block 1, blocks 2 and 3 pass through)
    const int half = a.rot >> 1;
    const float2* cs = a.rope + (size_t)(a.start_pos ? mm : tok) * half;
    auto rope_pair = [&](int f1, int f2, int j) {
      const int i0 = 32 * f1 + 8 * j + 4 * hh;
      // (cos, sin) of features i0 .. i0+3: two 16-byte loads
      const floatx4 c01 = *reinterpret_cast<const floatx4*>(cs + i0);
      const floatx4 c23 = *reinterpret_cast<const floatx4*>(cs + i0 + 2);
      const float cc[4] = {c01[0], c01[2], c23[0], c23[2]};
      const float sn[4] = {c01[1], c01[3], c23[1], c23[3]};
      const u32x2 w1 = wpk[f1][j], w2 = wpk[f2][j];
      const float g1[4] = {lo_bf16(w1.x), hi_bf16(w1.x), lo_bf16(w1.y), hi_bf16(w1.y)};
      const float g2[4] = {lo_bf16(w2.x), hi_bf16(w2.x), lo_bf16(w2.y), hi_bf16(w2.y)};
      float y1[4], y2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x1 = acc[f1][t][4 * j + e] * inv * g1[e];
        const float x2 = acc[f2][t][4 * j + e] * inv * g2[e];
        y1[e] = x1 * cc[e] - x2 * sn[e];
        y2[e] = x2 * cc[e] + x1 * sn[e];
      }
      u32x2 o1, o2;
      o1.x = pack_bf16x2(y1[0], y1[1]);
      o1.y = pack_bf16x2(y1[2], y1[3]);
      o2.x = pack_bf16x2(y2[0], y2[1]);
      o2.y = pack_bf16x2(y2[2], y2[3]);
      put8(row, i0, o1);
      put8(row, i0 + half, o2);
    };
    auto norm_only = [&](int f, int j) {
      const u32x2 w = wpk[f][j];
      u32x2 o;
      o.x = pack_bf16x2(acc[f][t][4 * j + 0] * inv * lo_bf16(w.x),
                        acc[f][t][4 * j + 1] * inv * hi_bf16(w.x));
      o.y = pack_bf16x2(acc[f][t][4 * j + 2] * inv * lo_bf16(w.y),
                        acc[f][t][4 * j + 3] * inv * hi_bf16(w.y));
      put8(row, 32 * f + 8 * j + 4 * hh, o);
    };
    if (a.rot == 128) {
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) rope_pair(f, f + 2, j);
    } else {  // rot == 64
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        rope_pair(0, 1, j);
        norm_only(2, j);
        norm_only(3, j);
      }
    }
  }

  // Store: lane l moves chunk l % 16 of row 4 i + l / 16.
  const int c = lane & 15;
#pragma unroll 4
  for (int i = 0; i < WM / 4; ++i) {
    const int row = 4 * i + (lane >> 4);
    const int m = m0 + wm * WM + row;
    if (m >= M) continue;
    const int b = m / a.L;
    const int tok = m - b * a.L;
    bf16* dst;
    if (kind == 0) {
      dst = a.q + (((size_t)b * Hq + h) * a.L + tok) * 128;
    } else {
      const int pos = (a.start_pos ? a.start_pos[b] : 0) + tok;
      if (pos < 0 || pos >= a.cap) continue;
      bf16* cache = kind == 1 ? a.k_cache : a.v_cache;
      dst = cache + (((size_t)b * Hkv + h) * a.cap + pos) * 128;
    }
    st16(dst + 8 * c, stage[row * 16 + (c ^ (row & 15))]);
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
