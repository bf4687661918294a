// Backward of the grouped attention on the bf16 matrix cores of gfx950,
// head_dim 64 or 128, without a cache (the keys are the sequence's own L
// tokens).
//
// With s = q k^T * scale, p = softmax(s) by rows and o = p v (tutorial
// "Multi-Head and Grouped-Query Attention (Full Layer)", section 4 step 6),
// the gradients for an upstream dO are
//   dv_j = sum_i p_ij dO_i,          dp_ij = dO_i . v_j,
//   ds_ij = p_ij (dp_ij - D_i),      D_i = sum_j p_ij dp_ij = dO_i . o_i,
//   dq_i = scale sum_j ds_ij k_j,    dk_j = scale sum_i ds_ij q_i,
// and the dk, dv of a KV head sum over the query heads of its group
// ("Attention head partitions: keep each head's dependencies intact").  p is
// recomputed from the forward's per-row log-sum-exp.
//
// Two kernels and no atomics, so the results do not depend on timing:
//   dQ : the forward prefill's work split; a wave owns 32 query rows of one
//        head and walks the key tiles.  Scores are formed transposed
//        (S^T = K Q^T and dP^T = V dO^T, lane = query), so the row terms
//        lse and D are one scalar per lane, and dS^T goes from registers
//        straight into dQ^T += K^T dS^T, whose K^T operand comes from
//        transposing LDS reads.  It also forms D from dO and o.
//   dKV: a workgroup owns 128 keys of one KV head (a wave 32 of them, as
//        MFMA columns: S = Q K^T and dP = dO V^T, lane = key), keeps their
//        K and V fragments in registers and walks every query head of the
//        group and every query tile that can see them; dV^T += dO^T P and
//        dK^T += Q^T dS take P and dS from registers, dO^T and Q^T from
//        transposing LDS reads of the staged tiles.
// Tiles sit in LDS with a swizzle under which both their row reads and their
// transposing reads are free of bank conflicts.
#include <type_traits>

#include "common.h"
#include "attn_tiles.h"
#include "kernels.h"

namespace gqa {
namespace {

constexpr int kBwdNT = 256;      // 4 waves
constexpr int kBwdTK = 32;       // keys per LDS tile (dQ): small enough for 2 waves per SIMD
constexpr int kBwdTQ = 64;       // queries per LDS tile (dK/dV)
constexpr int kBwdKeysWG = 128;  // keys per dK/dV workgroup, 32 per wave

// Fragment offsets into a tile stored with the both-way swizzle (Geo::bslot).
//   row[c]: 16-byte slot of the row fragment for feature step c (row l32,
//           chunk 2c + hh: features 16c + 8hh .. +7), MFMA A operand over
//           features.
//   tr0/tr1[d]: byte offsets of the two transposing reads that form the A
//           operand for 32-feature block d over the 16 rows of row group 0
//           (lane l = 16 G + i gets feature 32 d + l % 32 of rows
//           4 (G / 2) + 0..3 and, from the second read, 8 rows further on).
//           The swizzle repeats every 16 rows, so row group g is g * 16
//           rows further on.
template <int KD>
struct SwzOffsets {
  int row[Geo<KD>::NC];
  int tr0[Geo<KD>::NB];
  int tr1[Geo<KD>::NB];
};

template <int KD>
__device__ __forceinline__ void swz_offsets(SwzOffsets<KD>& o, int lane) {
  using G = Geo<KD>;
  const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int c = 0; c < G::NC; ++c) o.row[c] = G::bslot(l32, 2 * c + hh);
  const int Gq = lane >> 4, j = lane & 15;
  const int r0 = 4 * (Gq >> 1) + (j >> 2);
#pragma unroll
  for (int d = 0; d < G::NB; ++d) {
    const int feat = 32 * d + 16 * (Gq & 1) + 4 * (j & 3);
    o.tr0[d] = G::bslot(r0, feat >> 3) * 16 + (feat & 7) * 2;
    o.tr1[d] = G::bslot(r0 + 8, feat >> 3) * 16 + (feat & 7) * 2;
  }
}

// Loads of a tile of ROWS rows x KD bf16 straight into LDS (buffer_load ...
// lds) with the both-way swizzle; consecutive rows are `stride` bytes apart in
// global memory.  One instruction fills 64 consecutive slots; lane i writes
// slot i and so loads the chunk the swizzle puts there.  Rows past the
// descriptor's range read as zero.  USER tells the kernels' instantiations
// apart: hipcc emits the host launch stub of only the first of two kernel
// templates that call the same instantiation of this member.
template <int KD, int ROWS, int USER>
struct RowTile {
  using G = Geo<KD>;
  static constexpr int JW = ROWS / G::RPI / (kBwdNT / 64);
  static_assert(JW >= 1 && JW * G::RPI * (kBwdNT / 64) == ROWS, "rows split evenly over waves");
  unsigned off[JW];
  int slot0;

  __device__ __forceinline__ void init(int wave, int lane, int stride) {
#pragma unroll
    for (int j = 0; j < JW; ++j) {
      const int row = (wave * JW + j) * G::RPI + lane / G::NCH;
      const int p = lane % G::NCH;
      off[j] = (unsigned)(row * stride + ((p ^ G::bswz(row)) << 4));
    }
    slot0 = wave * JW * 64;
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, lds_u32x4* dst) const {
#pragma unroll
    for (int j = 0; j < JW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst + slot0 + 64 * j, 16, off[j], 0, 0, 0);
  }
};

// Descriptor over rows r0 .. nrows - 1 of a row-major bf16 array whose rows
// are `stride` bytes apart and KD * 2 bytes long.
template <int KD>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const bf16* row0, int n, int stride) {
  const long long bytes = n > 0 ? (long long)(n - 1) * stride + KD * 2 : 0;
  return make_rsrc(row0, bytes);
}

// sum of the 8 products of two bf16 x 8 vectors, accumulated into acc.
// Each element is copied to a scalar before the bit cast: hipcc bit-casts
// an element expression of a vector as if it were element 0.
__device__ __forceinline__ float dot8_bf16(u32x4 a, u32x4 b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned ai = a[i], bi = b[i];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ai),
                                          __builtin_bit_cast(bf16x2, bi), acc, false);
  }
  return acc;
}

// s_waitcnt with the vector-memory counter at N (0..63): all but this
// wave's N most recent vector memory operations (here: LDS DMA) are done.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// log-sum-exp of a row in log2 units of the scaled score; a row with no
// visible key (-inf) gets +inf, so that every p of it is 0.
__device__ __forceinline__ float lse_log2(float lse) {
  return lse == -INFINITY ? INFINITY : lse * GQA_LOG2E;
}

__device__ __forceinline__ u32x4 pack8(const float (&v)[8]) {
  u32x4 r;
  r.x = pack_bf16x2(v[0], v[1]);
  r.y = pack_bf16x2(v[2], v[3]);
  r.z = pack_bf16x2(v[4], v[5]);
  r.w = pack_bf16x2(v[6], v[7]);
  return r;
}

// A operand over 16 rows of row group g for feature block d, from a tile
// with the both-way swizzle: rows become the MFMA's K index in the order the score
// registers hold them (4 hh + 0..3, then 8 + 4 hh + 0..3).
template <int KD>
__device__ __forceinline__ u32x4 tr_frag(const lds_u32x4* tile, const SwzOffsets<KD>& so, int g,
                                         int d) {
  lds_cchar* base = reinterpret_cast<lds_cchar*>(tile) + g * 16 * Geo<KD>::RB;
  const u32x2 a = lds_read_tr16(base + so.tr0[d]);
  const u32x2 b = lds_read_tr16(base + so.tr1[d]);
  return u32x4{a.x, a.y, b.x, b.y};
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------

// One key tile of the dQ kernel.  Lane = query (l % 32); register r of a
// 32-key block holds key 8 (r / 4) + 4 hh + r % 4.
template <int KD, int TK>
__device__ __forceinline__ void dq_tile(floatx16 (&dq)[Geo<KD>::NB],
                                        const u32x4 (&qf)[Geo<KD>::NC],
                                        const u32x4 (&df)[Geo<KD>::NC], const lds_u32x4* sk,
                                        const lds_u32x4* sv, const SwzOffsets<KD>& so, int key0,
                                        int kend_row, bool masked, float c_log2, float lse2,
                                        float drow, int hh) {
  using G = Geo<KD>;
  constexpr int KB = TK / 32, NG = TK / 16;
  floatx16 s[KB], dp[KB];
  const floatx16 z = {};
  // S^T = K Q^T and dP^T = V dO^T over the feature steps; each step's row
  // fragments are read while the previous step's MFMAs run
  u32x4 fa[2][2 * KB];  // [buffer][K rows of block kb | V rows of block kb]
  auto read_rows = [&](int c, u32x4(&f)[2 * KB]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f[kb] = sk[kb * 32 * G::NCH + so.row[c]];
      f[KB + kb] = sv[kb * 32 * G::NCH + so.row[c]];
    }
  };
  read_rows(0, fa[0]);
#pragma unroll
  for (int c = 0; c < G::NC; ++c) {
    if (c + 1 < G::NC) read_rows(c + 1, fa[(c + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      s[kb] = mfma32x32x16(fa[c & 1][kb], qf[c], c == 0 ? z : s[kb]);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      dp[kb] = mfma32x32x16(fa[c & 1][KB + kb], df[c], c == 0 ? z : dp[kb]);
    __builtin_amdgcn_sched_barrier(0);
  }
  u32x4 fb[2][G::NB];  // K^T fragments of one 16-key group
  auto read_tr = [&](int g, u32x4(&f)[G::NB]) {
#pragma unroll
    for (int d = 0; d < G::NB; ++d) f[d] = tr_frag<KD>(sk, so, g, d);
  };
  read_tr(0, fb[0]);
  __builtin_amdgcn_sched_barrier(0);
  u32x4 dsf[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int kb = g >> 1, rb = 8 * (g & 1);
    float p[8], ds[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = fast_exp2(__builtin_fmaf(s[kb][rb + e], c_log2, -lse2));
    if (masked) {
      // a real branch: only the diagonal and tail tiles pay for the mask
      asm volatile("");
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = rb + e;
        const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key >= kend_row) p[e] = 0.f;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ds[e] = p[e] * (dp[kb][rb + e] - drow);
    dsf[g] = pack8(ds);
  }
  __builtin_amdgcn_sched_barrier(0);
  // dQ^T += K^T dS^T per 16-key group, the next group's K^T read meanwhile
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (g + 1 < NG) read_tr(g + 1, fb[(g + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < G::NB; ++d) dq[d] = mfma32x32x16(fb[g & 1][d], dsf[g], dq[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int KD>
__global__ __launch_bounds__(kBwdNT, 2) void attn_bwd_dq_kernel(AttnBwdArgs a) {
  using G = Geo<KD>;
  constexpr int TK = kBwdTK;
  using Tile = RowTile<KD, TK, 0>;
  __shared__ u32x4 sk0[TK * G::NCH], sk1[TK * G::NCH];
  __shared__ u32x4 sv0[TK * G::NCH], sv1[TK * G::NCH];
  poison_lds(sk0, sk1, sv0, sv1);
  lds_u32x4* const sk[2] = {(lds_u32x4*)sk0, (lds_u32x4*)sk1};
  lds_u32x4* const sv[2] = {(lds_u32x4*)sv0, (lds_u32x4*)sv1};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int qt = a.n_qtiles - 1 - (int)blockIdx.z;  // heaviest query tiles first
  const int b = blockIdx.y;
  // the n_hsub workgroups of one KV group's heads are Hkv apart in x, so
  // with Hkv a multiple of 8 they run on one XCD and share its L2 for the
  // group's K/V tiles
  const int kvh = blockIdx.x % a.Hkv;
  const int hsub = blockIdx.x / a.Hkv;
  const int head_local = wave % a.hpw;
  const int pblk = wave / a.hpw;
  const int hq = kvh * a.G + hsub * a.hpw + head_local;
  const int L = a.L;

  const int wg_t0 = qt * a.pb * 32;
  const int wg_tlast = min(wg_t0 + a.pb * 32, L) - 1;
  const int key_end_wg = a.causal ? wg_tlast + 1 : L;
  const int n_tiles = (key_end_wg + TK - 1) / TK;
  const int t0 = wg_t0 + pblk * 32;
  const bool wave_live = t0 < L;
  const int w_tlast = min(t0 + 31, L - 1);
  const int key_end_w = wave_live ? (a.causal ? w_tlast + 1 : L) : 0;
  const int kmin_w = a.causal ? min(L, t0 + 1) : L;  // keys below it: visible to every row
  const int tq = t0 + l32;
  const bool row_valid = tq < L;
  const int kend_row = row_valid ? (a.causal ? tq + 1 : L) : 0;

  // B operands (lane = query; features 16 c + 8 hh .. +7): q and dO; and
  // D = dO . o over the same features, summed with lane l ^ 32
  u32x4 qf[G::NC], df[G::NC];
  const size_t qrow = ((size_t)b * a.Hq + hq) * L + (row_valid ? tq : 0);
  const size_t orow = (((size_t)b * L + (row_valid ? tq : 0)) * a.Hq + hq) * KD;
  float dsum = 0.f;
#pragma unroll
  for (int c = 0; c < G::NC; ++c) {
    u32x4 qv = {0u, 0u, 0u, 0u}, dv = qv, ov = qv;
    if (row_valid) {
      qv = ld16(a.q + qrow * KD + 16 * c + 8 * hh);
      dv = ld16(a.dO + orow + 16 * c + 8 * hh);
      ov = ld16(a.o + orow + 16 * c + 8 * hh);
    }
    qf[c] = qv;
    df[c] = dv;
    dsum = dot8_bf16(dv, ov, dsum);
  }
  const float drow = sum_xor32(dsum);
  float lse2 = INFINITY;
  if (row_valid) {
    lse2 = lse_log2(a.lse[qrow]);
    if (hh == 0) {
      a.D[qrow] = drow;
      a.lse2[qrow] = lse2;
    }
  }

  floatx16 dq[G::NB];
#pragma unroll
  for (int d = 0; d < G::NB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[d][r] = 0.f;

  SwzOffsets<KD> so;
  swz_offsets<KD>(so, lane);
  Tile plan;
  plan.init(wave, lane, G::RB);
  const size_t kv_base = ((size_t)b * a.Hkv + kvh) * L * KD;
  auto rk_at = [&](int k0) { return rows_rsrc<KD>(a.k + kv_base + (size_t)k0 * KD, L - k0, G::RB); };
  auto rv_at = [&](int k0) { return rows_rsrc<KD>(a.v + kv_base + (size_t)k0 * KD, L - k0, G::RB); };

  if (n_tiles > 0) {
    plan.load(rk_at(0), sk[0]);
    plan.load(rv_at(0), sv[0]);
  }
  __syncthreads();
  // two tiles per trip, so each buffer's LDS addresses are constants; the
  // next tile goes to the other buffer, whose last reads were before the
  // barrier that ended the previous trip
  auto step = [&](auto bufc, int it) {
    constexpr int B = decltype(bufc)::value;
    if (it + 1 < n_tiles) {
      plan.load(rk_at((it + 1) * TK), sk[B ^ 1]);
      plan.load(rv_at((it + 1) * TK), sv[B ^ 1]);
    }
    const int key0 = it * TK;
    if (key0 < key_end_w) {
      const bool masked = key0 + TK > kmin_w;
      dq_tile<KD, TK>(dq, qf, df, sk[B], sv[B], so, key0, kend_row, masked, a.scale_log2, lse2,
                      drow, hh);
    }
    __syncthreads();
  };
  for (int it = 0; it < n_tiles; it += 2) {
    step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < n_tiles) step(std::integral_constant<int, 1>{}, it + 1);
  }

  if (!row_valid) return;
  // dQ^T: lane = query, register r of block d = feature 32 d + 8 (r / 4) + 4 hh + r % 4
  bf16* dst = a.dq + qrow * KD;
#pragma unroll
  for (int d = 0; d < G::NB; ++d)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 w;
      w.x = pack_bf16x2(dq[d][4 * j] * a.scale, dq[d][4 * j + 1] * a.scale);
      w.y = pack_bf16x2(dq[d][4 * j + 2] * a.scale, dq[d][4 * j + 3] * a.scale);
      st8(dst + 32 * d + 8 * j + 4 * hh, w);
    }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------

// One 64-query tile of one query head for the dK/dV kernel.  Lane = key
// (l % 32); register r of a 32-query block holds query 8 (r / 4) + 4 hh +
// r % 4.  sl / sD hold the tile's 64 row log-sum-exps (log2 units) and D.
// Both 32-query blocks always run: a block with no visible pair is masked
// to p = 0 (it only occurs on the diagonal tile).
template <int KD>
__device__ __forceinline__ void dkv_tile(floatx16 (&dk)[Geo<KD>::NB], floatx16 (&dv)[Geo<KD>::NB],
                                         const u32x4 (&kf)[Geo<KD>::NC],
                                         const u32x4 (&vf)[Geo<KD>::NC], const lds_u32x4* sq,
                                         const lds_u32x4* sd, const lds_float* sl,
                                         const lds_float* sD, const SwzOffsets<KD>& so, int q0,
                                         int kw0, int key, int L, bool causal, float c_log2,
                                         int hh) {
  using G = Geo<KD>;
  constexpr int TQ = kBwdTQ, QB = TQ / 32, NG = TQ / 16;
  floatx16 s[QB], dp[QB];
  const floatx16 z = {};
  // S = Q K^T and dP = dO V^T over the feature steps; each step's row
  // fragments are read while the previous step's MFMAs run
  u32x4 fa[2][2 * QB];  // [buffer][Q rows of block qb | dO rows of block qb]
  auto read_rows = [&](int c, u32x4(&f)[2 * QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f[qb] = sq[qb * 32 * G::NCH + so.row[c]];
      f[QB + qb] = sd[qb * 32 * G::NCH + so.row[c]];
    }
  };
  read_rows(0, fa[0]);
#pragma unroll
  for (int c = 0; c < G::NC; ++c) {
    if (c + 1 < G::NC) read_rows(c + 1, fa[(c + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      s[qb] = mfma32x32x16(fa[c & 1][qb], kf[c], c == 0 ? z : s[qb]);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      dp[qb] = mfma32x32x16(fa[c & 1][QB + qb], vf[c], c == 0 ? z : dp[qb]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the first row group's transposed fragments (dO^T, Q^T) go out now and
  // land while the softmax terms are formed
  u32x4 fb[2][2 * G::NB];  // [buffer][dO^T of block d | Q^T of block d]
  auto read_tr = [&](int g, u32x4(&f)[2 * G::NB]) {
#pragma unroll
    for (int d = 0; d < G::NB; ++d) {
      f[d] = tr_frag<KD>(sd, so, g, d);
      f[G::NB + d] = tr_frag<KD>(sq, so, g, d);
    }
  };
  read_tr(0, fb[0]);
  __builtin_amdgcn_sched_barrier(0);
  u32x4 pf[NG], dsf[NG];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qb0 = q0 + 32 * qb;
    const bool masked = (causal && qb0 < kw0 + 31) || qb0 + 32 > L;  // wave-uniform
    float pv[16], dsv[16];
    floatx4 d4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const floatx4 l4 = *reinterpret_cast<const lds_floatx4*>(sl + 32 * qb + 8 * i + 4 * hh);
      d4[i] = *reinterpret_cast<const lds_floatx4*>(sD + 32 * qb + 8 * i + 4 * hh);
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[4 * i + e] = fast_exp2(__builtin_fmaf(s[qb][4 * i + e], c_log2, -l4[e]));
    }
    if (masked) {
      // a real branch: only diagonal and tail tiles pay for the mask
      asm volatile("");
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = qb0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (q >= L || (causal && q < key)) pv[r] = 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) dsv[r] = pv[r] * (dp[qb][r] - d4[r >> 2][r & 3]);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      float p8[8], d8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p8[e] = pv[8 * h2 + e];
        d8[e] = dsv[8 * h2 + e];
      }
      pf[2 * qb + h2] = pack8(p8);
      dsf[2 * qb + h2] = pack8(d8);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // dV^T += dO^T P and dK^T += Q^T dS per 16-query group; the next group's
  // fragments are read while the current group's MFMAs run
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (g + 1 < NG) read_tr(g + 1, fb[(g + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < G::NB; ++d) {
      dv[d] = mfma32x32x16(fb[g & 1][d], pf[g], dv[d]);
      dk[d] = mfma32x32x16(fb[g & 1][G::NB + d], dsf[g], dk[d]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int KD>
__global__ __launch_bounds__(kBwdNT) void attn_bwd_dkv_kernel(AttnBwdArgs a) {
  using G = Geo<KD>;
  constexpr int TQ = kBwdTQ;
  using Tile = RowTile<KD, TQ, 1>;
  // a ring of 3 tile slots: tile it + 2 loads while tile it is used
  __shared__ u32x4 sq0[TQ * G::NCH], sq1[TQ * G::NCH], sq2[TQ * G::NCH];
  __shared__ u32x4 sd0[TQ * G::NCH], sd1[TQ * G::NCH], sd2[TQ * G::NCH];
  __shared__ float sl0[TQ], sl1[TQ], sl2[TQ], sD0[TQ], sD1[TQ], sD2[TQ];
  poison_lds(sq0, sq1, sq2, sd0, sd1, sd2, sl0, sl1, sl2, sD0, sD1, sD2);
  lds_u32x4* const sq[3] = {(lds_u32x4*)sq0, (lds_u32x4*)sq1, (lds_u32x4*)sq2};
  lds_u32x4* const sd[3] = {(lds_u32x4*)sd0, (lds_u32x4*)sd1, (lds_u32x4*)sd2};
  lds_float* const sl[3] = {(lds_float*)sl0, (lds_float*)sl1, (lds_float*)sl2};
  lds_float* const sD[3] = {(lds_float*)sD0, (lds_float*)sD1, (lds_float*)sD2};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  // XCD-aware order: workgroup i runs on XCD i % 8; the key blocks of one
  // (sequence, KV head) all go to the same XCD, so that they share its L2
  // for the query tiles they all read (in the same, descending order).  On
  // an XCD the key blocks go out block-index major: with the causal mask
  // block 0 sees every query tile and the last one the fewest, so the
  // heaviest workgroups start first and the lightest fill the end.
  const int L = a.L;
  const int gpx = (a.B * a.Hkv + 7) / 8;  // (sequence, KV head) pairs per XCD
  const int xcd = (int)(blockIdx.x % 8), slot = (int)(blockIdx.x / 8);
  const int kblk = slot / gpx;
  const int grp = xcd + 8 * (slot - kblk * gpx);  // (sequence, KV head) pair
  if (grp >= a.B * a.Hkv) return;  // padding of the grid to a multiple of 8 groups
  const int b = grp / a.Hkv, kvh = grp - b * a.Hkv;
  const int kwg0 = kblk * kBwdKeysWG;
  const int kw0 = kwg0 + wave * 32;
  const int key = kw0 + l32;
  const bool key_valid = key < L;

  // B operands (lane = key; features 16 c + 8 hh .. +7)
  u32x4 kf[G::NC], vf[G::NC];
  const size_t krow = ((size_t)b * a.Hkv + kvh) * L + (key_valid ? key : 0);
#pragma unroll
  for (int c = 0; c < G::NC; ++c) {
    u32x4 kv = {0u, 0u, 0u, 0u}, vv = kv;
    if (key_valid) {
      kv = ld16(a.k + krow * KD + 16 * c + 8 * hh);
      vv = ld16(a.v + krow * KD + 16 * c + 8 * hh);
    }
    kf[c] = kv;
    vf[c] = vv;
  }
  floatx16 dk[G::NB], dv[G::NB];
#pragma unroll
  for (int d = 0; d < G::NB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[d][r] = 0.f;
      dv[d][r] = 0.f;
    }

  const int nqt = (L + TQ - 1) / TQ;
  const int qt0 = a.causal ? kwg0 / TQ : 0;
  const int per_head = nqt - qt0;
  const int n_it = a.G * per_head;
  const int dstride = a.Hq * KD * 2;  // bytes between tokens of dO
  Tile plan_q, plan_d;
  plan_q.init(wave, lane, G::RB);
  plan_d.init(wave, lane, dstride);
  SwzOffsets<KD> so;
  swz_offsets<KD>(so, lane);

  auto head_of = [&](int it) { return kvh * a.G + it / per_head; };
  auto q0_of = [&](int it) { return (nqt - 1 - it % per_head) * TQ; };
  // a tile's Q and dO rows (every wave a share), and its 64 lse2 and D
  // values (one 4-byte load per lane, waves 0 and 1); rows past L read 0
  auto load = [&](int it, lds_u32x4* dq_, lds_u32x4* dd_, lds_float* dl_, lds_float* dD_) {
    const int hq = head_of(it), q0 = q0_of(it);
    plan_q.load(rows_rsrc<KD>(a.q + (((size_t)b * a.Hq + hq) * L + q0) * KD, L - q0, G::RB), dq_);
    plan_d.load(rows_rsrc<KD>(a.dO + (((size_t)b * L + q0) * a.Hq + hq) * KD, L - q0, dstride),
                dd_);
    const size_t lrow = ((size_t)b * a.Hq + hq) * L + q0;
    if (wave < 2) {
      const float* src = wave == 0 ? a.lse2 + lrow : a.D + lrow;
      lds_float* dst = wave == 0 ? dl_ : dD_;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(src, (long long)(L - q0) * 4),
                                               (__attribute__((address_space(3))) void*)dst, 4,
                                               (unsigned)lane * 4, 0, 0, 0);
    }
  };

  if (n_it > 0) load(0, sq[0], sd[0], sl[0], sD[0]);
  if (n_it > 1) load(1, sq[1], sd[1], sl[1], sD[1]);
  // Per tile: wait for this wave's loads of tile it (those of tile it + 1
  // may stay in flight; loads complete in order), barrier (every wave's
  // share landed, and every wave is done with tile it - 1), then load tile
  // it + 2 into the slot of tile it - 1.  Slots are compile-time constants.
  auto step = [&](auto slotc, int it) {
    constexpr int S = decltype(slotc)::value;
    if (it + 1 < n_it) {
      if (wave < 2) wait_vm<2 * Tile::JW + 1>();
      else wait_vm<2 * Tile::JW>();
    } else {
      wait_vm<0>();
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    constexpr int N2 = (S + 2) % 3;
    if (it + 2 < n_it) load(it + 2, sq[N2], sd[N2], sl[N2], sD[N2]);
    const int q0 = q0_of(it);
    if (kw0 < L && (!a.causal || q0 + TQ - 1 >= kw0))
      dkv_tile<KD>(dk, dv, kf, vf, sq[S], sd[S], sl[S], sD[S], so, q0, kw0, key, L,
                   a.causal != 0, a.scale_log2, hh);
  };
  for (int it = 0; it < n_it; it += 3) {
    step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < n_it) step(std::integral_constant<int, 1>{}, it + 1);
    if (it + 2 < n_it) step(std::integral_constant<int, 2>{}, it + 2);
  }

  if (!key_valid) return;
  // dK^T, dV^T: lane = key, register r of block d = feature 32 d + 8 (r / 4) + 4 hh + r % 4
  bf16* dkr = a.dk + krow * KD;
  bf16* dvr = a.dv + krow * KD;
#pragma unroll
  for (int d = 0; d < G::NB; ++d)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 wk, wv;
      wk.x = pack_bf16x2(dk[d][4 * j] * a.scale, dk[d][4 * j + 1] * a.scale);
      wk.y = pack_bf16x2(dk[d][4 * j + 2] * a.scale, dk[d][4 * j + 3] * a.scale);
      wv.x = pack_bf16x2(dv[d][4 * j], dv[d][4 * j + 1]);
      wv.y = pack_bf16x2(dv[d][4 * j + 2], dv[d][4 * j + 3]);
      st8(dkr + 32 * d + 8 * j + 4 * hh, wk);
      st8(dvr + 32 * d + 8 * j + 4 * hh, wv);
    }
}

template <int KD>
hipError_t launch_bwd(const AttnBwdArgs& a, hipStream_t stream) {
  dim3 g1(a.Hkv * a.n_hsub, a.B, a.n_qtiles);
  attn_bwd_dq_kernel<KD><<<g1, kBwdNT, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nkb = (a.L + kBwdKeysWG - 1) / kBwdKeysWG;
  const int groups = (a.B * a.Hkv + 7) / 8 * 8;  // the grid maps 8 groups at a time
  attn_bwd_dkv_kernel<KD><<<groups * nkb, kBwdNT, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch_bwd<64>(a, stream);
    case 128: return launch_bwd<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
