// Grouped causal attention on the bf16 matrix cores of gfx950, head_dim 128.
//
// Computes softmax(q k^T * d^-0.5 + mask) v with query head h reading KV
// head h / (Hq/Hkv) (tutorial "Multi-Head and Grouped-Query Attention (Full
// Layer)", section 4 step 6; "Attention head partitions: keep each head's
// dependencies intact" for the grouping; GPT-NeoX issue "Scaling and RoPE"
// for the scale).  The softmax is exact: it is evaluated tile by tile over
// the keys with a running maximum and sum ("num_heads Is Not a Capacity
// Knob", "Why the cost does not move": a flash-style kernel changes the
// memory traffic of the same products, not their result).
//
// Layout inside a wave.  A wave owns 32 query rows.  Scores are formed
// transposed, S^T = K Q^T (keys are MFMA rows, queries MFMA columns), so
// lane l holds one query (l % 32) and half of each 32-key block; the row max
// and sum need a single exchange with lane l ^ 32, and the rescale factor is
// one scalar per lane.  O^T = V^T P^T then takes P^T straight from the score
// registers; V^T is built in LDS while the tile is stored, with the keys of
// each 16-key group in the order the score registers hold them.
//
// Softmax bookkeeping per key tile: the tile's row max is taken on the raw
// scores (the scale is positive), exp2(s * scale*log2(e) - m) is one FMA and
// one v_exp, and the running max m is moved (and the output rescaled) only
// when some row's max grew by more than 2^8; until then p may exceed 1 by up
// to that factor, which bf16 P and the fp32 sums carry as well.  The row
// sums add the bf16-rounded P that the PV product uses (v_dot2).
//
// Two kernels:
//   prefill: a workgroup of 4 waves covers up to 4 query heads of one KV
//            group at the same 32 positions (or 2 heads x 64 positions, or
//            1 head x 128), so every wave walks the same causal key range and
//            each K/V tile is staged in LDS once for the whole group.
//   decode : one wave per (sequence, KV head, key split); its 32 rows are the
//            group's query heads (x the few new tokens).  Partial (max, sum,
//            unnormalised output) per split are merged by a second kernel.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gqa {
namespace {

constexpr int kD = 128;
constexpr float kLazyRescale = 8.0f;  // log2 of the growth allowed before rescaling

// K tile: rows = keys, 256 B = 16 chunks each; chunk c of row r at slot
// c ^ (r & 15).
__device__ __forceinline__ int kslot(int row, int chunk) { return (row << 4) + (chunk ^ (row & 15)); }

// V^T tile: rows = the 128 value features, TK keys each (TK/8 chunks).  Key
// 16g + 8a + 4h + i is stored at position 16g + 8h + 4a + i, so chunk 2g + h
// holds exactly the eight keys lane-half h feeds to the PV product of key
// group g.  Chunks are XOR-swizzled with (r ^ r>>2) to spread rows over banks.
template <int TK>
__device__ __forceinline__ int vslot(int row, int chunk) {
  constexpr int NCH = TK / 8;
  return row * NCH + (chunk ^ ((row ^ (row >> 2)) & (NCH - 1)));
}

// K tile straight into LDS (buffer_load ... lds): one instruction fills 64
// consecutive slots = 4 key rows; lane i writes slot i, so it loads the
// chunk the swizzle puts there.  Keys past the descriptor's range read as 0.
template <int NT, int TK>
__device__ __forceinline__ void dma_k(__amdgpu_buffer_rsrc_t rk, u32x4* sk, int key0, int wave,
                                      int lane) {
  constexpr int JW = TK / 4 / (NT / 64);  // instructions per wave
  const int r_in = lane >> 4;
  const int slot = lane & 15;
#pragma unroll
  for (int j = 0; j < JW; ++j) {
    const int r0 = (wave * JW + j) * 4;
    const int row = r0 + r_in;
    const int c = slot ^ (row & 15);
    dma16(rk, sk + r0 * 16, (unsigned)((key0 + row) * (kD * 2) + c * 16));
  }
}

// V tile through registers: a thread loads 4 keys x 4 features (8-byte
// loads, zero past the range) ...
template <int NT, int TK>
struct VRegs {
  static constexpr int kG = TK * 8 / NT;  // 4-key x 4-feature groups per thread
  u32x2 v[kG][4];
};

template <int NT, int TK>
__device__ __forceinline__ void load_v(VRegs<NT, TK>& r, __amdgpu_buffer_rsrc_t rv, int key0,
                                       int tid) {
#pragma unroll
  for (int i = 0; i < VRegs<NT, TK>::kG; ++i) {
    const int idx = tid + i * NT;
    const int g4 = idx & 31;
    const int kq = idx >> 5;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r.v[i][e] = buf_ld8(rv, (unsigned)((key0 + 4 * kq + e) * (kD * 2) + 8 * g4));
  }
}

// ... and stores them transposed: 4 features x 4 keys, each 8 bytes.
template <int NT, int TK>
__device__ __forceinline__ void store_vt(const VRegs<NT, TK>& r, u32x4* sv, int tid) {
  u32x2* sv2 = reinterpret_cast<u32x2*>(sv);
#pragma unroll
  for (int i = 0; i < VRegs<NT, TK>::kG; ++i) {
    const int idx = tid + i * NT;
    const int g4 = idx & 31;
    const int kq = idx >> 5;                 // keys 4kq .. 4kq+3 of the tile
    const int chunk = 2 * (kq >> 2) + (kq & 1);
    const int half = (kq >> 1) & 1;
    const u32x2* v = r.v[i];
    u32x2 t0, t1, t2, t3;
    t0.x = (v[0].x & 0xffffu) | (v[1].x << 16);
    t0.y = (v[2].x & 0xffffu) | (v[3].x << 16);
    t1.x = (v[0].x >> 16) | (v[1].x & 0xffff0000u);
    t1.y = (v[2].x >> 16) | (v[3].x & 0xffff0000u);
    t2.x = (v[0].y & 0xffffu) | (v[1].y << 16);
    t2.y = (v[2].y & 0xffffu) | (v[3].y << 16);
    t3.x = (v[0].y >> 16) | (v[1].y & 0xffff0000u);
    t3.y = (v[2].y >> 16) | (v[3].y & 0xffff0000u);
    const int row = 4 * g4;
    sv2[vslot<TK>(row + 0, chunk) * 2 + half] = t0;
    sv2[vslot<TK>(row + 1, chunk) * 2 + half] = t1;
    sv2[vslot<TK>(row + 2, chunk) * 2 + half] = t2;
    sv2[vslot<TK>(row + 3, chunk) * 2 + half] = t3;
  }
}

// Per-lane LDS offsets (u32x4 units) of the MFMA fragments; the same for
// every tile and buffer.
template <int TK>
struct LaneOffsets {
  int k[8];            // K fragment of d-chunk c: key row l32 (+32 kb)
  int v[TK / 16];      // V^T fragment of key group g: feature row l32 (+32 d)
};

template <int TK>
__device__ __forceinline__ void lane_offsets(LaneOffsets<TK>& o, int l32, int hh) {
#pragma unroll
  for (int c = 0; c < 8; ++c) o.k[c] = kslot(l32, 2 * c + hh);
#pragma unroll
  for (int g = 0; g < TK / 16; ++g) o.v[g] = vslot<TK>(l32, 2 * g + hh);
}

// Running state of one wave: 32 query rows, lane = row (l % 32).
struct RowState {
  floatx16 o[4];   // O^T: value feature 32*db + 8*(r/4) + 4*(l/32) + r%4
  float m;         // running max (log2 units, scaled scores)
  float l;         // running sum, this lane-half's keys only
};

__device__ __forceinline__ void init_state(RowState& st) {
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[d][r] = 0.f;
  st.m = -INFINITY;
  st.l = 0.f;
}

// One key tile: scores, online softmax, PV.  `kend_row` = one past the last
// key this lane's query may see; `masked` (wave-uniform) = some key of the
// tile may be past it for some row of the wave.
template <int TK>
__device__ __forceinline__ void attend_tile(RowState& st, const u32x4 (&qf)[8], const u32x4* sk,
                                            const u32x4* sv, const LaneOffsets<TK>& lo, int key0,
                                            int kend_row, bool masked, float c_log2, int hh) {
  constexpr int KB = TK / 32;
  constexpr int NCH = TK / 8;
  floatx16 s[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const floatx16 z = {};
    s[kb] = mfma32x32x16(sk[kb * 512 + lo.k[0]], qf[0], z);
#pragma unroll
    for (int c = 1; c < 8; ++c) s[kb] = mfma32x32x16(sk[kb * 512 + lo.k[c]], qf[c], s[kb]);
  }
  if (masked) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key >= kend_row) s[kb][r] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = fmaxf(mx, wave_xor32(mx));
  const float mt = mx * c_log2;  // -inf stays -inf (c_log2 > 0)
  if (__builtin_amdgcn_ballot_w64(mt > st.m + kLazyRescale)) {
    const float mn = fmaxf(st.m, mt);
    const float alpha = mn == -INFINITY ? 1.0f : fast_exp2(st.m - mn);
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[d][r] *= alpha;
    st.l *= alpha;
    st.m = mn;
  }
  const float mb = st.m == -INFINITY ? 0.f : st.m;
#pragma unroll
  for (int g = 0; g < TK / 16; ++g) {
    const int kb = g >> 1;
    const int rb = 8 * (g & 1);
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = fast_exp2(__builtin_fmaf(s[kb][rb + e], c_log2, -mb));
    u32x4 pf;
    pf.x = pack_bf16x2(p[0], p[1]);
    pf.y = pack_bf16x2(p[2], p[3]);
    pf.z = pack_bf16x2(p[4], p[5]);
    pf.w = pack_bf16x2(p[6], p[7]);
    st.l = sum_bf16x2(pf.x, st.l);
    st.l = sum_bf16x2(pf.y, st.l);
    st.l = sum_bf16x2(pf.z, st.l);
    st.l = sum_bf16x2(pf.w, st.l);
#pragma unroll
    for (int d = 0; d < 4; ++d) st.o[d] = mfma32x32x16(sv[d * 32 * NCH + lo.v[g]], pf, st.o[d]);
  }
}

__device__ __forceinline__ int kv_len_of(const AttnArgs& a, int b) {
  int n = (a.kv_base ? a.kv_base[b] : 0) + a.kv_add;
  return n < 0 ? 0 : (n > a.cap ? a.cap : n);
}

__device__ __forceinline__ void load_q(u32x4 (&qf)[8], const bf16* qrow, bool valid, int hh) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (valid) v = ld16(qrow + 16 * c + 8 * hh);
    qf[c] = v;
  }
}

// Four consecutive output features as bf16; with `split` also the rounding
// residual (value - bf16(value)) as bf16, `width` elements further on.
__device__ __forceinline__ void store_o4(bf16* p, size_t width, const float (&v)[4], int split) {
  u32x2 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  st8(p, w);
  if (split) {
    u32x2 r;
    r.x = pack_bf16x2(v[0] - lo_bf16(w.x), v[1] - hi_bf16(w.x));
    r.y = pack_bf16x2(v[2] - lo_bf16(w.y), v[3] - hi_bf16(w.y));
    st8(p + width, r);
  }
}

constexpr int kPrefillTK = 64;
constexpr int kPrefillNT = 256;

__global__ __launch_bounds__(kPrefillNT, 2) void attn_prefill_kernel(AttnArgs a) {
  constexpr int TK = kPrefillTK, NT = kPrefillNT;
  __shared__ u32x4 sk[2][TK * 16];
  __shared__ u32x4 sv[2][kD * TK / 8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int qt = a.n_qtiles - 1 - (int)blockIdx.z;  // heaviest query tiles first
  const int b = blockIdx.y;
  const int kvh = blockIdx.x / a.n_hsub;
  const int hsub = blockIdx.x - kvh * a.n_hsub;
  const int head_local = wave % a.hpw;
  const int pblk = wave / a.hpw;
  const int hq = kvh * a.G + hsub * a.hpw + head_local;

  const int kvl = kv_len_of(a, b);
  const int off = kvl - a.Lq;  // query i sits at position off + i
  const int wg_t0 = qt * a.pb * 32;
  const int wg_tlast = min(wg_t0 + a.pb * 32, a.Lq) - 1;
  const int key_end_wg = a.causal ? min(kvl, off + wg_tlast + 1) : kvl;
  const int n_tiles = key_end_wg > 0 ? (key_end_wg + TK - 1) / TK : 0;

  const int t0 = wg_t0 + pblk * 32;
  const bool wave_live = t0 < a.Lq;
  const int w_tlast = min(t0 + 31, a.Lq - 1);
  const int key_end_w = wave_live ? (a.causal ? min(kvl, off + w_tlast + 1) : kvl) : 0;
  const int kmin_w = a.causal ? min(kvl, off + t0 + 1) : kvl;
  const int tq = t0 + l32;
  const bool row_valid = tq < a.Lq;
  const int kend_row = row_valid ? (a.causal ? min(kvl, off + tq + 1) : kvl) : 0;

  u32x4 qf[8];
  load_q(qf, a.q + (((size_t)b * a.Hq + hq) * a.Lq + (row_valid ? tq : 0)) * kD, row_valid, hh);

  const size_t kv_base = ((size_t)b * a.Hkv + kvh) * a.cap * kD;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + kv_base, (long long)kvl * kD * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + kv_base, (long long)kvl * kD * 2);
  LaneOffsets<TK> lo;
  lane_offsets<TK>(lo, l32, hh);

  RowState st;
  init_state(st);
  VRegs<NT, TK> vr;
  if (n_tiles > 0) {
    dma_k<NT, TK>(rk, sk[0], 0, wave, lane);
    load_v<NT, TK>(vr, rv, 0, tid);
    store_vt<NT, TK>(vr, sv[0], tid);
  }
  __syncthreads();
  // two tiles per trip, so each buffer's LDS addresses are constants
  auto step = [&](auto bufc, int it) {
    constexpr int B = decltype(bufc)::value;
    const bool more = it + 1 < n_tiles;
    if (more) {
      dma_k<NT, TK>(rk, sk[B ^ 1], (it + 1) * TK, wave, lane);
      load_v<NT, TK>(vr, rv, (it + 1) * TK, tid);
    }
    const int key0 = it * TK;
    if (key0 < key_end_w) {
      const bool masked = key0 + TK > kmin_w;
      attend_tile<TK>(st, qf, sk[B], sv[B], lo, key0, kend_row, masked, a.scale_log2, hh);
    }
    if (more) store_vt<NT, TK>(vr, sv[B ^ 1], tid);
    __syncthreads();
  };
  for (int it = 0; it < n_tiles; it += 2) {
    step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < n_tiles) step(std::integral_constant<int, 1>{}, it + 1);
  }

  const float lt = st.l + wave_xor32(st.l);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (!row_valid) return;
  const size_t width = (size_t)a.Hq * kD;
  bf16* orow = a.o + ((size_t)b * a.Lq + tq) * width * (a.o_split ? 2 : 1) + (size_t)hq * kD;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = st.o[d][4 * j + i] * inv;
      store_o4(orow + 32 * d + 8 * j + 4 * hh, width, v, a.o_split);
    }
}

constexpr int kDecodeTK = 32;
constexpr int kDecodeNT = 64;

__global__ __launch_bounds__(kDecodeNT) void attn_decode_kernel(AttnArgs a) {
  constexpr int TK = kDecodeTK, NT = kDecodeNT;
  __shared__ u32x4 sk[2][TK * 16];
  __shared__ u32x4 sv[2][kD * TK / 8];

  const int lane = threadIdx.x;
  const int l32 = lane & 31, hh = lane >> 5;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int rows = a.G * a.Lq;
  const bool row_valid = l32 < rows;
  const int head_local = row_valid ? l32 / a.Lq : 0;
  const int tq = row_valid ? l32 - head_local * a.Lq : 0;
  const int hq = kvh * a.G + head_local;

  const int kvl = kv_len_of(a, b);
  const int off = kvl - a.Lq;
  const int ks = split * a.chunk;
  int ke = min(ks + a.chunk, kvl);
  if (a.causal) ke = min(ke, off + a.Lq);
  const int n_tiles = ke > ks ? (ke - ks + TK - 1) / TK : 0;
  const int kend_row = row_valid ? min(ke, a.causal ? min(kvl, off + tq + 1) : kvl) : 0;
  const int kmin = min(ke, a.causal ? min(kvl, off + 1) : kvl);

  u32x4 qf[8];
  load_q(qf, a.q + (((size_t)b * a.Hq + hq) * a.Lq + tq) * kD, row_valid, hh);

  const size_t kv_base = ((size_t)b * a.Hkv + kvh) * a.cap * kD;
  const long long bytes = (long long)(ke > 0 ? ke : 0) * kD * 2;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + kv_base, bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + kv_base, bytes);
  LaneOffsets<TK> lo;
  lane_offsets<TK>(lo, l32, hh);

  RowState st;
  init_state(st);
  VRegs<NT, TK> vr;
  if (n_tiles > 0) {
    dma_k<NT, TK>(rk, sk[0], ks, 0, lane);
    load_v<NT, TK>(vr, rv, ks, lane);
    store_vt<NT, TK>(vr, sv[0], lane);
  }
  __syncthreads();
  auto step = [&](auto bufc, int it) {
    constexpr int B = decltype(bufc)::value;
    const int key0 = ks + it * TK;
    const bool more = it + 1 < n_tiles;
    if (more) {
      dma_k<NT, TK>(rk, sk[B ^ 1], key0 + TK, 0, lane);
      load_v<NT, TK>(vr, rv, key0 + TK, lane);
    }
    const bool masked = key0 + TK > kmin;
    attend_tile<TK>(st, qf, sk[B], sv[B], lo, key0, kend_row, masked, a.scale_log2, hh);
    if (more) store_vt<NT, TK>(vr, sv[B ^ 1], lane);
    __syncthreads();
  };
  for (int it = 0; it < n_tiles; it += 2) {
    step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < n_tiles) step(std::integral_constant<int, 1>{}, it + 1);
  }

  const float lt = st.l + wave_xor32(st.l);
  if (!row_valid) return;  // only the group's real rows are merged
  const size_t pidx = (((size_t)b * a.Hkv + kvh) * a.n_splits + split) * 32 + l32;
  if (hh == 0) a.part_ml[pidx] = make_float2(st.m, lt);
  float* po = a.part_o + pidx * kD;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      floatx4 w = {st.o[d][4 * j + 0], st.o[d][4 * j + 1], st.o[d][4 * j + 2], st.o[d][4 * j + 3]};
      *reinterpret_cast<floatx4*>(po + 32 * d + 8 * j + 4 * hh) = w;
    }
}

// Merge the per-split partials of one (sequence, KV head, row) with their
// log-sum-exp weights.
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnArgs a) {
  const int lane = threadIdx.x;
  const int row = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int head_local = row / a.Lq;
  const int tq = row - head_local * a.Lq;
  const int hq = kvh * a.G + head_local;
  const size_t base = (((size_t)b * a.Hkv + kvh) * a.n_splits) * 32 + row;
  float mmax = -INFINITY;
  for (int s = 0; s < a.n_splits; ++s) mmax = fmaxf(mmax, a.part_ml[base + (size_t)s * 32].x);
  const float muse = mmax == -INFINITY ? 0.f : mmax;
  float lsum = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s = 0; s < a.n_splits; ++s) {
    const float2 ml = a.part_ml[base + (size_t)s * 32];
    const float w = fast_exp2(ml.x - muse);
    lsum += w * ml.y;
    const float* po = a.part_o + (base + (size_t)s * 32) * kD + 2 * lane;
    o0 += w * po[0];
    o1 += w * po[1];
  }
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  const size_t width = (size_t)a.Hq * kD;
  bf16* orow = a.o + ((size_t)b * a.Lq + tq) * width * (a.o_split ? 2 : 1) + (size_t)hq * kD;
  const float h0 = o0 * inv, h1 = o1 * inv;
  const unsigned int hi = pack_bf16x2(h0, h1);
  *reinterpret_cast<unsigned int*>(orow + 2 * lane) = hi;
  if (a.o_split)
    *reinterpret_cast<unsigned int*>(orow + width + 2 * lane) =
        pack_bf16x2(h0 - lo_bf16(hi), h1 - hi_bf16(hi));
}

}  // namespace

hipError_t launch_attn_prefill_bf16(const AttnArgs& a, hipStream_t stream) {
  dim3 grid(a.Hkv * a.n_hsub, a.B, a.n_qtiles);
  attn_prefill_kernel<<<grid, kPrefillNT, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_attn_decode_bf16(const AttnArgs& a, hipStream_t stream) {
  dim3 grid(a.n_splits, a.Hkv, a.B);
  attn_decode_kernel<<<grid, kDecodeNT, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid2(a.G * a.Lq, a.Hkv, a.B);
  attn_combine_kernel<<<grid2, 64, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace gqa
