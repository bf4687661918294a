// Grouped causal attention on the bf16 matrix cores of gfx950, head_dim 64,
// 128 or 256 (the template parameter KD).
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
// transposed, S^T = K Q^T (keys are MFMA rows, queries MFMA columns), so a
// lane holds whole queries and the rescale factor is one scalar per lane and
// query.  O^T = V^T P^T then takes P^T straight from the score registers;
// the V^T operand is read from V (stored as in memory) with transposing LDS
// reads, keys in the order the score registers hold them.  The decode
// kernels use 32x32x16 products (lane l holds query l % 32 and half of each
// 32-key block: one exchange with lane l ^ 32 per row max and sum), the
// prefill kernel 16x16x32 ones (two 16-query blocks per wave; see below).
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
//            each K/V tile is staged in LDS once per workgroup: once per KV
//            group for groups of up to 4 query heads, twice for 8.
//   decode : one wave per (sequence, KV head, key split); its 32 rows are the
//            group's query heads (x the few new tokens).  Partial (max, sum,
//            unnormalised output) per split are merged by a second kernel.
#include <type_traits>

#include "common.h"
#include "attn_tiles.h"
#include "kernels.h"

namespace gqa {
namespace {

constexpr float kLazyRescale = 8.0f;  // log2 of the growth allowed before rescaling

// Running state of one wave: 32 query rows, lane = row (l % 32).
template <int KD>
struct RowState {
  floatx16 o[Geo<KD>::NB];  // O^T: value feature 32*db + 8*(r/4) + 4*(l/32) + r%4
  float m;                  // running max (log2 units, scaled scores)
  float l;                  // running sum, this lane-half's keys only
};

template <int KD>
__device__ __forceinline__ void init_state(RowState<KD>& st) {
#pragma unroll
  for (int d = 0; d < Geo<KD>::NB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[d][r] = 0.f;
  st.m = -INFINITY;
  st.l = 0.f;
}

// One key tile: scores, online softmax, PV.  `kend_row` = one past the last
// key this lane's query may see; `masked` (wave-uniform) = some key of the
// tile may be past it for some row of the wave.  `loads` issues the JW K
// (loads.k(j)) and JW V (loads.v(j)) loads of the next tile, kPer after each
// of the first QK MFMAs.
//
// LDS reads are issued a whole phase ahead of their MFMAs: all K fragments of
// the tile before the QK product, all V^T fragments (into the same registers)
// while the QK MFMAs drain and the softmax runs.
template <int KD, int TK, int JW, typename Loads>
__device__ __forceinline__ void attend_tile(RowState<KD>& st, const u32x4 (&qf)[Geo<KD>::NC],
                                            const lds_u32x4* sk, const lds_u32x4* sv,
                                            const LaneOffsets<KD>& lo, int key0, int kend_row,
                                            bool masked, float c_log2, int hh, const Loads& loads) {
  using G = Geo<KD>;
  constexpr int KB = TK / 32;
  constexpr int NF = KB * G::NC;  // K fragments per tile = V^T fragments per tile
  static_assert(NF == TK / 16 * G::NB, "as many V^T as K fragments");
  constexpr int kPer = (2 * JW + NF - 1) / NF;  // loads per leading QK MFMA
  u32x4 fr[NF];
#pragma unroll
  for (int m = 0; m < NF; ++m) fr[m] = sk[(m / G::NC) * 32 * G::NCH + lo.k[m % G::NC]];
  __builtin_amdgcn_sched_barrier(0);
  floatx16 s[KB];
  // the KB accumulation chains are interleaved
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    const int kb = i % KB, c = i / KB, m = kb * G::NC + c;
    const floatx16 z = {};
    s[kb] = mfma32x32x16(fr[m], qf[c], c == 0 ? z : s[kb]);
    if (i * kPer < 2 * JW) {
      // all of the next tile's loads go out during the first MFMAs, so
      // they have the whole tile to land before the closing barrier
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int idx = i * kPer + q;
        if (idx < JW) loads.k(idx);
        else if (idx < 2 * JW) loads.v(idx - JW);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int g = 0; g < TK / 16; ++g) {
    lds_cchar* vg = reinterpret_cast<lds_cchar*>(sv) + g * 16 * G::RB;
#pragma unroll
    for (int d = 0; d < G::NB; ++d) {
      const u32x2 k0 = lds_read_tr16(vg + lo.v[d]);
      const u32x2 k1 = lds_read_tr16(vg + lo.v[d] + 8 * G::RB);
      fr[g * G::NB + d] = u32x4{k0.x, k0.y, k1.x, k1.y};
    }
  }
  __builtin_amdgcn_sched_barrier(0);
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
  mx = max_xor32(mx);
  const float mt = mx * c_log2;  // -inf stays -inf (c_log2 > 0)
  if (__builtin_amdgcn_ballot_w64(mt > st.m + kLazyRescale)) {
    const float mn = fmaxf(st.m, mt);
    const float alpha = mn == -INFINITY ? 1.0f : fast_exp2(st.m - mn);
#pragma unroll
    for (int d = 0; d < G::NB; ++d)
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
    for (int d = 0; d < G::NB; ++d) st.o[d] = mfma32x32x16(fr[g * G::NB + d], pf, st.o[d]);
  }
}

__device__ __forceinline__ int kv_len_of(const AttnArgs& a, int b) {
  int n = (a.kv_base ? a.kv_base[b] : 0) + a.kv_add;
  return n < 0 ? 0 : (n > a.cap ? a.cap : n);
}

template <int KD>
__device__ __forceinline__ void load_q(u32x4 (&qf)[Geo<KD>::NC], const bf16* qrow, bool valid,
                                       int hh) {
#pragma unroll
  for (int c = 0; c < Geo<KD>::NC; ++c) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (valid) v = ld16(qrow + 16 * c + 8 * hh);
    qf[c] = v;
  }
}

// Four consecutive output features as bf16 (or, with `f16`, as fp16); with
// `split` also the rounding residual (value - bf16(value)) as bf16, `width`
// elements further on.
__device__ __forceinline__ void store_o4(bf16* p, size_t width, const float (&v)[4], int split,
                                        int f16) {
  u32x2 w;
  if (f16) {
    w.x = pack_f16x2(v[0], v[1]);
    w.y = pack_f16x2(v[2], v[3]);
    st8(p, w);
    return;
  }
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

// ---- prefill on 16x16x32 MFMAs ----
// A wave's 32 query rows are two 16-row blocks (qb): lane l holds queries
// l16 and 16 + l16 (l16 = l % 16) and, of each 16-key block of the scores
// S^T = K Q^T, the keys 4 q + 0..3 (q = l / 16).  The row max and sum of a
// query then span the four lanes l16 + 16 q (two exchanges, for the max only
// when the wave rescales), the rescale
// factor is one scalar per lane and query block, and the P^T operand of
// O^T = V^T P^T comes straight from the score registers: for a 32-key step,
// lane l holds keys 4 q + 0..3 and 16 + 4 q + 0..3 of the query, which is
// an MFMA K-group of eight.  The V^T operand is read with transposing LDS
// reads in that key order.  The matrix cores do the same work per cycle as
// with 32x32x16 products, for less power (the board's power limit sets the
// clock): 1-3% faster at 2x16384 than the 32x32x16 version of this kernel.
template <int KD>
struct RowState16 {
  floatx4 o[KD / 16][2];  // O^T: feature 16 db + 4 q + r, query 16 qb + l16
  float nm[2];            // minus the running max per query block (log2 units, scaled
                          // scores), kept negated: it enters every exp offset as is
  float l[2];             // running sum, this lane's keys only
};

template <int KD>
__device__ __forceinline__ void init_state16(RowState16<KD>& st) {
#pragma unroll
  for (int d = 0; d < KD / 16; ++d)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 4; ++r) st.o[d][qb][r] = 0.f;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    st.nm[qb] = INFINITY;
    st.l[qb] = 0.f;
  }
}

// Per-lane LDS offsets of the 16x16 fragments, as one base per operand: the
// swizzles XOR the chunk with a lane term, so the offset of step s (K) or
// block db (V) is the base XOR a constant (two registers instead of one per
// step and block, for one VALU op per read).
template <int KD>
struct LaneOffsets16 {
  int k;  // K fragment of feature step 0 (bytes): key row l16, chunk q; step s: k ^ (64 s)
  int v;  // V^T fragment of feature block 0 (bytes), first read, key group 0; block db: v ^ (32 db)
  __device__ __forceinline__ int kofs(int s) const { return k ^ (64 * s); }
  __device__ __forceinline__ int vofs(int db) const { return v ^ (32 * db); }
};

// K fragment (A operand of a 16-key x 16-query score block, 32 features per
// step): lane l reads key row l16, features 32 s + 8 q + 0..7.  V^T fragment
// (A operand of O^T, 16 features x 32 keys): lane l = 16 q + i must hold
// feature 16 db + i of keys 4 q + 0..3 and 16 + 4 q + 0..3.  A transposing
// read in which lane j of group q points at row (key) 4 q + j / 4,
// features 16 db + 4 (j % 4) + 0..3 hands lane i feature 16 db + i of the 4
// keys 4 q + e; the second read is the same, 16 rows further on.  Both
// swizzles depend on the row modulo 16 (K) or 8 (V) only, so key block and
// key step offsets are whole rows.
//
// K: chunk 4 s + q of row l16 sits at slot (4 s + q) ^ kswz(l16), whose
// bits 2 and up are s ^ (kswz / 4) (kswz < 16 for 256-byte rows, < 8 for
// 128-byte ones; 512-byte rows keep the row's chunk bits 4 and up): byte
// offset = base ^ 64 s.  V: chunk 2 db + c of row r sits at (2 db + c) ^
// vswz16(r) = 2 (db ^ vswz16 / 2) + c: byte offset = base ^ 32 db.
template <int KD>
__device__ __forceinline__ void lane_offsets16(LaneOffsets16<KD>& o, int lane) {
  using G = Geo<KD>;
  const int l16 = lane & 15, q = lane >> 4;
  o.k = G::kslot(l16, q) * 16;
  const int row = 4 * q + (l16 >> 2);
  const int feat = 4 * (l16 & 3);
  o.v = G::vslot16(row, feat >> 3) * 16 + (feat & 7) * 2;
}

// Both query blocks' Q fragments (B operands): feature step s of block qb
// is features 32 s + 8 q + 0..7 of query row 16 qb + l16.
template <int KD>
__device__ __forceinline__ void load_q16(u32x4 (&qf)[2][KD / 32], const bf16* q0, const bf16* q1,
                                         bool v0, bool v1, int q) {
#pragma unroll
  for (int s = 0; s < KD / 32; ++s) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    qf[0][s] = v0 ? ld16(q0 + 32 * s + 8 * q) : z;
    qf[1][s] = v1 ? ld16(q1 + 32 * s + 8 * q) : z;
  }
}

// One key tile on 16x16x32 products: scores, online softmax, PV.
// `kend0` = one past the last key the lane's query of block 0 may see, and
// `kstep1` what block 1's query (16 rows further on) sees beyond it: 16
// keys with the causal mask, none without;
// `masked` (wave-uniform) = some key of the tile may be past it for some
// row of the wave.  `loads` issues the JW K and JW V loads of the next tile
// right after this tile's K fragment reads.
template <int KD, int TK, int JW, typename Loads>
__device__ __forceinline__ void attend_tile16(RowState16<KD>& st, const u32x4 (&qf)[2][KD / 32],
                                              const lds_u32x4* sk, const lds_u32x4* sv,
                                              const LaneOffsets16<KD>& lo, int key0,
                                              int kend0, int kstep1, bool masked, float c_log2,
                                              int q, const Loads& loads) {
  using G = Geo<KD>;
  constexpr int NS = KD / 32;   // feature steps of the QK product
  constexpr int ND = KD / 16;   // feature blocks of O^T
  constexpr int KB = TK / 16;   // key blocks
  constexpr int KS = TK / 32;   // key steps of the PV product
  constexpr int NF = KB * NS;   // K fragments per tile = V^T fragments per tile
  static_assert(NF == KS * ND, "as many V^T as K fragments");
  constexpr int NQK = 2 * NF;   // QK MFMAs per tile
  u32x4 fr[NF];
  // K fragments in the order the products use them: feature step major
#pragma unroll
  for (int m = 0; m < NF; ++m) {
    const int s = m / KB, kb = m % KB;
    fr[m] = *reinterpret_cast<const lds_u32x4*>(reinterpret_cast<lds_cchar*>(sk) + 16 * kb * G::RB +
                                                 lo.kofs(s));
  }
  // the next tile's loads, all at once (interleaving them with the
  // products was slower)
#pragma unroll
  for (int j = 0; j < JW; ++j) loads.k(j);
#pragma unroll
  for (int j = 0; j < JW; ++j) loads.v(j);
  __builtin_amdgcn_sched_barrier(0);
  // The products run at a raised wave priority, so that a wave whose
  // MFMAs are ready issues them ahead of the softmax work of the other
  // waves on its SIMD, which then fills the matrix core's cycles.
  __builtin_amdgcn_s_setprio(1);
  floatx4 sc[KB][2];
  // 2 KB independent accumulation chains, interleaved
#pragma unroll
  for (int i = 0; i < NQK; ++i) {
    const int m = i / 2, qb = i % 2, s = m / KB, kb = m % KB;
    const floatx4 z = {};
    sc[kb][qb] = mfma16x16x32(fr[m], qf[qb][s], s == 0 ? z : sc[kb][qb]);
  }
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
  // V^T fragments of key step ks, feature blocks db of one half of the
  // head (the register budget of three waves per SIMD holds half of them
  // at a time): the first half is read now and lands while the softmax
  // runs, the second after the first half's products
  constexpr int NH = ND / 2;
  auto read_v = [&](int ks, int half, u32x4(&vf)[NH]) {
    lds_cchar* vg = reinterpret_cast<lds_cchar*>(sv) + 32 * ks * G::RB;
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const int vo = lo.vofs(half * NH + j);
      const u32x2 k0 = lds_read_tr16(vg + vo);
      const u32x2 k1 = lds_read_tr16(vg + vo + 16 * G::RB);
      vf[j] = u32x4{k0.x, k0.y, k1.x, k1.y};
    }
  };
  u32x4 vf[NH];
  read_v(0, 0, vf);
  __builtin_amdgcn_sched_barrier(0);
  if (masked) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key0 + 16 * kb + 4 * q + r >= kend0 + kstep1 * qb) sc[kb][qb][r] = -INFINITY;
  }
  // this lane's share of each row max (a row spans lanes l16 + 16 q)
  float mx[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    mx[qb] = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx[qb] = fmaxf(mx[qb], sc[kb][qb][r]);
  }
  // A row max passes its threshold exactly when one of its four shares
  // does (c_log2 > 0), so the wave tests the shares and exchanges them only
  // when it rescales.  An unset max (-inf) takes any finite share.
  if (__builtin_amdgcn_ballot_w64(__builtin_fmaf(mx[0], c_log2, st.nm[0]) > kLazyRescale ||
                                  __builtin_fmaf(mx[1], c_log2, st.nm[1]) > kLazyRescale)) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float mt = max_xor32(max_xor16(mx[qb])) * c_log2;
      const float nmn = fminf(st.nm[qb], -mt);  // minus the new max
      const float alpha = nmn == INFINITY ? 1.0f : fast_exp2(nmn - st.nm[qb]);
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int r = 0; r < 4; ++r) st.o[d][qb][r] *= alpha;
      st.l[qb] *= alpha;
      st.nm[qb] = nmn;
    }
  }
  // P^T operands of both query blocks (and the row sums of their bf16
  // values), then the products, half of the feature blocks at a time.  The
  // running max is finite here: key 0 is visible to every row (causal or
  // not), so the first tile sets it.
  u32x4 pf[KS][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        p[e] = fast_exp2(__builtin_fmaf(sc[2 * ks + e / 4][qb][e % 4], c_log2, st.nm[qb]));
      u32x4 f;
      f.x = pack_bf16x2(p[0], p[1]);
      f.y = pack_bf16x2(p[2], p[3]);
      f.z = pack_bf16x2(p[4], p[5]);
      f.w = pack_bf16x2(p[6], p[7]);
      st.l[qb] = sum_bf16x2(f.x, st.l[qb]);
      st.l[qb] = sum_bf16x2(f.y, st.l[qb]);
      st.l[qb] = sum_bf16x2(f.z, st.l[qb]);
      st.l[qb] = sum_bf16x2(f.w, st.l[qb]);
      pf[ks][qb] = f;
    }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (ks + half > 0) {
        __builtin_amdgcn_sched_barrier(0);
        read_v(ks, half, vf);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (ks + half == 0) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int j = 0; j < NH; ++j)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          st.o[half * NH + j][qb] = mfma16x16x32(vf[j], pf[ks][qb], st.o[half * NH + j][qb]);
    }
  __builtin_amdgcn_s_setprio(0);
}

// Prefill tile sizes and occupancy: head_dim 128 takes 32-key tiles, whose
// registers (168, with the V^T fragments read half a head at a time) and LDS
// (32 KB) let three workgroups share a CU, so three waves per SIMD hide each
// other's softmax and LDS latency (64-key tiles need two waves per SIMD and
// were slower); head_dim 64 keeps 64-key tiles (three waves per SIMD
// already); head_dim 256 takes 32 keys at one wave per SIMD (its fragments
// would not fit otherwise).
template <int KD>
struct PrefillCfg {
  static constexpr int TK = KD == 64 ? 64 : 32;
  static constexpr int NT = 256;
  static constexpr int MIN_BLOCKS = KD == 256 ? 1 : KD == 128 ? 3 : 2;
};

template <int KD>
__global__ __launch_bounds__(PrefillCfg<KD>::NT, PrefillCfg<KD>::MIN_BLOCKS) void attn_prefill_kernel(
    AttnArgs a) {
  using G = Geo<KD>;
  constexpr int TK = PrefillCfg<KD>::TK, NT = PrefillCfg<KD>::NT;
  using Plan = TileLoads<KD, NT, TK, true>;
  // Separate arrays per buffer: the compiler then knows that the loads into
  // one buffer cannot touch the other, and does not make reads of the
  // current tile wait for the loads of the next.
  __shared__ u32x4 sk0[TK * G::NCH], sk1[TK * G::NCH];
  __shared__ u32x4 sv0[TK * G::NCH], sv1[TK * G::NCH];
  poison_lds(sk0, sk1, sv0, sv1);
  lds_u32x4* const sk[2] = {(lds_u32x4*)sk0, (lds_u32x4*)sk1};
  lds_u32x4* const sv[2] = {(lds_u32x4*)sv0, (lds_u32x4*)sv1};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int l16 = lane & 15, q = lane >> 4;
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
  // The lane's two query rows: tq and tq + 16.  Masking needs only the
  // first row's key end: the second one's is 16 keys later.  The masked
  // tiles are those that reach past kmin_w, where every row of the wave
  // that exists sees all keys before it; rows past the end of the
  // sequence take part in the products but are never stored.
  const int tq = t0 + l16;
  const int kend0 = a.causal ? off + tq + 1 : kvl;

  u32x4 qf[2][KD / 32];
  {
    const bf16* qhead = a.q + ((size_t)b * a.Hq + hq) * a.Lq * KD;
    const bool v0 = tq < a.Lq, v1 = tq + 16 < a.Lq;
    load_q16<KD>(qf, qhead + (size_t)(v0 ? tq : 0) * KD, qhead + (size_t)(v1 ? tq + 16 : 0) * KD,
                 v0, v1, q);
  }

  const size_t kv_base = ((size_t)b * a.Hkv + kvh) * a.cap * KD;
  const bf16* kb = a.k + kv_base;
  const bf16* vb = a.v + kv_base;
  // descriptors of the tile starting at key k0 (keys k0 .. kvl - 1 valid)
  auto rk_at = [&](int k0) { return make_rsrc(kb + (size_t)k0 * KD, (long long)(kvl - k0) * G::RB); };
  auto rv_at = [&](int k0) { return make_rsrc(vb + (size_t)k0 * KD, (long long)(kvl - k0) * G::RB); };
  LaneOffsets16<KD> lo;
  lane_offsets16<KD>(lo, lane);

  RowState16<KD> st;
  init_state16<KD>(st);
  Plan plan;
  plan.init(wave, lane);
  const TileDst<KD, NT, TK, true> first{&plan, rk_at(0), rv_at(0), sk[0], sv[0], n_tiles > 0};
  first.all();
  __syncthreads();
  // two tiles per trip, so each buffer's LDS addresses are constants
  auto step = [&](auto bufc, int it) {
    constexpr int B = decltype(bufc)::value;
    // the next tile goes to the other buffer, last read before the barrier
    // that ended the previous trip
    const TileDst<KD, NT, TK, true> next{&plan, rk_at((it + 1) * TK), rv_at((it + 1) * TK),
                                         sk[B ^ 1], sv[B ^ 1], it + 1 < n_tiles};
    const int key0 = it * TK;
    if (key0 < key_end_w) {
      const bool masked = key0 + TK > kmin_w;
      attend_tile16<KD, TK, Plan::JW>(st, qf, sk[B], sv[B], lo, key0, kend0, a.causal ? 16 : 0,
                                      masked, a.scale_log2, q, next);
    } else {
      next.all();  // the other waves still need this wave's share
    }
    __syncthreads();
  };
  for (int it = 0; it < n_tiles; it += 2) {
    step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < n_tiles) step(std::integral_constant<int, 1>{}, it + 1);
  }

  const size_t width = (size_t)a.Hq * KD;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = sum_xor32(sum_xor16(st.l[qb]));
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int t = tq + 16 * qb;
    if (t >= a.Lq) continue;
    if (a.lse && q == 0) {
      // log sum_j exp(s_j * scale) = (m + log2(l)) * ln 2, m in log2 units
      a.lse[((size_t)b * a.Hq + hq) * a.Lq + t] =
          lt > 0.f ? (log2f(lt) - st.nm[qb]) * 0.69314718055994531f : -INFINITY;
    }
    bf16* orow = a.o + ((size_t)b * a.Lq + t) * width * (a.o_split ? 2 : 1) + (size_t)hq * KD;
#pragma unroll
    for (int d = 0; d < KD / 16; ++d) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = st.o[d][qb][i] * inv;
      store_o4(orow + 16 * d + 4 * q, width, v, a.o_split, a.o_f16);
    }
  }
}

constexpr int kDecodeTK = 32;
constexpr int kDecodeNT = 64;

template <int KD>
__global__ __launch_bounds__(kDecodeNT) void attn_decode_kernel(AttnArgs a) {
  using G = Geo<KD>;
  constexpr int TK = kDecodeTK, NT = kDecodeNT;
  using Plan = TileLoads<KD, NT, TK>;
  __shared__ u32x4 sk0[TK * G::NCH], sk1[TK * G::NCH];
  __shared__ u32x4 sv0[TK * G::NCH], sv1[TK * G::NCH];
  poison_lds(sk0, sk1, sv0, sv1);
  lds_u32x4* const sk[2] = {(lds_u32x4*)sk0, (lds_u32x4*)sk1};
  lds_u32x4* const sv[2] = {(lds_u32x4*)sv0, (lds_u32x4*)sv1};

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

  u32x4 qf[G::NC];
  load_q<KD>(qf, a.q + (((size_t)b * a.Hq + hq) * a.Lq + tq) * KD, row_valid, hh);

  const size_t kv_base = ((size_t)b * a.Hkv + kvh) * a.cap * KD;
  const bf16* kb = a.k + kv_base;
  const bf16* vb = a.v + kv_base;
  // descriptors of the tile starting at key k0 (keys k0 .. ke - 1 valid)
  auto rk_at = [&](int k0) { return make_rsrc(kb + (size_t)k0 * KD, (long long)(ke - k0) * G::RB); };
  auto rv_at = [&](int k0) { return make_rsrc(vb + (size_t)k0 * KD, (long long)(ke - k0) * G::RB); };
  LaneOffsets<KD> lo;
  lane_offsets<KD>(lo, lane);

  RowState<KD> st;
  init_state<KD>(st);
  Plan plan;
  plan.init(0, lane);
  // With `rotate` the wave walks its chunk's tiles starting at tile
  // 13 * (wave index) mod n_tiles, wrapping round, so that the waves resident
  // at one time do not all read the same offset of their chunks.
  const int rot = a.rotate && n_tiles > 0
                      ? (int)(((blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * 13u %
                              (unsigned)n_tiles)
                      : 0;
  auto key_of = [&](int it) {
    int j = it + rot;
    if (j >= n_tiles) j -= n_tiles;
    return ks + j * TK;
  };
  const TileDst<KD, NT, TK> first{&plan, rk_at(key_of(0)), rv_at(key_of(0)), sk[0], sv[0],
                                  n_tiles > 0};
  first.all();
  __syncthreads();
  auto step = [&](auto bufc, int it) {
    constexpr int B = decltype(bufc)::value;
    const int key0 = key_of(it);
    const int key1 = key_of(it + 1 < n_tiles ? it + 1 : it);
    const TileDst<KD, NT, TK> next{&plan, rk_at(key1), rv_at(key1), sk[B ^ 1],
                                   sv[B ^ 1], it + 1 < n_tiles};
    const bool masked = key0 + TK > kmin;
    attend_tile<KD, TK, Plan::JW>(st, qf, sk[B], sv[B], lo, key0, kend_row, masked, a.scale_log2,
                                  hh, next);
    __syncthreads();
  };
  for (int it = 0; it < n_tiles; it += 2) {
    step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < n_tiles) step(std::integral_constant<int, 1>{}, it + 1);
  }

  const float lt = sum_xor32(st.l);
  if (!row_valid) return;  // only the group's real rows are kept and merged
  const size_t pidx = (((size_t)b * a.Hkv + kvh) * a.n_splits + split) * rows + l32;
  if (hh == 0) a.part_ml[pidx] = make_float2(st.m, lt);
  float* po = a.part_o + pidx * KD;
#pragma unroll
  for (int d = 0; d < G::NB; ++d)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      floatx4 w = {st.o[d][4 * j + 0], st.o[d][4 * j + 1], st.o[d][4 * j + 2], st.o[d][4 * j + 3]};
      *reinterpret_cast<floatx4*>(po + 32 * d + 8 * j + 4 * hh) = w;
    }
}

// FP8 (E4M3) caches: the decode kernel above with K and V tiles staged
// through registers.  A tile's codes (KD bytes per key) arrive by 16-byte
// register loads issued during the first QK MFMAs of the previous tile;
// after that tile the codes are widened to bf16 (exact: every E4M3 value is
// a bf16 value) and written into the other LDS buffer in the layout the
// DMA path produces, so the same attend_tile runs on them.  The scales are
// applied outside the products: the K scale is part of the score scale,
// the V scale is applied when the splits are merged.
template <int KD, int TK>
struct Fp8TileLoads {
  static constexpr int P = KD / 16;     // 16-byte pieces of one key's codes
  static constexpr int RPL = 64 / P;    // keys per load instruction
  static constexpr int NI = TK / RPL;   // load instructions per tile and operand
  static_assert(NI * RPL == TK, "a tile splits into whole load instructions");
  __amdgpu_buffer_rsrc_t rk, rv;        // the tile's codes, from its first key
  unsigned off[NI];                     // per-lane byte offsets within a tile
  bool live;
  mutable u32x4 kc[NI], vc[NI];         // codes in flight
  __device__ __forceinline__ void k(int j) const {
    if (live) kc[j] = buf_ld16(rk, off[j]);
  }
  __device__ __forceinline__ void v(int j) const {
    if (live) vc[j] = buf_ld16(rv, off[j]);
  }
  __device__ __forceinline__ void all() const {
#pragma unroll
    for (int j = 0; j < NI; ++j) k(j);
#pragma unroll
    for (int j = 0; j < NI; ++j) v(j);
  }
};

// 8 E4M3 codes (two dwords) -> 8 bf16 (one 16-byte LDS chunk)
GQA_DEV unsigned widen_e4m3_lo(unsigned w) {  // codes in bytes 0, 1
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
GQA_DEV unsigned widen_e4m3_hi(unsigned w) {  // codes in bytes 2, 3
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}
GQA_DEV u32x4 widen_e4m3(unsigned lo, unsigned hi) {
  return u32x4{widen_e4m3_lo(lo), widen_e4m3_hi(lo), widen_e4m3_lo(hi), widen_e4m3_hi(hi)};
}

template <int KD>
__global__ __launch_bounds__(kDecodeNT) void attn_decode_fp8_kernel(AttnArgs a) {
  using G = Geo<KD>;
  constexpr int TK = kDecodeTK, NT = kDecodeNT;
  using L8 = Fp8TileLoads<KD, TK>;
  __shared__ u32x4 sk0[TK * G::NCH], sk1[TK * G::NCH];
  __shared__ u32x4 sv0[TK * G::NCH], sv1[TK * G::NCH];
  poison_lds(sk0, sk1, sv0, sv1);
  lds_u32x4* const sk[2] = {(lds_u32x4*)sk0, (lds_u32x4*)sk1};
  lds_u32x4* const sv[2] = {(lds_u32x4*)sv0, (lds_u32x4*)sv1};

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

  u32x4 qf[G::NC];
  load_q<KD>(qf, a.q + (((size_t)b * a.Hq + hq) * a.Lq + tq) * KD, row_valid, hh);

  const size_t kv_base = ((size_t)b * a.Hkv + kvh) * a.cap * KD;  // one byte per element
  const unsigned char* kb = a.k8 + kv_base;
  const unsigned char* vb = a.v8 + kv_base;
  LaneOffsets<KD> lo;
  lane_offsets<KD>(lo, lane);

  // lane -> (key row_in + RPL i, piece p) of a tile: 16 codes, features
  // 16 p .. 16 p + 15 = bf16 chunks 2 p and 2 p + 1
  const int row_in = lane / L8::P, piece = lane % L8::P;
  L8 ld;
#pragma unroll
  for (int i = 0; i < L8::NI; ++i) ld.off[i] = (unsigned)((row_in + L8::RPL * i) * KD + 16 * piece);
  auto aim = [&](int k0, bool live) {  // the loads of the tile starting at key k0
    const long long bytes = live ? (long long)(ke - k0) * KD : 0;
    ld.rk = make_rsrc(kb + (size_t)k0 * KD, bytes);
    ld.rv = make_rsrc(vb + (size_t)k0 * KD, bytes);
    ld.live = live;
  };
  auto widen_into = [&](lds_u32x4* dk, lds_u32x4* dv) {
#pragma unroll
    for (int i = 0; i < L8::NI; ++i) {
      const int row = row_in + L8::RPL * i;
      dk[G::kslot(row, 2 * piece)] = widen_e4m3(ld.kc[i].x, ld.kc[i].y);
      dk[G::kslot(row, 2 * piece + 1)] = widen_e4m3(ld.kc[i].z, ld.kc[i].w);
      dv[G::vslot(row, 2 * piece)] = widen_e4m3(ld.vc[i].x, ld.vc[i].y);
      dv[G::vslot(row, 2 * piece + 1)] = widen_e4m3(ld.vc[i].z, ld.vc[i].w);
    }
  };

  RowState<KD> st;
  init_state<KD>(st);
  aim(ks, n_tiles > 0);
  ld.all();
  widen_into(sk[0], sv[0]);
  __syncthreads();
  auto step = [&](auto bufc, int it) {
    constexpr int B = decltype(bufc)::value;
    const int key0 = ks + it * TK;
    const bool more = it + 1 < n_tiles;
    aim(key0 + TK, more);
    const bool masked = key0 + TK > kmin;
    attend_tile<KD, TK, L8::NI>(st, qf, sk[B], sv[B], lo, key0, kend_row, masked, a.scale_log2,
                                hh, ld);
    if (more) widen_into(sk[B ^ 1], sv[B ^ 1]);
    __syncthreads();
  };
  for (int it = 0; it < n_tiles; it += 2) {
    step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < n_tiles) step(std::integral_constant<int, 1>{}, it + 1);
  }

  const float lt = sum_xor32(st.l);
  if (!row_valid) return;  // only the group's real rows are kept and merged
  const size_t pidx = (((size_t)b * a.Hkv + kvh) * a.n_splits + split) * rows + l32;
  if (hh == 0) a.part_ml[pidx] = make_float2(st.m, lt);
  float* po = a.part_o + pidx * KD;
#pragma unroll
  for (int d = 0; d < G::NB; ++d)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      floatx4 w = {st.o[d][4 * j + 0], st.o[d][4 * j + 1], st.o[d][4 * j + 2], st.o[d][4 * j + 3]};
      *reinterpret_cast<floatx4*>(po + 32 * d + 8 * j + 4 * hh) = w;
    }
}

// Merge of the decode splits: one workgroup per (query row, KV head,
// sequence).  Lane s first holds split s for the maxima and sums.  For the
// outputs the wave is cut into 256 / KD groups of KD / 4 lanes; group g
// adds splits g, g + 256 / KD, ... with one 16-byte load of four features
// per lane and split (several splits' loads in flight at once), and the
// groups' sums are added across lanes at the end.
template <int KD>
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnArgs a) {
  constexpr int LPR = KD / 4;    // lanes per row of KD features
  constexpr int SPL = 64 / LPR;  // splits read per load step
  const int lane = threadIdx.x;
  const int sg = lane / LPR, e4 = lane % LPR;
  const int row = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int head_local = row / a.Lq;
  const int tq = row - head_local * a.Lq;
  const int hq = kvh * a.G + head_local;
  const int ns = a.n_splits;
  const int rows = a.G * a.Lq;  // partial rows per split
  const size_t base = (((size_t)b * a.Hkv + kvh) * ns) * rows + row;
  float mmax = -INFINITY;
  for (int s = lane; s < ns; s += 64) mmax = fmaxf(mmax, a.part_ml[base + (size_t)s * rows].x);
#pragma unroll
  for (int x = 32; x > 0; x >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, x, 64));
  const float muse = mmax == -INFINITY ? 0.f : mmax;
  __shared__ float wsh[64];
  poison_lds(wsh);
  float lsum = 0.f;
  floatx4 o = {0.f, 0.f, 0.f, 0.f};
  const float* po = a.part_o + base * KD + 4 * e4;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    float w = 0.f;
    if (s0 + lane < ns) {
      const float2 ml = a.part_ml[base + (size_t)(s0 + lane) * rows];
      w = fast_exp2(ml.x - muse);
      lsum += w * ml.y;
    }
    __syncthreads();  // the previous chunk's weights are consumed
    wsh[lane] = w;
    __syncthreads();
    const int n = min(64, ns - s0);
#pragma unroll 4
    for (int i = sg; i < n; i += SPL) {
      const float wi = wsh[i];
      const floatx4 v = *reinterpret_cast<const floatx4*>(po + (size_t)(s0 + i) * rows * KD);
      o += wi * v;
    }
  }
#pragma unroll
  for (int x = 32; x > 0; x >>= 1) lsum += __shfl_xor(lsum, x, 64);
#pragma unroll
  for (int x = LPR; x < 64; x <<= 1)
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] += __shfl_xor(o[c], x, 64);
  if (sg != 0) return;
  const float inv = lsum > 0.f ? a.v_scale / lsum : 0.f;
  const size_t width = (size_t)a.Hq * KD;
  bf16* orow = a.o + ((size_t)b * a.Lq + tq) * width * (a.o_split ? 2 : 1) + (size_t)hq * KD;
  const float v[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
  store_o4(orow + 4 * e4, width, v, a.o_split, a.o_f16);
}

template <int KD>
hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream) {
  dim3 grid(a.Hkv * a.n_hsub, a.B, a.n_qtiles);
  attn_prefill_kernel<KD><<<grid, PrefillCfg<KD>::NT, 0, stream>>>(a);
  return hipGetLastError();
}

template <int KD>
hipError_t launch_decode(const AttnArgs& a, hipStream_t stream) {
  dim3 grid(a.n_splits, a.Hkv, a.B);
  if constexpr (KD <= 128) {
    if (a.k8)
      attn_decode_fp8_kernel<KD><<<grid, kDecodeNT, 0, stream>>>(a);
    else
      attn_decode_kernel<KD><<<grid, kDecodeNT, 0, stream>>>(a);
  } else {
    // FP8 caches: head_dim 64 and 128 (the host rejects 256: its staged
    // codes would not fit the registers next to the kernel's own)
    if (a.k8) return hipErrorInvalidValue;
    attn_decode_kernel<KD><<<grid, kDecodeNT, 0, stream>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid2(a.G * a.Lq, a.Hkv, a.B);
  attn_combine_kernel<KD><<<grid2, 64, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_prefill_bf16(const AttnArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch_prefill<64>(a, stream);
    case 128: return launch_prefill<128>(a, stream);
    case 256: return launch_prefill<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_decode_bf16(const AttnArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch_decode<64>(a, stream);
    case 128: return launch_decode<128>(a, stream);
    case 256: return launch_decode<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
