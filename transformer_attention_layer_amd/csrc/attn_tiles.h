// Tile machinery shared by the bf16 matrix-core attention kernels of gfx950
// (forward and backward): the geometry and LDS swizzles of K/V-shaped tiles
// (rows of head_dim bf16 features), their direct global-to-LDS loads, the
// transposing LDS read and the per-lane fragment offsets.
#pragma once

#include "common.h"

namespace gqa {
namespace {

// LDS pointers are kept in the LDS address space from the arrays on, so no
// generic-to-LDS conversion (and its null check) is left for the compiler.
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) const char lds_cchar;
typedef __attribute__((address_space(3))) float lds_float;
typedef __attribute__((address_space(3))) const floatx4 lds_floatx4;

// Geometry of a K or V tile row for head size KD: KD bf16 = NCH 16-byte
// chunks; one 64-lane load instruction (64 x 16 B) fills RPI rows.
template <int KD>
struct Geo {
  static_assert(KD == 64 || KD == 128 || KD == 256, "head_dim 64, 128 or 256");
  static constexpr int NCH = KD / 8;
  static constexpr int RB = KD * 2;     // bytes per row
  static constexpr int RPI = 64 / NCH;  // rows per load instruction
  static constexpr int NB = KD / 32;    // 32-feature blocks of O^T
  static constexpr int NC = KD / 16;    // 16-feature steps of the QK product

  // K tile: a fragment read has 16 lanes on 16 consecutive rows at one chunk;
  // gfx950's LDS serves them over 64 banks (256 B).  Chunk c of row r sits at
  // slot c ^ kswz(r): 128-byte rows pair up in a bank window, so the 8 even
  // and the 8 odd rows each take 8 slots; 256- and 512-byte rows start on the
  // same bank, so 16 rows take 16 slots (the XOR keeps a 512-byte row's
  // chunks in their 256-byte half).
  __device__ static __forceinline__ int kswz(int row) {
    return KD == 64 ? ((row >> 1) & 7) : (row & 15);
  }
  // V tile: one transposing read by 32 lanes touches 4 consecutive rows x 4
  // chunks; chunk c of row r sits at slot c ^ vswz(r) so that the 16 chunks
  // land on 16 distinct bank groups (rows r and r + 2 share a bank window
  // when rows are 128 bytes).
  __device__ static __forceinline__ int vswz(int row) {
    return KD == 64 ? (((row >> 1) & 1) << 2) : ((row & 3) << 2);
  }
  // V tile read by the 16x16 kernels: a transposing read by 32 lanes touches
  // 8 consecutive rows x 2 aligned chunks; chunk c of row r sits at slot
  // c ^ vswz16(r), an even term, so the 16 chunks land on 16 distinct bank
  // groups (with 128-byte rows, the 4 rows of each parity take 4 terms).
  __device__ static __forceinline__ int vswz16(int row) {
    return KD == 64 ? 2 * ((row >> 1) & 3) : 2 * (row & 7);
  }
  __device__ static __forceinline__ int vslot16(int row, int chunk) {
    return row * NCH + (chunk ^ vswz16(row));
  }
  // Tiles read both as MFMA rows and transposed (the backward kernels): a
  // row fragment read wants the 16 rows of a 16-row run on 16 distinct
  // 16-byte bank slots, a transposing read by 32 lanes wants 4 aligned rows
  // x 4 aligned chunks on 16 distinct slots.  With 256-byte rows, slot =
  // chunk ^ (4 (r % 4) + (r / 4) % 4) does both (a bijection over 16 rows
  // whose bits 2-3 differ across 4 aligned rows); with 128-byte rows two
  // rows share a bank window and the same holds for
  // chunk ^ (4 ((r / 2) % 2) + (r / 4) % 4) within each row parity.
  __device__ static __forceinline__ int bswz(int row) {
    static_assert(KD == 64 || KD == 128, "both-way tiles: head_dim 64 or 128");
    return KD == 64 ? ((((row >> 1) & 1) << 2) | ((row >> 2) & 3))
                    : (((row & 3) << 2) | ((row >> 2) & 3));
  }
  __device__ static __forceinline__ int bslot(int row, int chunk) {
    return row * NCH + (chunk ^ bswz(row));
  }
  __device__ static __forceinline__ int kslot(int row, int chunk) {
    return row * NCH + (chunk ^ kswz(row));
  }
  __device__ static __forceinline__ int vslot(int row, int chunk) {
    return row * NCH + (chunk ^ vswz(row));
  }
};

// K or V tile straight into LDS (buffer_load ... lds): one instruction fills
// 64 consecutive slots = RPI key rows; lane i writes slot i, so it loads the
// chunk that the tile's swizzle puts there.  Keys past the descriptor's
// range read as 0.  A wave issues JW instructions per tile and per operand;
// the per-lane byte offsets within a tile are fixed.  Each tile gets
// descriptors based at its first key, so that the hardware range check
// (which covers the per-lane offset only, not a scalar offset) still
// zero-fills the keys past the end.
// V16: the V tile takes the swizzle of the 16x16 kernels.
template <int KD, int NT, int TK, bool V16 = false>
struct TileLoads {
  using G = Geo<KD>;
  static constexpr int JW = TK / G::RPI / (NT / 64);
  static_assert(JW >= 1 && JW * G::RPI * (NT / 64) == TK, "tile rows split evenly over waves");
  unsigned ko[JW], vo[JW];  // per-lane byte offsets of instruction j
  int slot0;                // first LDS slot of this wave's rows

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < JW; ++j) {
      const int row = (wave * JW + j) * G::RPI + lane / G::NCH;
      const int slot = lane % G::NCH;
      ko[j] = (unsigned)(row * G::RB + ((slot ^ G::kswz(row)) << 4));
      vo[j] = (unsigned)(row * G::RB + ((slot ^ (V16 ? G::vswz16(row) : G::vswz(row))) << 4));
    }
    slot0 = wave * JW * 64;
  }
};

// The loads of one tile into one buffer; rk / rv start at the tile's first
// key and end at the last valid key.
template <int KD, int NT, int TK, bool V16 = false>
struct TileDst {
  const TileLoads<KD, NT, TK, V16>* plan;
  __amdgpu_buffer_rsrc_t rk, rv;
  lds_u32x4* sk;
  lds_u32x4* sv;
  bool live;  // the tile exists
  __device__ __forceinline__ void k(int j) const {
    if (live)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, sk + plan->slot0 + 64 * j, 16, plan->ko[j], 0, 0,
                                               0);
  }
  __device__ __forceinline__ void v(int j) const {
    if (live)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, sv + plan->slot0 + 64 * j, 16, plan->vo[j], 0, 0,
                                               0);
  }
  __device__ __forceinline__ void all() const {
#pragma unroll
    for (int j = 0; j < TileLoads<KD, NT, TK, V16>::JW; ++j) k(j);
#pragma unroll
    for (int j = 0; j < TileLoads<KD, NT, TK, V16>::JW; ++j) v(j);
  }
};

typedef short shortx4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 at a byte address of LDS.  Within each 16-lane group,
// lane i receives element i % 4 of the 8 bytes that lane 4e + i / 4 of the
// group points at, as its element e (a 16 x 4 block of 16-bit values comes
// back transposed).
GQA_DEV u32x2 lds_read_tr16(lds_cchar* p) {
  const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Per-lane LDS offsets of the MFMA fragments; the same for every tile and
// buffer.
template <int KD>
struct LaneOffsets {
  int k[Geo<KD>::NC];  // K fragment of feature step c (16-byte slots): key row l32
  int v[Geo<KD>::NB];  // V^T fragment of feature block d (bytes), first read of key group 0
};

// V^T fragment (A operand of O^T = V^T P^T) for 32 features x 16 keys: lane
// l = 16 G + i must hold feature l % 32 and, in MFMA K order, the keys its
// P^T half holds: 4 hh + 0..3 and 8 + 4 hh + 0..3 of the 16-key group
// (hh = l / 32 = G / 2).  A transposing read in which lane j of group G
// points at row (key) 4 (G / 2) + j / 4, features 16 (G % 2) + 4 (j % 4)
// + 0..3, hands lane i features 16 (G % 2) + i of the 4 keys 4 (G / 2) + e;
// the second read is the same, 8 keys (rows) further on.  The swizzle term
// of those rows depends on the row modulo 4, the same for every key group,
// so only the feature block changes the lane offset.
template <int KD>
__device__ __forceinline__ void lane_offsets(LaneOffsets<KD>& o, int lane) {
  using G = Geo<KD>;
  const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int c = 0; c < G::NC; ++c) o.k[c] = G::kslot(l32, 2 * c + hh);
  const int Gq = lane >> 4, j = lane & 15;
  const int row = 4 * (Gq >> 1) + (j >> 2);
#pragma unroll
  for (int d = 0; d < G::NB; ++d) {
    const int feat = 32 * d + 16 * (Gq & 1) + 4 * (j & 3);
    o.v[d] = G::vslot(row, feat >> 3) * 16 + (feat & 7) * 2;
  }
}

}  // namespace
}  // namespace gqa
