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
// operands are K-contiguous.  The products run as 16x16x32 MFMAs (the
// 32x32x16 form does the same work per cycle but draws more power, and
// under the board's power limit the clock drops: about 4% slower here).
// With this orientation one lane of the accumulators holds, for one token,
// 32 of the 128 features of a head (4 consecutive features of each 16-row
// block) and the other 96 sit in lanes l ^ 16, l ^ 32 and l ^ 48: the
// per-head RMS needs two cross-lane exchanges, and the RoPE partners
// (feature i and i + 64) sit in the same lane.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gqa {

namespace {

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kBK = 64;          // K elements per LDS stage: one 128-byte line per row
constexpr int kStages = 2;       // loads run kStages stages ahead
constexpr int kWSlots = 3;       // LDS ring slots of W stages
constexpr int kXSlots = 2;       // LDS ring slots of X stages
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

// One operand's share of a K stage, staged straight from global memory into
// LDS (buffer_load ... lds, no register staging).  One instruction fills 64
// consecutive 16-byte LDS slots = kRowsPerDma rows, each one whole 128-byte
// line of the operand (half lines cost the address unit and L2 one request
// per 64 bytes); lane i writes slot i, so it loads the global chunk that the
// swizzle places there.  A wave issues kInstr of them per stage; the
// per-lane byte offsets at K = 0 are computed once, and chunks at or past
// column `kcols` read as zero.
constexpr int kRowsPerDma = 64 / kCPR;
// the swizzle term of a lane alternates between even and odd instructions
static_assert(2 * kRowsPerDma == kRPW * kCPR, "two swizzle terms per lane");

template <int ROWS>
struct DmaPlan {
  static constexpr int kInstr = ROWS / kRowsPerDma / (kThreads / 64);
  static_assert(kInstr % 2 == 0, "instruction parity fixes the swizzle term");
  unsigned voff[kInstr];  // byte offset of this lane's chunk at K = 0
  int kc[2];              // K offset (elements) of this lane's chunk: even, odd instructions
  int slot0;              // first LDS slot of this wave's rows

  // swap12: LDS rows 64..127 take operand rows 128..191 and the other
  // way round (a head_dim-256 head's RoPE partners then sit in one wave)
  __device__ __forceinline__ void init(int ld, int wave, int lane, bool swap12 = false) {
    const int r_in = lane / kCPR;
    // row = (wave kInstr + j) kRowsPerDma + r_in, so (row / kRPW) % kCPR
    // depends on the lane and on the parity of j only
#pragma unroll
    for (int p = 0; p < 2; ++p)
      kc[p] = ((lane % kCPR) ^ (((p * kRowsPerDma + r_in) / kRPW) & (kCPR - 1))) * 8;
#pragma unroll
    for (int j = 0; j < kInstr; ++j) {
      int row = (wave * kInstr + j) * kRowsPerDma + r_in;
      if (swap12 && (row >> 6) == 1) row += 64;
      else if (swap12 && (row >> 6) == 2) row -= 64;
      voff[j] = (unsigned)((row * ld + kc[j & 1]) * 2);
    }
    slot0 = wave * kInstr * kRowsPerDma * kCPR;
  }

  // instruction j of the stage whose K offset (along X) is k0, into `stage`
  // (the operand's first slot in that LDS stage).  kalign (the row lengths
  // are multiples of kBK, so no stage has a K tail; a compile-time constant
  // at every call): the descriptor is already based at the stage's K
  // offset, and the per-lane offset alone decides whether the row exists.
  // Otherwise each chunk finds its own column: X column k reads operand
  // column k - wrap once k >= wrap (wrap > 0: W read twice for X = [hi |
  // lo]), and chunks at or past column `kcols` are redirected out of range.
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rsrc, u32x4* stage, int j, int k0,
                                        int kcols, int wrap, bool kalign) const {
    unsigned v = voff[j];
    if (!kalign) {
      const int kk = k0 + kc[j & 1];
      const int kw = wrap > 0 && kk >= wrap ? kk - wrap : kk;
      v = kw < kcols ? v + (unsigned)((kw - kc[j & 1]) * 2) : 0x80000000u;
    }
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

// s_waitcnt for all of this wave's LDS reads
__device__ __forceinline__ void wait_lds() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Output tiles and their order.  The tile order walks groups of kGroupM
// token tiles and, inside a group, the feature tiles token tile by token
// tile, so that tiles close in the order share activations and weights.
// The order is cut into kXcds contiguous runs, one per XCD: workgroup i
// runs on XCD i % 8 and takes tiles i / 8, i / 8 + G, i / 8 + 2 G, ... of
// its XCD's run, where G is the number of workgroups per XCD, so the G
// tiles an XCD works on at one time are neighbours in the order and share
// its L2.
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

// A batch of independent products (the plain epilogues) walks the members'
// tiles one member after the other.
struct TileOrder {
  int ntn, ntm, per_z, total, per_xcd;
  __device__ __forceinline__ TileOrder(int N, int M, int BN, int BM, int batch) {
    ntn = (N + BN - 1) / BN;
    ntm = (M + BM - 1) / BM;
    per_z = ntn * ntm;
    total = per_z * batch;
    per_xcd = (total + kXcds - 1) / kXcds;
  }
  // position id of the order -> (batch member, feature tile, token tile)
  __device__ __forceinline__ void at(int id, int& z, int& tn, int& tm) const {
    z = id / per_z;
    id -= z * per_z;
    const int group = id / (kGroupM * ntn);
    const int first_m = group * kGroupM;
    const int gm = min(ntm - first_m, kGroupM);
    const int in = id - group * kGroupM * ntn;
    tm = first_m + in % gm;
    tn = in / gm;
  }
};

__host__ __device__ constexpr int gemm_tiles(int N, int M, int BN, int BM) {
  return ((N + BN - 1) / BN) * ((M + BM - 1) / BM);
}

// Bytes of the operands' bf16 rows [row0, nrows) with `ld` elements per row,
// clamped to what one buffer descriptor addresses.
__device__ __forceinline__ int rows_bytes(int row0, int nrows, int ld) {
  long long bytes = (long long)(nrows - row0) * ld * 2;
  if (bytes < 0) bytes = 0;
  if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
  return (int)bytes;
}

// A persistent workgroup computes its tiles one after the other through one
// continuous LDS pipeline: its K stages are numbered across tiles, W of
// stage s sits in ring slot s % 3 and X in slot s % 2 (160 KB), and the
// loads that run two stages ahead cross into the next tile during the last
// trips of the current one, so the next tile's first stage (and the W half
// of its second) is in LDS when the current tile's epilogue starts; the
// rest of its second stage is loaded right after it.  The epilogue stages
// its output through the X slot of the tile's last stage (32 tokens x 128
// features per wave at a time) after one barrier; a barrier after it makes
// the next tile's first stage visible.  Compared with one workgroup
// per tile, the next tile's prologue and the workgroup launch are off the
// critical path, which pays at short K (a few stages per tile).
//
// F16 (plain epilogues only): W and X hold fp16 values and the products run
// on the fp16 matrix cores; everything else (staging, order, epilogue) is
// the same, since the loads move bytes.
template <int BN, int BM, int EPI, bool KALIGN, bool F16 = false>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmArgs a) {
  static_assert(!F16 || !is_qkv_epi(EPI), "the QKV epilogues take bf16 operands");
  constexpr int WN = BN / 2, WM = BM / 2;
  constexpr int FB = WN / 16, TB = WM / 16;
  static_assert(WN == 128, "the epilogues stage 128 features per wave");
  static_assert(kBK == 64 && kStages == 2 && kWSlots == 3 && kXSlots == 2,
                "the pipeline below is written for 2 steps, W 3 and X 2 stages deep");
  static_assert(FB == 8 && TB == 8, "64 MFMAs per step");
  // One LDS array: the W ring, then the X ring.  A second __shared__ array
  // would give the compiler alias scopes under which it waits for every
  // LDS DMA in flight before each fragment read; the waits below already
  // order them.
  constexpr int kWStage = BN * kCPR, kXStage = BM * kCPR;  // 16-byte slots per stage
  static_assert((kThreads / 64) * 32 * 16 <= kXStage, "the epilogue stages through an X slot");
  __shared__ u32x4 lds[kWSlots * kWStage + kXSlots * kXStage];
  poison_lds(lds);
  auto wring = [&](unsigned slot) { return &lds[slot * kWStage]; };
  auto xring = [&](unsigned slot) { return &lds[kWSlots * kWStage + slot * kXStage]; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int N = a.N, M = a.M, K = a.K;
  const int batch = is_qkv_epi(EPI) ? 1 : max(a.batch, 1);
  const TileOrder order(N, M, BN, BM, batch);
  const int xcd = (int)(blockIdx.x % kXcds);
  const int per_wg = (int)(gridDim.x / kXcds);  // workgroups on this XCD
  const int run_end = min((xcd + 1) * order.per_xcd, order.total);
  int id = xcd * order.per_xcd + (int)(blockIdx.x / kXcds);
  if (id >= run_end) return;  // no tile for this workgroup

  const int nk = (K + kBK - 1) / kBK;
  // W may be narrower than X along K (w_kmod): X = [hi | lo] reads W twice
  const int Kw = a.w_kmod > 0 ? a.w_kmod : K;
  DmaPlan<BN> pw;
  DmaPlan<BM> px;
  pw.init(Kw, wave, lane, EPI == kEpiQKV256);
  px.init(K, wave, lane);
  constexpr int kLw = DmaPlan<BN>::kInstr, kLx = DmaPlan<BM>::kInstr;
  static_assert(kLw == 8 && kLx == 8, "one load per four MFMAs in the second half of a step");
  const int wrap = a.w_kmod > 0 ? Kw : 0;
  // K offset into W of a tile's stage kt when K is aligned (K <= 2 Kw: X =
  // [hi | lo] reads W at most twice, and Kw is a multiple of kBK)
  auto w_k0 = [&](int kt) { const int k0 = kt * kBK; return k0 >= Kw ? k0 - Kw : k0; };

  // Operand rows of the current tile (cur) and of this workgroup's next
  // tile (nxt; zero bytes when there is none: its loads then read zeros
  // into ring slots nobody reads).
  struct Src { const bf16* w; const bf16* x; int wbytes, xbytes; int n0, m0; };
  auto src_of = [&](int tile) {
    Src s;
    if (tile >= run_end) {
      s.w = a.W; s.x = a.X; s.wbytes = 0; s.xbytes = 0; s.n0 = 0; s.m0 = 0;
      return s;
    }
    int z, tn, tm;
    order.at(tile, z, tn, tm);
    s.n0 = tn * BN;
    s.m0 = tm * BM;
    s.w = a.W + (size_t)z * a.sW + (size_t)s.n0 * Kw;
    s.x = a.X + (size_t)z * a.sX + (size_t)s.m0 * K;
    s.wbytes = rows_bytes(s.n0, N, Kw);
    s.xbytes = rows_bytes(s.m0, M, K);
    return s;
  };
  Src cur = src_of(id);
  Src nxt = src_of(id + per_wg);

  // The loads of stage kt of a tile into W ring slot ws and X ring slot xs:
  // two buffer descriptors (rebased to the stage's K offset when K is
  // aligned) and 8 + 8 instructions, issued one at a time (half 0 = W, 1 =
  // X).
  struct StageLoad {
    __amdgpu_buffer_rsrc_t w, x;
    u32x4 *dw, *dx;
    int kx;
  };
  auto stage_load = [&](const Src& s, int kt, unsigned ws, unsigned xs) {
    StageLoad l;
    l.dw = wring(ws);
    l.dx = xring(xs);
    l.kx = kt * kBK;
    const int ow = KALIGN ? w_k0(kt) : 0, ox = KALIGN ? l.kx : 0;
    l.w = __builtin_amdgcn_make_buffer_rsrc((void*)(s.w + ow), 0, max(s.wbytes - 2 * ow, 0),
                                            0x00020000);
    l.x = __builtin_amdgcn_make_buffer_rsrc((void*)(s.x + ox), 0, max(s.xbytes - 2 * ox, 0),
                                            0x00020000);
    return l;
  };
  auto issue = [&](const StageLoad& l, int j, int half) {
    if (half == 0) pw.issue(l.w, l.dw, j, l.kx, Kw, wrap, KALIGN);
    else px.issue(l.x, l.dx, j, l.kx, K, 0, KALIGN);
  };

  // LDS offsets (16-byte slots) of this lane's fragments: row-major
  // fragments of W (features) and X (tokens), row l16 of a 16-row block,
  // chunk 4 s + q4 for the K step s (0, 1) of a stage.  Every fragment row
  // is l16 plus a multiple of 16, so the swizzle term is l16's and one base
  // per step serves all fragments.
  static_assert(WN % 16 == 0 && WM % 16 == 0 && BN % 16 == 0, "fragment rows keep l16's swizzle");
  int cs[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) cs[s] = swz(l16, 4 * s + q4);
  // offsets within a W slot and within an X slot
  auto offa = [&](int s, int f) { return cs[s] + (wn * WN + 16 * f) * kCPR; };
  auto offb = [&](int s, int t) { return cs[s] + (wm * WM + 16 * t) * kCPR; };

  // Prologue: the first tile's stages 0 and 1 (or, for a one-stage K,
  // whatever follows stage 0) in flight, stage 0 landed and visible.
#pragma unroll
  for (int p = 0; p < kStages; ++p) {
    const bool in_cur = p < nk;
    const StageLoad l = stage_load(in_cur ? cur : nxt, in_cur ? p : p - nk, p, p);
#pragma unroll
    for (int j = 0; j < kLw; ++j) issue(l, j, 0);
#pragma unroll
    for (int j = 0; j < kLx; ++j) issue(l, j, 1);
  }
  wait_vmem<kLw + kLx>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // fragments of K step 0 of the first stage
  u32x4 fa[2][FB], fb[2][TB];
  {
    const u32x4* sw = wring(0);
    const u32x4* sx = xring(0);
#pragma unroll
    for (int f = 0; f < FB; ++f) fa[0][f] = sw[offa(0, f)];
#pragma unroll
    for (int t = 0; t < TB; ++t) fb[0][t] = sx[offb(0, t)];
  }

  // One K stage (two 32-wide steps of 64 MFMAs) per trip; g is the stage's
  // number in this workgroup's sequence and kt its index in the current
  // tile.  The fragments of each step are read during the step before,
  // into the other of two register sets, one read per two MFMAs in the
  // first half of the step, so a read has at least half a step to return.
  // The loads of stage g + 2 go to the slots of stages g - 1 (W) and g (X):
  // W's, free since the previous trip's barrier, one per four MFMAs in the
  // second half of the first step, X's likewise in the second step.  Before
  // the second step every wave waits for stage g + 1 (only the W half of
  // stage g + 2 may still be in flight) and meets the others at a barrier:
  // stage g + 1 is then visible, and every wave's reads of stage g are done
  // (the second step's fragments were read during the first), so the
  // second step reloads stage g's X slot while it reads the first fragments
  // of stage g + 1.  Stage g + 2 is stage kt + 2 of this tile or, past its
  // end, a stage of the next one.  A tile's last trip (NEXT false) loads W
  // of stage g + 2 (the next tile's stage 1) but no X, reads no fragments
  // in its second step and has no barrier: X of the next tile's stage 1 is
  // loaded, and the next tile's first fragments are read, after the
  // epilogue.
  floatx4 acc[FB][TB];
  unsigned g = 0;  // unsigned: the X slot g % 2 is a mask
  // A trip loads stage kt + kofs of tile rl (kofs = 2 with this tile,
  // 2 - nk with the next one).
  auto trip = [&](int kt, const Src& rl, int kofs, auto NEXT) {
    const unsigned w0 = g % kWSlots, w1 = (g + 1) % kWSlots, w2 = (g + 2) % kWSlots;
    const u32x4* sw = wring(w0);
    const u32x4* sx = xring(g % kXSlots);
    const u32x4* sw1 = wring(w1);
    const u32x4* sx1 = xring((g + 1) % kXSlots);
    const StageLoad ld = stage_load(rl, kt + kofs, w2, g % kXSlots);
#pragma unroll
    for (int step = 0; step < 2; ++step) {
      if (step == 1) {
        if constexpr (NEXT) {
          wait_vmem<kLw, true>();
          __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      const bool reads = step == 0 || NEXT;
      const int ns = step ^ 1;  // the K step whose fragments are read
      const int cb = step, nb = ns;
      // this lane's fragment bases in the slots read (one VALU op each per
      // step; the fragments are then constant offsets below 64 KB, which the
      // reads take as immediates, while offsets from the LDS array's start
      // would pass 64 KB in the X ring and cost an add per read)
      lds_u32x4* rw = (lds_u32x4*)((step == 0 ? sw : sw1) + offa(ns, 0));
      lds_u32x4* rx = (lds_u32x4*)((step == 0 ? sx : sx1) + offb(ns, 0));
      asm volatile("" : "+v"(rw));
      asm volatile("" : "+v"(rx));
#pragma unroll
      for (int i = 0; i < FB * TB; ++i) {
        const int f = i / TB, t = i % TB;
        acc[f][t] = F16 ? mfma16x16x32_f16(fa[cb][f], fb[cb][t], acc[f][t])
                        : mfma16x16x32(fa[cb][f], fb[cb][t], acc[f][t]);
        if (i < 32 && (i & 1) == 0 && reads) {
          // next step's fragments in the order its MFMAs use them
          const int r = i / 2;
          if (r == 0) fa[nb][0] = rw[0];
          else if (r <= TB) fb[nb][r - 1] = rx[16 * (r - 1) * kCPR];
          else fa[nb][r - TB] = rw[16 * (r - TB) * kCPR];
        }
        if (step == 0 && i >= 32 && (i & 3) == 0) issue(ld, (i - 32) / 4, 0);
        if constexpr (NEXT) {
          if (step == 1 && i >= 32 && (i & 3) == 0) issue(ld, (i - 32) / 4, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    ++g;
  };
  using True = std::integral_constant<bool, true>;
  using False = std::integral_constant<bool, false>;

  for (;;) {
#pragma unroll
    for (int f = 0; f < FB; ++f)
#pragma unroll
      for (int t = 0; t < TB; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[f][t][r] = 0.f;

    const int n0 = cur.n0, m0 = cur.m0;
    const int nw = n0 + wn * WN;  // first feature of this wave

    {
      // from trip nk - 2 on, the loads run into the next tile (one uniform
      // branch per trip; the descriptors change once per tile).  A
      // one-stage K has one tile per workgroup: its last trip loads zeros.
      Src rl = nk < kStages ? nxt : cur;
      int kofs = nk < kStages ? 0 : kStages;
      for (int kt = 0; kt < nk - 1; ++kt) {
        if (kt == nk - kStages) {
          // a real branch, not selects executed on every trip
          asm volatile("");
          rl = nxt;
          kofs -= nk;
        }
        trip(kt, rl, kofs, True());
      }
      trip(nk - 1, rl, kofs, False());
    }
    // every wave's reads of the last stage done: its X slot stages the output
    wait_lds();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // The accumulators of token blocks t0 .. TB - 1 stay in the
    // matrix-core registers until block t0's epilogue starts: the compiler
    // would otherwise copy all of them into vector registers at once (right
    // after their last MFMA, stalling on each result) and spill.
    auto pin_from = [&](int t0) {
#pragma unroll
      for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int t = 0; t < TB; ++t)
          if (t >= t0) asm volatile("" : "+a"(acc[f][t]));
    };

    // The output goes out in chunks of 32 tokens, token blocks 2 p and
    // 2 p + 1: lane l holds rows l16 and 16 + l16 of the chunk, each with
    // the wave's features 16 f + 4 q4 + (0..3), f = 0..7.  A chunk is staged
    // as 32 rows x 16 chunks per wave in the X slot of the last stage (g - 1).
    u32x4* const stage = xring((g + 1) % kXSlots) + wave * 32 * 16;
    // lane-derived epilogue addresses are computed here, not kept live
    // (and spilled) across the K loop
    int lane = tid & 63;
    asm volatile("" : "+v"(lane));
    const int l16 = lane & 15, q4 = lane >> 4;
    u32x2* const stage8 = reinterpret_cast<u32x2*>(stage);
    // 4 features at feat (a multiple of 4) of row `row`; chunk c of row r
    // sits at slot c ^ (r & 15)
    auto put8 = [&](int row, int feat, u32x2 v) {
      stage8[(row * 16 + ((feat >> 3) ^ (row & 15))) * 2 + ((feat >> 2) & 1)] = v;
    };
    auto pack4 = [](const floatx4& v) {
      u32x2 w;
      w.x = pack_bf16x2(v[0], v[1]);
      w.y = pack_bf16x2(v[2], v[3]);
      return w;
    };
    // batch member of this tile: its output block
    const size_t oz = is_qkv_epi(EPI) ? 0 : (size_t)(id / order.per_z) * a.sOut;
    if constexpr (EPI == kEpiPlainF32) {
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        pin_from(t);
        const int m = m0 + wm * WM + 16 * t + l16;
        if (m >= M) continue;
#pragma unroll
        for (int f = 0; f < FB; ++f) {
          const int n = nw + 16 * f + 4 * q4;
          if (n >= N) continue;
          *reinterpret_cast<floatx4*>(static_cast<float*>(a.out) + oz + (size_t)m * N + n) = acc[f][t];
        }
      }
    } else if constexpr (EPI == kEpiPlain) {
      // per 32-token chunk: rows of 128 bf16 features per token in LDS,
      // then stored 16 bytes per lane, 4 whole rows per instruction
#pragma unroll
      for (int p = 0; p < TB / 2; ++p) {
        pin_from(2 * p);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int f = 0; f < FB; ++f) put8(16 * tt + l16, 16 * f + 4 * q4, pack4(acc[f][2 * p + tt]));
        const int c = lane & 15;
        const int n = nw + 8 * c;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = 4 * i + (lane >> 4);
          const int m = m0 + wm * WM + 32 * p + row;
          const u32x4 v = stage[row * 16 + (c ^ (row & 15))];
          if (m < M && n < N) st16(static_cast<bf16*>(a.out) + oz + (size_t)m * N + n, v);
        }
      }
    } else if constexpr (EPI == kEpiQKV64) {
      // ---- QKV epilogue, head_dim 64: two heads per wave ----
      // As for head_dim 128 (below), with each 64-feature half of the wave
      // (blocks 0-3 and 4-7) a head of its own: its norm sums the lane's four
      // blocks of the head over the token's four lanes, and RoPE pairs block
      // f with f + 2 (rot 64) or, for rot 32, block 0 with block 1 (blocks 2
      // and 3 pass through).  Past the last head (an odd head count) the
      // second half is skipped.
      if (nw < N) {  // wave-uniform
        const int Hq = a.Hq, Hkv = a.Hkv;
        int kind[2], hid[2];
        bool live[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int head = (nw >> 6) + hb;
          live[hb] = nw + 64 * hb < N;
          if (head < Hq) { kind[hb] = 0; hid[hb] = head; }
          else if (head < Hq + Hkv) { kind[hb] = 1; hid[hb] = head - Hq; }
          else { kind[hb] = 2; hid[hb] = head - Hq - Hkv; }
        }
        // norm weights of this lane's features 16 (f % 4) + 4 q4 + (0..3) of head f / 4
        u32x2 wpk[FB];
#pragma unroll
        for (int f = 0; f < FB; ++f) {
          const int hb = f >> 2;
          const u32x2 one = {0x3f803f80u, 0x3f803f80u};  // bf16 1.0
          const bool dn = live[hb] && kind[hb] != 2 && a.qk_norm;
          wpk[f] = dn ? ld8((kind[hb] == 0 ? a.q_norm_w : a.k_norm_w) + 16 * (f & 3) + 4 * q4) : one;
        }
        const int half = a.rot >> 1;
        const int L = a.L;
#pragma unroll
        for (int p = 0; p < TB / 2; ++p) {
          pin_from(2 * p);
          const int mb = m0 + wm * WM + 32 * p;
          const int b0 = mb / L;
          const int tok0 = mb - b0 * L;
          const bool long_seq = L >= 32;
          auto locate = [&](int r, int& b, int& tok) {  // row mb + r, 0 <= r < 32
            if (long_seq) {
              tok = tok0 + r;
              b = b0;
              if (tok >= L) { tok -= L; ++b; }
            } else {
              b = (mb + r) / L;
              tok = mb + r - b * L;
            }
          };
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int t = 2 * p + tt;
            const int row = 16 * tt + l16;
            const int mr = mb + row;
            if (a.y_raw && mr < M) {
              float* yr = a.y_raw + (size_t)mr * N + nw + 4 * q4;
#pragma unroll
              for (int f = 0; f < FB; ++f) {
                // only the normalised heads' rows are kept (the norm backward)
                if (!live[f >> 2] || kind[f >> 2] == 2 || !a.qk_norm) continue;
                *reinterpret_cast<floatx4*>(yr + 16 * f) = acc[f][t];
              }
            }
            int rb, rtok;
            locate(row, rb, rtok);
            const float2* cs = a.rope + (size_t)(a.start_pos ? (mr < M ? mr : 0) : rtok) * half;
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
              if (!live[hb]) continue;  // wave-uniform
              const int f0 = 4 * hb;
              float inv = 1.0f;
              if (kind[hb] != 2 && a.qk_norm) {
                float ss = 0.f;
#pragma unroll
                for (int f = f0; f < f0 + 4; ++f)
#pragma unroll
                  for (int r = 0; r < 4; ++r) ss += acc[f][t][r] * acc[f][t][r];
                ss = sum_xor32(sum_xor16(ss));
                inv = 1.0f / __builtin_sqrtf(ss * (1.0f / 64.0f) + a.eps);
              }
              // x of feature 16 fl + 4 q4 + e of head hb, normalised
              auto xn = [&](int fl, int e) {
                const u32x2 w = wpk[f0 + fl];
                const float gg = (e & 1) ? hi_bf16(e < 2 ? w.x : w.y) : lo_bf16(e < 2 ? w.x : w.y);
                return acc[f0 + fl][t][e] * inv * gg;
              };
              auto put4 = [&](int feat, const floatx4& y) { put8(row, 64 * hb + feat, pack4(y)); };
              if (kind[hb] == 2) {
#pragma unroll
                for (int fl = 0; fl < 4; ++fl) put4(16 * fl + 4 * q4, acc[f0 + fl][t]);
              } else {
                // feature i < rot/2 pairs with i + rot/2: block fl with fl + 2
                // for rot 64, block 0 with block 1 for rot 32 (every index a
                // constant)
                auto pair = [&](int fl, int fl2) {
                  const int i0 = 16 * fl + 4 * q4;
                  const floatx4 c01 = *reinterpret_cast<const floatx4*>(cs + i0);
                  const floatx4 c23 = *reinterpret_cast<const floatx4*>(cs + i0 + 2);
                  const float cc[4] = {c01[0], c01[2], c23[0], c23[2]};
                  const float sn[4] = {c01[1], c01[3], c23[1], c23[3]};
                  floatx4 y1, y2;
#pragma unroll
                  for (int e = 0; e < 4; ++e) {
                    const float x1 = xn(fl, e), x2 = xn(fl2, e);
                    y1[e] = x1 * cc[e] - x2 * sn[e];
                    y2[e] = x2 * cc[e] + x1 * sn[e];
                  }
                  put4(i0, y1);
                  put4(16 * fl2 + 4 * q4, y2);
                };
                if (half == 32) {
                  pair(0, 2);
                  pair(1, 3);
                } else {  // blocks 2 and 3 are past the rotary width: norm only
                  pair(0, 1);
#pragma unroll
                  for (int fl = 2; fl < 4; ++fl) {
                    const floatx4 y = {xn(fl, 0), xn(fl, 1), xn(fl, 2), xn(fl, 3)};
                    put4(16 * fl + 4 * q4, y);
                  }
                }
              }
            }
          }
          int sp0 = 0, sp1 = 0;
          if (a.start_pos && long_seq) {
            sp0 = a.start_pos[b0];
            if ((b0 + 1) * L < M) sp1 = a.start_pos[b0 + 1];
          }
          // lane l moves chunk l % 16 of row 4 i + l / 16: chunks 0-7 are head
          // 0's row, 8-15 head 1's
          const int c = lane & 15;
          const int hb = c >> 3;
          const int kd = hb ? kind[1] : kind[0];
          const int h = hb ? hid[1] : hid[0];
          const bool lv = hb ? live[1] : live[0];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int row = 4 * i + (lane >> 4);
            const int m = mb + row;
            const u32x4 v = stage[row * 16 + (c ^ (row & 15))];
            if (m >= M || !lv) continue;
            int b, tok;
            locate(row, b, tok);
            bf16* dst;
            if (kd == 0) {
              dst = a.q + (((size_t)b * Hq + h) * L + tok) * 64;
            } else {
              const int base = !a.start_pos ? 0 : long_seq ? (b == b0 ? sp0 : sp1) : a.start_pos[b];
              const int pos = base + tok;
              if (pos < 0 || pos >= a.cap) continue;
              dst = (kd == 1 ? a.k_cache : a.v_cache) + (((size_t)b * Hkv + h) * a.cap + pos) * 64;
            }
            st16(dst + 8 * (c & 7), v);
          }
        }
      }
    } else if constexpr (EPI == kEpiQKV256) {
      // ---- QKV epilogue, head_dim 256 (full rotary): a tile is one head ----
      // W's rows were loaded with 64-row blocks 1 and 2 swapped, so wave wn
      // holds features 64 wn + (0..63) in blocks 0-3 and 128 + 64 wn + (0..63)
      // in blocks 4-7: every RoPE pair (i, i + 128) sits in one lane, block f
      // with f + 4, as for head_dim 128.  Only the norm's sum of squares
      // spans the two waves of a pair (wn = 0, 1 over the same tokens): per
      // 32-token chunk each wave posts its two partial sums per lane in LDS
      // (two slots, alternating by chunk) and reads its partner's after one
      // barrier.  The slots are in the W ring slot of the tile's last stage,
      // which no load writes before the next tile's first trip; the head is
      // the same for the whole workgroup, so every wave runs the same
      // barriers.
      float* const xss = reinterpret_cast<float*>(wring((g + 2) % kWSlots));
      const int Hq = a.Hq, Hkv = a.Hkv;
      const int head = n0 >> 8;
      int kind, h;
      if (head < Hq) { kind = 0; h = head; }
      else if (head < Hq + Hkv) { kind = 1; h = head - Hq; }
      else { kind = 2; h = head - Hq - Hkv; }
      const bool do_norm = kind != 2 && a.qk_norm;
      // head feature of this wave's feature fl (0..127)
      auto feat = [&](int fl) { return fl < 64 ? 64 * wn + fl : 64 + 64 * wn + fl; };
      u32x2 wpk[FB];
#pragma unroll
      for (int f = 0; f < FB; ++f) {
        const u32x2 one = {0x3f803f80u, 0x3f803f80u};  // bf16 1.0
        wpk[f] = do_norm ? ld8((kind == 0 ? a.q_norm_w : a.k_norm_w) + feat(16 * f + 4 * q4)) : one;
      }
      const int L = a.L;
#pragma unroll
      for (int p = 0; p < TB / 2; ++p) {
        pin_from(2 * p);
        const int mb = m0 + wm * WM + 32 * p;
        const int b0 = mb / L;
        const int tok0 = mb - b0 * L;
        const bool long_seq = L >= 32;
        auto locate = [&](int r, int& b, int& tok) {  // row mb + r, 0 <= r < 32
          if (long_seq) {
            tok = tok0 + r;
            b = b0;
            if (tok >= L) { tok -= L; ++b; }
          } else {
            b = (mb + r) / L;
            tok = mb + r - b * L;
          }
        };
        const float2* cs[2];
        float ss[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int t = 2 * p + tt;
          const int row = 16 * tt + l16;
          const int mr = mb + row;
          if (a.y_raw && do_norm && mr < M) {  // kept for the norm backward only
            float* yr = a.y_raw + (size_t)mr * N + n0;
#pragma unroll
            for (int f = 0; f < FB; ++f)
              *reinterpret_cast<floatx4*>(yr + feat(16 * f + 4 * q4)) = acc[f][t];
          }
          int rb, rtok;
          locate(row, rb, rtok);
          cs[tt] = a.rope + (size_t)(a.start_pos ? (mr < M ? mr : 0) : rtok) * 128;
          ss[tt] = 0.f;
          if (do_norm) {
#pragma unroll
            for (int f = 0; f < FB; ++f)
#pragma unroll
              for (int r = 0; r < 4; ++r) ss[tt] += acc[f][t][r] * acc[f][t][r];
            ss[tt] = sum_xor32(sum_xor16(ss[tt]));
          }
        }
        float inv[2] = {1.0f, 1.0f};
        if (do_norm) {
          float* slot = xss + (p & 1) * 512;
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) slot[(wave * 64 + lane) * 2 + tt] = ss[tt];
          wait_lds();
          __builtin_amdgcn_s_barrier();
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const float s = ss[tt] + slot[((wave ^ 1) * 64 + lane) * 2 + tt];
            inv[tt] = 1.0f / __builtin_sqrtf(s * (1.0f / 256.0f) + a.eps);
          }
        }
        if (kind == 2) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int f = 0; f < FB; ++f) put8(16 * tt + l16, 16 * f + 4 * q4, pack4(acc[f][2 * p + tt]));
        } else {
          // block f (head features 64 wn + i, i < 64) with block f + 4 (the
          // same + 128); rotary frequency 64 wn + i
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int f = 0; f < 4; ++f) {
              const int t = 2 * p + tt;
              const int i0 = 16 * f + 4 * q4;
              const floatx4 c01 = *reinterpret_cast<const floatx4*>(cs[tt] + 64 * wn + i0);
              const floatx4 c23 = *reinterpret_cast<const floatx4*>(cs[tt] + 64 * wn + i0 + 2);
              const float cc[4] = {c01[0], c01[2], c23[0], c23[2]};
              const float sn[4] = {c01[1], c01[3], c23[1], c23[3]};
              const u32x2 w1 = wpk[f], w2 = wpk[f + 4];
              const float g1[4] = {lo_bf16(w1.x), hi_bf16(w1.x), lo_bf16(w1.y), hi_bf16(w1.y)};
              const float g2[4] = {lo_bf16(w2.x), hi_bf16(w2.x), lo_bf16(w2.y), hi_bf16(w2.y)};
              floatx4 y1, y2;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float x1 = acc[f][t][e] * inv[tt] * g1[e];
                const float x2 = acc[f + 4][t][e] * inv[tt] * g2[e];
                y1[e] = x1 * cc[e] - x2 * sn[e];
                y2[e] = x2 * cc[e] + x1 * sn[e];
              }
              put8(16 * tt + l16, i0, pack4(y1));
              put8(16 * tt + l16, i0 + 64, pack4(y2));
            }
        }
        int sp0 = 0, sp1 = 0;
        if (kind != 0 && a.start_pos && long_seq) {
          sp0 = a.start_pos[b0];
          if ((b0 + 1) * L < M) sp1 = a.start_pos[b0 + 1];
        }
        // chunk l % 16 of row 4 i + l / 16: the wave's features 8 c .. 8 c + 7
        const int c = lane & 15;
        const int fo = feat(8 * c);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = 4 * i + (lane >> 4);
          const int m = mb + row;
          const u32x4 v = stage[row * 16 + (c ^ (row & 15))];
          if (m >= M) continue;
          int b, tok;
          locate(row, b, tok);
          bf16* dst;
          if (kind == 0) {
            dst = a.q + (((size_t)b * Hq + h) * L + tok) * 256;
          } else {
            const int base = !a.start_pos ? 0 : long_seq ? (b == b0 ? sp0 : sp1) : a.start_pos[b];
            const int pos = base + tok;
            if (pos < 0 || pos >= a.cap) continue;
            dst = (kind == 1 ? a.k_cache : a.v_cache) + (((size_t)b * Hkv + h) * a.cap + pos) * 256;
          }
          st16(dst + fo, v);
        }
      }
    } else if (nw < N) {  // wave-uniform
      // ---- QKV epilogue: one head of 128 features per wave ----
      // Per 32-token chunk a lane holds two tokens (rows l16 and 16 + l16)
      // and, of each, the features 16 f + 4 q4 + (0..3), f = 0..7; the
      // token's other 96 features sit in lanes l16 + 16 q, q != q4.  The
      // values are normalised (a sum of squares over the lane's 32 values,
      // then over the four lanes) and rotated in registers (feature i <
      // rot/2 pairs with i + rot/2: block f with block f + rot/32, in the
      // same lane), written to LDS as rows of 128 bf16 per token and stored
      // 16 bytes per lane, 4 whole rows per instruction (a head's rows are
      // contiguous in q and in the caches).
      const int head = nw >> 7;
      const int Hq = a.Hq, Hkv = a.Hkv;
      int kind;  // 0 = q, 1 = k, 2 = v
      int h;
      if (head < Hq) { kind = 0; h = head; }
      else if (head < Hq + Hkv) { kind = 1; h = head - Hq; }
      else { kind = 2; h = head - Hq - Hkv; }
      const bool do_norm = (kind != 2) && a.qk_norm;
      const bf16* wsrc = kind == 0 ? a.q_norm_w : a.k_norm_w;
      // norm weights of this lane's features 16 f + 4 q4 + (0..3), kept packed
      u32x2 wpk[FB];
#pragma unroll
      for (int f = 0; f < FB; ++f) {
        const u32x2 one = {0x3f803f80u, 0x3f803f80u};  // bf16 1.0
        wpk[f] = do_norm ? ld8(wsrc + 16 * f + 4 * q4) : one;
      }
      const int half = a.rot >> 1;
      const int L = a.L;
      // RoPE table rows of this lane's two rows of chunk p, and the table
      // loads of a chunk's first four rope_pair calls.  The loads of chunk
      // p + 1 go out at the end of chunk p's rotation, so their latency
      // runs under chunk p's stores and chunk p + 1's norm.
      const float2* cs[2];
      auto rope_rows = [&](int p) {
        const int mb = m0 + wm * WM + 32 * p;
        const int b0 = mb / L;  // wave-uniform
        const int tok0 = mb - b0 * L;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int mr = mb + 16 * tt + l16;
          int tok;
          if (L >= 32) {
            tok = tok0 + 16 * tt + l16;
            if (tok >= L) tok -= L;
          } else {
            tok = mr - (mr / L) * L;
          }
          cs[tt] = a.rope + (size_t)(a.start_pos ? (mr < M ? mr : 0) : tok) * half;
        }
      };
      floatx4 pre[4][2];
      auto fetch = [&](int k, int tt, int f1) {
        const int i0 = 16 * f1 + 4 * q4;
        pre[k & 3][0] = *reinterpret_cast<const floatx4*>(cs[tt] + i0);
        pre[k & 3][1] = *reinterpret_cast<const floatx4*>(cs[tt] + i0 + 2);
      };
      // rot 128: call k rotates row k / 4, block k % 4 with k % 4 + 4;
      // rot 64: call k rotates row k / 2, block k % 2 with k % 2 + 2
      auto fetch_first = [&]() {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (half == 64) fetch(k, 0, k);
          else fetch(k, k / 2, k % 2);
        }
      };
      if (kind != 2) {
        rope_rows(0);
        fetch_first();
      }
#pragma unroll
      for (int p = 0; p < TB / 2; ++p) {
        pin_from(2 * p);
        // the weights stay packed between chunks (unpacked, they would
        // take 16 more registers through the stores)
#pragma unroll
        for (int f = 0; f < FB; ++f) asm volatile("" : "+v"(wpk[f]));
        // Token rows mb .. mb + 31 of this chunk: row m is token tok of
        // sequence b (m = b L + tok).  One division per chunk (wave-uniform);
        // a row's (b, tok) follows by carrying over sequence ends, which
        // takes at most one step per row when L >= 32.
        const int mb = m0 + wm * WM + 32 * p;
        const int b0 = mb / L;
        const int tok0 = mb - b0 * L;
        const bool long_seq = L >= 32;
        auto locate = [&](int r, int& b, int& tok) {  // row mb + r, 0 <= r < 32
          if (long_seq) {
            tok = tok0 + r;
            b = b0;
            if (tok >= L) { tok -= L; ++b; }
          } else {
            b = (mb + r) / L;
            tok = mb + r - b * L;
          }
        };
        // the lane's two rows: raw projection out and norm scales
        float inv[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int t = 2 * p + tt;
          const int row = 16 * tt + l16;
          const int mr = mb + row;
          if (a.y_raw && do_norm && mr < M) {  // wave-uniform; kept for the norm backward only
            float* yr = a.y_raw + (size_t)mr * N + nw + 4 * q4;
#pragma unroll
            for (int f = 0; f < FB; ++f) *reinterpret_cast<floatx4*>(yr + 16 * f) = acc[f][t];
          }
          inv[tt] = 1.0f;
          if (do_norm) {
            float ss = 0.f;
#pragma unroll
            for (int f = 0; f < FB; ++f)
#pragma unroll
              for (int r = 0; r < 4; ++r) ss += acc[f][t][r] * acc[f][t][r];
            ss = sum_xor32(sum_xor16(ss));
            inv[tt] = 1.0f / __builtin_sqrtf(ss * (1.0f / 128.0f) + a.eps);
          }
        }
        if (kind == 2) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int f = 0; f < FB; ++f) put8(16 * tt + l16, 16 * f + 4 * q4, pack4(acc[f][2 * p + tt]));
        } else {
          // Rotate-half RoPE over the first `rot` features.  A rope_pair
          // call rotates block f1 of row tt with its partner block f2 and
          // needs the (cos, sin) of features 16 f1 + 4 q4 + (0..3): two
          // 16-byte loads, issued four calls ahead.
          auto rope_pair = [&](int tt, int f1, int f2, const floatx4& c01, const floatx4& c23) {
            const int t = 2 * p + tt;
            const int i0 = 16 * f1 + 4 * q4;
            const float cc[4] = {c01[0], c01[2], c23[0], c23[2]};
            const float sn[4] = {c01[1], c01[3], c23[1], c23[3]};
            const u32x2 w1 = wpk[f1], w2 = wpk[f2];
            const float g1[4] = {lo_bf16(w1.x), hi_bf16(w1.x), lo_bf16(w1.y), hi_bf16(w1.y)};
            const float g2[4] = {lo_bf16(w2.x), hi_bf16(w2.x), lo_bf16(w2.y), hi_bf16(w2.y)};
            floatx4 y1, y2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x1 = acc[f1][t][e] * inv[tt] * g1[e];
              const float x2 = acc[f2][t][e] * inv[tt] * g2[e];
              y1[e] = x1 * cc[e] - x2 * sn[e];
              y2[e] = x2 * cc[e] + x1 * sn[e];
            }
            put8(16 * tt + l16, i0, pack4(y1));
            put8(16 * tt + l16, i0 + half, pack4(y2));
          };
          auto norm_only = [&](int tt, int f) {
            const int t = 2 * p + tt;
            const u32x2 w = wpk[f];
            const floatx4 y = {acc[f][t][0] * inv[tt] * lo_bf16(w.x), acc[f][t][1] * inv[tt] * hi_bf16(w.x),
                               acc[f][t][2] * inv[tt] * lo_bf16(w.y), acc[f][t][3] * inv[tt] * hi_bf16(w.y)};
            put8(16 * tt + l16, 16 * f + 4 * q4, pack4(y));
          };
          if (half == 64) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              rope_pair(k / 4, k % 4, k % 4 + 4, pre[k & 3][0], pre[k & 3][1]);
              if (k + 4 < 8) fetch(k + 4, 1, k % 4);
              __builtin_amdgcn_sched_barrier(0);
            }
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) rope_pair(k / 2, k % 2, k % 2 + 2, pre[k][0], pre[k][1]);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
              for (int f = 4; f < FB; ++f) norm_only(tt, f);
          }
          if (p + 1 < TB / 2) {
            rope_rows(p + 1);
            fetch_first();
          }
        }
        // cache offsets of the (at most two, when L >= 32) sequences the
        // chunk's rows belong to, read once per chunk
        int sp0 = 0, sp1 = 0;
        if (kind != 0 && a.start_pos && long_seq) {
          sp0 = a.start_pos[b0];
          if ((b0 + 1) * L < M) sp1 = a.start_pos[b0 + 1];
        }
        // Store the chunk: lane l moves chunk l % 16 of row 4 i + l / 16.
        const int c = lane & 15;
        if (long_seq) {
          // The chunk's rows are tokens tok0 + r of sequence b0, then (past
          // its end) tokens tok0 + r - L of sequence b0 + 1: row r goes to
          // base0 + (pos0 + r) rows or base1 + (pos1 + r) rows, with
          // wave-uniform bases and offsets.
          bf16* base0;
          ptrdiff_t stride1;  // from sequence b0's rows to b0 + 1's
          int pos0 = tok0, pos1 = tok0 - L;
          if (kind == 0) {
            base0 = a.q + ((size_t)b0 * Hq + h) * L * 128;
            stride1 = (ptrdiff_t)Hq * L * 128;
          } else {
            bf16* cache = kind == 1 ? a.k_cache : a.v_cache;
            base0 = cache + ((size_t)b0 * Hkv + h) * a.cap * 128;
            stride1 = (ptrdiff_t)Hkv * a.cap * 128;
            pos0 += sp0;
            pos1 += sp1;
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int row = 4 * i + (lane >> 4);
            const u32x4 v = stage[row * 16 + (c ^ (row & 15))];
            const bool second = tok0 + row >= L;
            const int pos = (second ? pos1 : pos0) + row;
            const bool ok = mb + row < M && (kind == 0 || (pos >= 0 && pos < a.cap));
            if (ok) st16(base0 + (second ? stride1 : 0) + (ptrdiff_t)pos * 128 + 8 * c, v);
            // at most four rows in flight: the next chunk's table loads are
            // live here
            if (i == 3) __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int row = 4 * i + (lane >> 4);
            const int m = mb + row;
            const u32x4 v = stage[row * 16 + (c ^ (row & 15))];
            if (m >= M) continue;
            int b, tok;
            locate(row, b, tok);
            bf16* dst;
            if (kind == 0) {
              dst = a.q + (((size_t)b * Hq + h) * L + tok) * 128;
            } else {
              const int pos = (a.start_pos ? a.start_pos[b] : 0) + tok;
              if (pos < 0 || pos >= a.cap) continue;
              bf16* cache = kind == 1 ? a.k_cache : a.v_cache;
              dst = cache + (((size_t)b * Hkv + h) * a.cap + pos) * 128;
            }
            st16(dst + 8 * c, v);
          }
        }
      }
    }

    // every load and store of this wave done (the next tile's stage 0
    // landed), on the way out of the loop too
    wait_vmem<0, true>();
    id += per_wg;
    if (id >= run_end) break;
    cur = nxt;
    nxt = src_of(id + per_wg);
    // stage 0 of the next tile visible; every wave's staging is done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // X of the next tile's stage 1 (held back by the last trip) into the X
    // slot that staged the output; the stage index is opaque so that its
    // load offsets are not hoisted out of the tile loop
    int k1 = kStages - 1;
    asm volatile("" : "+s"(k1));
    {
      const StageLoad l = stage_load(cur, k1, (g + 1) % kWSlots, (g + 1) % kXSlots);
#pragma unroll
      for (int j = 0; j < kLx; ++j) issue(l, j, 1);
    }
    const u32x4* sw = wring(g % kWSlots);
    const u32x4* sx = xring(g % kXSlots);
#pragma unroll
    for (int f = 0; f < FB; ++f) fa[0][f] = sw[offa(0, f)];
#pragma unroll
    for (int t = 0; t < TB; ++t) fb[0][t] = sx[offb(0, t)];
  }
}


// cos/sin of position * theta^(-2i/d) for i < d/2, angles in double.
// Entry idx of the RoPE table: row `row` is token row - b L of sequence b
// (position start_pos[b] + that token), or position row without start_pos.
__device__ __forceinline__ void rope_entry(float2* table, const int* start_pos, int rows, int L,
                                           int half, double theta, long idx) {
  if (idx >= (long)rows * half) return;
  const int row = (int)(idx / half);
  const int i = (int)(idx - (long)row * half);
  long pos;
  if (start_pos) {
    const int b = row / L;
    pos = (long)start_pos[b] + (row - b * L);
  } else {
    pos = row;
  }
  table[idx] = rope_cos_sin(pos, i, half, theta);
}

__global__ void rope_table_kernel(float2* __restrict__ table, const int* __restrict__ start_pos,
                                  int rows, int L, int half, double theta) {
  rope_entry(table, start_pos, rows, L, half, theta, (long)blockIdx.x * blockDim.x + threadIdx.x);
}

// Few-token projection (decode): weight streaming.  A workgroup computes a
// C^T tile of 32 features x 64 tokens; its 8 waves each take one eighth of
// K, reading the MFMA fragments straight from global memory (the weights
// are read once; the activations stay in L2), and the partial tiles are
// summed through LDS.  Out-of-range rows and K tails read as zero.
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyUnroll = 4;

template <bool F16>
__global__ __launch_bounds__(64 * kSkinnyWaves) void gemm_skinny_kernel(GemmArgs a) {
  __shared__ floatx16 red[kSkinnyWaves - 1][2][64];
  poison_lds(red);
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int N = a.N, M = a.M, K = a.K;
  const int f0 = blockIdx.x * 32;
  const int m0 = blockIdx.y * 64;
  const int Kw = a.w_kmod > 0 ? a.w_kmod : K;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.W + (size_t)f0 * Kw, (long long)(N - f0) * Kw * 2);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.X + (size_t)m0 * K, (long long)(M - m0) * K * 2);
  // this workgroup's share of K (split z of gridDim.z), then each wave's
  const int ksteps = (K + 15) / 16;
  const int zsteps = (ksteps + (int)gridDim.z - 1) / (int)gridDim.z;
  const int zb = (int)blockIdx.z * zsteps;
  const int ze = min(ksteps, zb + zsteps);
  const int per = (max(ze - zb, 0) + kSkinnyWaves - 1) / kSkinnyWaves;
  const int kb = (zb + wave * per) * 16;
  const int ke = min(min(K, ze * 16), kb + per * 16);
  constexpr unsigned kOob = 0x80000000u;

  floatx16 acc0 = {}, acc1 = {};
  auto step = [&](int k) {
    const int kwc = k % Kw + 8 * hh;
    const int kxc = k + 8 * hh;
    const u32x4 fa = buf_ld16(rw, kwc < Kw ? (unsigned)((l32 * Kw + kwc) * 2) : kOob);
    const u32x4 fb0 = buf_ld16(rx, kxc < K ? (unsigned)((l32 * K + kxc) * 2) : kOob);
    const u32x4 fb1 = buf_ld16(rx, kxc < K ? (unsigned)(((32 + l32) * K + kxc) * 2) : kOob);
    acc0 = F16 ? mfma32x32x16_f16(fa, fb0, acc0) : mfma32x32x16(fa, fb0, acc0);
    acc1 = F16 ? mfma32x32x16_f16(fa, fb1, acc1) : mfma32x32x16(fa, fb1, acc1);
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
  // split z's partial product goes to part[z]
  const bool partial = gridDim.z > 1;
  float* const pz = partial ? a.part + (size_t)blockIdx.z * M * N : nullptr;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const floatx16& c = t == 0 ? acc0 : acc1;
    const int m = m0 + 32 * t + l32;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = f0 + 8 * j + 4 * hh;
      if (n >= N) continue;
      if (partial) {
        floatx4 w = {c[4 * j + 0], c[4 * j + 1], c[4 * j + 2], c[4 * j + 3]};
        *reinterpret_cast<floatx4*>(pz + (size_t)m * N + n) = w;
      } else if (a.out_f32) {
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

// The few-token GEMM for K (and a hi|lo X's W width) a multiple of 64: a
// workgroup computes 64 features x 64 tokens over its share of K.  Its
// stages of 64 K (whole 128-byte lines of 64 W rows and 64 X rows, 16 KB)
// are loaded straight into a ring of kSkR LDS slots, kSkR - 2 stages ahead
// of the products, so a workgroup keeps about 48 KB of loads in flight and
// the weights stream at close to the memory's rate; each wave owns one
// 32 x 32 block of the output (4 MFMAs per stage).  Stage i's slot is
// reloaded with stage i + kSkR - 1 right after the barrier that opens
// stage i + 1: every wave has read it by then.
constexpr int kSkR = 5;
constexpr int kSkStage = 2 * 64 * 8;  // 16-byte slots per stage (W rows, then X rows)

template <int N>
__device__ __forceinline__ void wait_vmem_upto(int n) {
  // s_waitcnt needs an immediate: n (0 .. N) in steps of 4 loads per stage
  if constexpr (N > 0) {
    if (n >= N) {
      wait_vmem<N>();
      return;
    }
    wait_vmem_upto<N - 4>(n);
  } else {
    wait_vmem<0>();
  }
}

template <bool F16, bool WCVT = false>
__global__ __launch_bounds__(256, 2) void gemm_skinny_lds_kernel(GemmArgs a) {
  static_assert(!WCVT || F16, "W is rounded to fp16 for the fp16 products");
  __shared__ u32x4 lds[kSkR * kSkStage];
  poison_lds(lds);
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int N = a.N, M = a.M, K = a.K;
  const int Kw = a.w_kmod > 0 ? a.w_kmod : K;
  const int f0 = blockIdx.x * 64, m0 = blockIdx.y * 64;
  // this workgroup's stages [s0, s0 + n) of the K/64 stages
  const int nst = K / 64;
  const int zs = (nst + (int)gridDim.z - 1) / (int)gridDim.z;
  const int s0 = (int)blockIdx.z * zs;
  const int n = max(min(nst, s0 + zs) - s0, 0);

  // Loads: waves 0-1 move W rows, waves 2-3 X rows, 32 rows per wave in 4
  // instructions of 8 whole rows each, into the swizzled slots the
  // fragment reads expect (chunk c of row r at c ^ ((r / 2) % 8)).
  const int op = wave >> 1;
  const int rbase = 32 * (wave & 1);
  const int ld = op ? K : Kw;
  const long long opbytes = op ? (long long)(M - m0) * K * 2 : (long long)(N - f0) * Kw * 2;
  const __bf16* opbase = op ? a.X + (size_t)m0 * K : a.W + (size_t)f0 * Kw;
  unsigned voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = rbase + 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    voff[j] = (unsigned)((row * ld + c * 8) * 2);
  }
  auto issue_stage = [&](int i) {
    const int k0 = (s0 + i) * 64;
    const int kc = op ? k0 : (k0 >= Kw ? k0 - Kw : k0);  // W is read twice for X = [hi | lo]
    const __amdgpu_buffer_rsrc_t r = make_rsrc(opbase + kc, opbytes - 2LL * kc);
    u32x4* dst = &lds[(i % kSkR) * kSkStage + op * 512 + rbase * 8];
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(r, dst + 64 * j, voff[j]);
  };

  // fragments: wave = (feature block fb, token block tb)
  const int fb = wave & 1, tb = wave >> 1;
  int oa[4], ob[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int c = (2 * st + hh) ^ ((l32 >> 1) & 7);  // rows 32 fb + l32 and 32 tb + l32 share it
    oa[st] = (32 * fb + l32) * 8 + c;
    ob[st] = 512 + (32 * tb + l32) * 8 + c;
  }

  const int pro = min(n, kSkR);
  for (int i = 0; i < pro; ++i) issue_stage(i);
  if (a.rope_table) {
    const long nthreads = (long)gridDim.x * gridDim.y * gridDim.z * 256;
    const long gid = (((long)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * 256 +
                     threadIdx.x;
    for (long e = gid; e < (long)a.rope_rows * a.rope_half; e += nthreads)
      rope_entry(a.rope_table, a.rope_start_pos, a.rope_rows, a.rope_L, a.rope_half, a.rope_theta, e);
  }
  floatx16 acc = {};
  for (int i = 0; i < n; ++i) {
    // stage i landed: only the stages issued after it may be in flight
    // (up to kSkR - 1 of them, 4 loads each)
    const int issued = i == 0 ? pro : min(n, i + kSkR - 1);
    wait_vmem_upto<4 * (kSkR - 1)>(4 * (issued - i - 1));
    __builtin_amdgcn_s_barrier();
    // every wave is past its reads of stage i - 1: reload that slot
    if (i >= 1 && i + kSkR - 1 < n) issue_stage(i + kSkR - 1);
    const u32x4* sl = &lds[(i % kSkR) * kSkStage];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      u32x4 fa = sl[oa[st]];
      const u32x4 fbv = sl[ob[st]];
      if constexpr (WCVT) {
        fa.x = pack_f16x2(lo_bf16(fa.x), hi_bf16(fa.x));
        fa.y = pack_f16x2(lo_bf16(fa.y), hi_bf16(fa.y));
        fa.z = pack_f16x2(lo_bf16(fa.z), hi_bf16(fa.z));
        fa.w = pack_f16x2(lo_bf16(fa.w), hi_bf16(fa.w));
      }
      acc = F16 ? mfma32x32x16_f16(fa, fbv, acc) : mfma32x32x16(fa, fbv, acc);
    }
    wait_lds();
  }

  const bool partial = gridDim.z > 1;
  float* const pz = partial ? a.part + (size_t)blockIdx.z * M * N : nullptr;
  const int m = m0 + 32 * tb + l32;
  if (m >= M) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int nn = f0 + 32 * fb + 8 * j + 4 * hh;
    if (nn >= N) continue;
    if (partial) {
      floatx4 w = {acc[4 * j + 0], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]};
      *reinterpret_cast<floatx4*>(pz + (size_t)m * N + nn) = w;
    } else if (a.out_f32) {
      floatx4 w = {acc[4 * j + 0], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]};
      *reinterpret_cast<floatx4*>(static_cast<float*>(a.out) + (size_t)m * N + nn) = w;
    } else {
      u32x2 w;
      w.x = pack_bf16x2(acc[4 * j + 0], acc[4 * j + 1]);
      w.y = pack_bf16x2(acc[4 * j + 2], acc[4 * j + 3]);
      st8(static_cast<bf16*>(a.out) + (size_t)m * N + nn, w);
    }
  }
}

// out = sum over the splits of part[z] (four elements per thread), fp32 or
// bf16 (N % 4 == 0)
__global__ __launch_bounds__(256) void skinny_sum_kernel(const float* __restrict__ part, int S,
                                                         long long n4, void* out, int out_f32) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  floatx4 acc = reinterpret_cast<const floatx4*>(part)[i];
  for (int z = 1; z < S; ++z) acc += reinterpret_cast<const floatx4*>(part + (size_t)z * n4 * 4)[i];
  if (out_f32) {
    reinterpret_cast<floatx4*>(out)[i] = acc;
  } else {
    u32x2 w;
    w.x = pack_bf16x2(acc[0], acc[1]);
    w.y = pack_bf16x2(acc[2], acc[3]);
    reinterpret_cast<u32x2*>(out)[i] = w;
  }
}

// bf16 -> fp16, eight values per thread (16-byte loads and stores); bf16 to
// fp32 is exact, fp32 to fp16 rounds to nearest even.
__global__ __launch_bounds__(256) void cvt_bf16_f16_kernel(const u32x4* __restrict__ in,
                                                           u32x4* __restrict__ out, long long n8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const u32x4 v = in[i];
  u32x4 r;
  r.x = pack_f16x2(lo_bf16(v.x), hi_bf16(v.x));
  r.y = pack_f16x2(lo_bf16(v.y), hi_bf16(v.y));
  r.z = pack_f16x2(lo_bf16(v.z), hi_bf16(v.z));
  r.w = pack_f16x2(lo_bf16(v.w), hi_bf16(v.w));
  out[i] = r;
}

}  // namespace

hipError_t launch_cvt_bf16_f16(const __bf16* in, void* out, long long n, hipStream_t stream) {
  if (n % 8 != 0) return hipErrorInvalidValue;
  const long long n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  cvt_bf16_f16_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, stream>>>(
      reinterpret_cast<const u32x4*>(in), static_cast<u32x4*>(out), n8);
  return hipGetLastError();
}

// The 64-aligned kernel: K splits that bring the workgroups (64 x 64
// output blocks) to about one per CU (one round; two per CU streamed the
// weights no faster and left more partial products to sum: the 64-token
// decode layer took 0.2206 ms with 10 splits of its projections, 0.2185
// with 6 and 5), each with at least two K stages of 64, and no split left
// short or empty.  Otherwise (the general kernel, 32 features per workgroup) only when
// the features alone leave more than half of the CUs idle: a decode step's
// o_proj (2560 features: 80 workgroups) went from 58 to 30 us (+4 us for
// the sum) with 4 splits, while its QKV projection (4352 features: 136
// workgroups) did not gain from 2.
int skinny_ksplit(int N, int K, int M) {
  if (K % 64 == 0) {
    const int wgs = max(1, ((N + 63) / 64) * ((M + 63) / 64));  // M = 0: an empty call
    const int nst = K / 64;
    int ks = 256 / wgs;
    if (ks > nst / 2) ks = nst / 2;
    if (ks > 16) ks = 16;
    if (ks <= 1) return 1;
    const int per = (nst + ks - 1) / ks;  // stages per split
    return (nst + per - 1) / per;
  }
  const int wgs = (N + 31) / 32;
  if (wgs >= 128) return 1;
  int ks = (256 + wgs - 1) / wgs;
  const int max_ks = (K + 15) / 16 / kSkinnyWaves;  // at least one K step per wave
  if (ks > max_ks) ks = max_ks;
  if (ks > 8) ks = 8;
  return ks < 1 ? 1 : ks;
}

bool skinny_lds_ok(int K, int w_kmod) { return K % 64 == 0 && (w_kmod <= 0 || w_kmod % 64 == 0); }

hipError_t launch_gemm_skinny_bf16(const GemmArgs& args, hipStream_t stream) {
  const int ks = args.part && args.ksplit > 1 ? args.ksplit : 1;
  if (args.w_bf16_to_f16 && (!args.f16 || !skinny_lds_ok(args.K, args.w_kmod)))
    return hipErrorInvalidValue;
  if (args.rope_table && !skinny_lds_ok(args.K, args.w_kmod)) return hipErrorInvalidValue;
  if (skinny_lds_ok(args.K, args.w_kmod)) {
    dim3 grid((args.N + 63) / 64, (args.M + 63) / 64, ks);
    if (args.w_bf16_to_f16)
      gemm_skinny_lds_kernel<true, true><<<grid, 256, 0, stream>>>(args);
    else if (args.f16)
      gemm_skinny_lds_kernel<true><<<grid, 256, 0, stream>>>(args);
    else
      gemm_skinny_lds_kernel<false><<<grid, 256, 0, stream>>>(args);
  } else {
    dim3 grid((args.N + 31) / 32, (args.M + 63) / 64, ks);
    if (args.f16)
      gemm_skinny_kernel<true><<<grid, 64 * kSkinnyWaves, 0, stream>>>(args);
    else
      gemm_skinny_kernel<false><<<grid, 64 * kSkinnyWaves, 0, stream>>>(args);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ks == 1 || args.keep_parts) return e;
  const long long n4 = (long long)args.M * args.N / 4;
  skinny_sum_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, stream>>>(args.part, ks, n4, args.out,
                                                                       args.out_f32);
  return hipGetLastError();
}

hipError_t launch_rope_table(float2* table, const int* start_pos, int rows, int L, int half,
                             double theta, hipStream_t stream) {
  const int n = rows * half;
  if (n == 0) return hipSuccess;
  rope_table_kernel<<<(n + 255) / 256, 256, 0, stream>>>(table, start_pos, rows, L, half, theta);
  return hipGetLastError();
}

namespace {

// Workgroups of the large GEMMs: one per tile (padded to a multiple of the
// XCDs), at most one per compute unit (each holds 160 KB of LDS), rounded
// down to a multiple of the XCDs.  With fewer than kStages K stages a load
// that runs ahead could reach two tiles further, so every workgroup then
// gets exactly one tile.
int gemm_workgroups(int N, int M, int K, int batch = 1) {
  constexpr int BN = 256, BM = 256;
  const int tiles = gemm_tiles(N, M, BN, BM) * batch;
  int grid = (tiles + kXcds - 1) / kXcds * kXcds;
  if ((K + kBK - 1) / kBK < kStages) return grid;
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return grid;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    cus[dev] = n >= kXcds ? n / kXcds * kXcds : -1;
  }
  return cus[dev] > 0 ? min(grid, cus[dev]) : grid;
}

// No stage of either operand has a K tail.
bool k_aligned(const GemmArgs& a) {
  return a.K % kBK == 0 && (a.w_kmod <= 0 || a.w_kmod % kBK == 0);
}

}  // namespace

template <int EPI>
void launch_qkv(const GemmArgs& args, int grid, hipStream_t stream) {
  if (k_aligned(args))
    gemm_bf16_kernel<256, 256, EPI, true><<<grid, kThreads, 0, stream>>>(args);
  else
    gemm_bf16_kernel<256, 256, EPI, false><<<grid, kThreads, 0, stream>>>(args);
}

hipError_t launch_gemm_qkv_bf16(const GemmArgs& args, hipStream_t stream) {
  const int grid = gemm_workgroups(args.N, args.M, args.K);
  switch (args.hd) {
    case 0:
    case 128:
      if (args.rot != 128 && args.rot != 64) return hipErrorInvalidValue;
      launch_qkv<kEpiQKV>(args, grid, stream);
      break;
    case 64:
      if (args.rot != 64 && args.rot != 32) return hipErrorInvalidValue;
      launch_qkv<kEpiQKV64>(args, grid, stream);
      break;
    case 256:
      if (args.rot != 256) return hipErrorInvalidValue;
      launch_qkv<kEpiQKV256>(args, grid, stream);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_plain_bf16(const GemmArgs& args, hipStream_t stream) {
  const int grid = gemm_workgroups(args.N, args.M, args.K, args.batch > 1 ? args.batch : 1);
  const bool kal = k_aligned(args);
  if (args.f16) {  // the output projection of an fp16-carried attention output
    if (args.out_f32) {
      if (kal)
        gemm_bf16_kernel<256, 256, kEpiPlainF32, true, true><<<grid, kThreads, 0, stream>>>(args);
      else
        gemm_bf16_kernel<256, 256, kEpiPlainF32, false, true><<<grid, kThreads, 0, stream>>>(args);
    } else {
      if (kal)
        gemm_bf16_kernel<256, 256, kEpiPlain, true, true><<<grid, kThreads, 0, stream>>>(args);
      else
        gemm_bf16_kernel<256, 256, kEpiPlain, false, true><<<grid, kThreads, 0, stream>>>(args);
    }
    return hipGetLastError();
  }
  if (args.out_f32) {
    if (kal)
      gemm_bf16_kernel<256, 256, kEpiPlainF32, true><<<grid, kThreads, 0, stream>>>(args);
    else
      gemm_bf16_kernel<256, 256, kEpiPlainF32, false><<<grid, kThreads, 0, stream>>>(args);
  } else {
    if (kal)
      gemm_bf16_kernel<256, 256, kEpiPlain, true><<<grid, kThreads, 0, stream>>>(args);
    else
      gemm_bf16_kernel<256, 256, kEpiPlain, false><<<grid, kThreads, 0, stream>>>(args);
  }
  return hipGetLastError();
}

}  // namespace gqa
