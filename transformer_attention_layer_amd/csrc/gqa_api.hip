// C ABI of the GQA layer library: host-side resolution and validation of the
// configuration, workspace sizing, and dispatch to the gfx950 kernels.
//
// Configuration rules (GPT-NeoX issue "Support explicit attention head_dim
// independent of hidden_size / num_attention_heads", sections "Proposed
// configuration behavior", "Proposed implementation" and "Scaling and
// RoPE"; "Attention head partitions: keep each head's dependencies intact"
// for whole GQA groups):
//   d   = head_dim if set, else hidden / Hq (which must then divide evenly)
//   Hkv = num_kv_heads if set, else Hq;  Hq % Hkv == 0;  d even.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/gqa.h"
#include "kernels.h"

// Scratch memory of gqa_layer_forward_noalloc (see scratch_of_current_device).
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local char g_err[512] = "";

gqa_status fail(gqa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

gqa_status ok() {
  g_err[0] = '\0';
  return GQA_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Shape {
  int H, Hq, Hkv, d, G, n_qkv;
  bool bf16;
  bool mfma;     // bf16 with head_dim 64, 128 or 256: the matrix-core attention
  int rot;       // rotary width
  bool fused;    // mfma, and the rotary width (128 or 64) fits the fused QKV epilogue
  bool out_f32;  // o_proj output in fp32
  bool o_split;  // layer forward: attention output as a bf16 hi + lo pair
  bool o_f16;    // layer forward: attention output as fp16, o_proj on the fp16 matrix cores
  bool kv_fp8;   // caches hold E4M3 codes
  float k_scale, v_scale;
};

gqa_status resolve(const gqa_config* in, gqa_config* out, Shape* sh) {
  if (!in) return fail(GQA_ERR_INVALID_ARG, "config pointer is null");
  gqa_config c = *in;
  if (c.hidden_size <= 0 || c.num_heads <= 0)
    return fail(GQA_ERR_INVALID_ARG, "hidden_size (%d) and num_heads (%d) must be positive",
                c.hidden_size, c.num_heads);
  if (c.num_kv_heads < 0 || c.head_dim < 0)
    return fail(GQA_ERR_INVALID_ARG, "num_kv_heads and head_dim must be >= 0 (0 = unset)");
  if (c.head_dim == 0) {
    if (c.hidden_size % c.num_heads != 0)
      return fail(GQA_ERR_HEAD_DIM_INDIVISIBLE,
                  "head_dim unset and hidden_size %d is not divisible by num_heads %d",
                  c.hidden_size, c.num_heads);
    c.head_dim = c.hidden_size / c.num_heads;
  }
  if (c.num_kv_heads == 0) c.num_kv_heads = c.num_heads;
  if (c.num_heads % c.num_kv_heads != 0)
    return fail(GQA_ERR_GROUP_INDIVISIBLE, "num_heads %d is not a multiple of num_kv_heads %d",
                c.num_heads, c.num_kv_heads);
  if (c.head_dim % 2 != 0)
    return fail(GQA_ERR_ODD_HEAD_DIM, "head_dim %d is odd; RoPE needs an even head_dim",
                c.head_dim);
  if (c.dtype != GQA_F32 && c.dtype != GQA_BF16)
    return fail(GQA_ERR_UNSUPPORTED_DTYPE, "dtype %d is not GQA_F32 or GQA_BF16", c.dtype);
  if (c.rotary_dim < 0 || c.rotary_dim > c.head_dim || c.rotary_dim % 2 != 0)
    return fail(GQA_ERR_INVALID_ARG, "rotary_dim %d must be even and in [0, head_dim %d]",
                c.rotary_dim, c.head_dim);
  if (c.rotary_dim == 0) c.rotary_dim = c.head_dim;
  if (c.head_dim > 256)
    return fail(GQA_ERR_UNSUPPORTED_HEAD_DIM,
                "Unsupported head_dim %d: the kernels take even head_dim up to 256", c.head_dim);
  if (c.dtype == GQA_BF16) {
    // bf16 rows are moved in 16-byte pieces and stored 4 features at a time
    if (c.hidden_size % 8 != 0)
      return fail(GQA_ERR_UNSUPPORTED_SHAPE, "hidden_size %d must be a multiple of 8 for bf16",
                  c.hidden_size);
    if (((long long)c.num_heads * c.head_dim) % 8 != 0 ||
        ((long long)(c.num_heads + 2LL * c.num_kv_heads) * c.head_dim) % 8 != 0)
      return fail(GQA_ERR_UNSUPPORTED_SHAPE,
                  "bf16 needs num_heads*head_dim and (num_heads+2*num_kv_heads)*head_dim to be "
                  "multiples of 8");
    if (c.o_split && ((long long)c.num_heads * c.head_dim) % 32 != 0)
      return fail(GQA_ERR_UNSUPPORTED_SHAPE,
                  "o_split needs num_heads*head_dim to be a multiple of 32");
  }
  if (c.kv_fp8 != 0 && c.kv_fp8 != 1)
    return fail(GQA_ERR_INVALID_ARG, "kv_fp8 must be 0 or 1");
  if (c.kv_fp8) {
    if (c.dtype != GQA_BF16)
      return fail(GQA_ERR_UNSUPPORTED_DTYPE, "kv_fp8 needs dtype GQA_BF16");
    if (c.head_dim != 64 && c.head_dim != 128)
      return fail(GQA_ERR_UNSUPPORTED_HEAD_DIM,
                  "Unsupported head_dim %d with kv_fp8: the FP8 cache is read by the "
                  "matrix-core decode kernel for head_dim 64 and 128", c.head_dim);
    if (c.k_scale == 0.f) c.k_scale = 1.f;
    if (c.v_scale == 0.f) c.v_scale = 1.f;
    if (!(c.k_scale > 0.f) || !isfinite(c.k_scale) || !(c.v_scale > 0.f) || !isfinite(c.v_scale))
      return fail(GQA_ERR_INVALID_ARG, "k_scale and v_scale must be positive and finite");
  }
  if (!(c.rope_theta > 0.f) || !isfinite(c.rope_theta))
    return fail(GQA_ERR_INVALID_ARG, "rope_theta must be positive and finite");
  if (!(c.rms_eps >= 0.f) || !isfinite(c.rms_eps))
    return fail(GQA_ERR_INVALID_ARG, "rms_eps must be >= 0 and finite");
  if ((c.qk_norm != 0 && c.qk_norm != 1) || (c.causal != 0 && c.causal != 1) ||
      (c.out_f32 != 0 && c.out_f32 != 1) || (c.o_split != 0 && c.o_split != 1) ||
      (c.o_fp16 != 0 && c.o_fp16 != 1))
    return fail(GQA_ERR_INVALID_ARG, "qk_norm, causal, out_f32, o_split and o_fp16 must be 0 or 1");
  if (c.o_split && c.o_fp16)
    return fail(GQA_ERR_INVALID_ARG, "o_split and o_fp16 are two carriers of the same value: set one");
  // every kernel indexes heads and widths in 32-bit
  const long long n_qkv = (long long)(c.num_heads + 2LL * c.num_kv_heads) * c.head_dim;
  if (n_qkv > (1LL << 30) || (long long)c.num_heads * c.head_dim > (1LL << 30))
    return fail(GQA_ERR_UNSUPPORTED_SHAPE, "projection widths exceed 2^30");
  if (out) *out = c;
  if (sh) {
    sh->H = c.hidden_size;
    sh->Hq = c.num_heads;
    sh->Hkv = c.num_kv_heads;
    sh->d = c.head_dim;
    sh->G = c.num_heads / c.num_kv_heads;
    sh->n_qkv = (int)n_qkv;
    sh->bf16 = c.dtype == GQA_BF16;
    sh->mfma = sh->bf16 && (c.head_dim == 64 || c.head_dim == 128 || c.head_dim == 256);
    sh->rot = c.rotary_dim;
    sh->fused = sh->bf16 && ((c.head_dim == 128 && (c.rotary_dim == 128 || c.rotary_dim == 64)) ||
                             (c.head_dim == 64 && (c.rotary_dim == 64 || c.rotary_dim == 32)) ||
                             (c.head_dim == 256 && c.rotary_dim == 256));
    sh->out_f32 = c.out_f32 || c.dtype == GQA_F32;
    sh->o_split = c.o_split && c.dtype == GQA_BF16;
    sh->o_f16 = c.o_fp16 && c.dtype == GQA_BF16;
    sh->kv_fp8 = c.kv_fp8 != 0;
    sh->k_scale = c.kv_fp8 ? c.k_scale : 1.f;
    sh->v_scale = c.kv_fp8 ? c.v_scale : 1.f;
  }
  return GQA_OK;
}

size_t esize(const Shape& s) { return s.bf16 ? 2 : 4; }

// split-KV decode is used when a KV group's query rows fit one wave
bool use_decode(const Shape& s, int q_len) { return s.mfma && s.G * q_len <= 32; }

// Splits of at least kDecodeMinChunk keys: shorter ones make the partial
// results (G * q_len rows x head_dim floats per split) a sizeable share of
// the traffic.
// About 4096 waves in all (4 per SIMD of an MI355X) by default.  With few
// (sequence, KV head) streams, one round of waves with longer chunks is
// faster, as long as it still gives each stream 8 or more splits: 512 waves
// (two per CU) over a bf16 cache, 1024 over an FP8 cache, whose kernel
// spends more time per tile in each wave.  Measured on 32768-token caches:
// MQA (64 streams) 5.40-5.55 TB/s with 8 splits, 5.23-5.33 with 16, 4.5
// with 6; GQA (512 streams) 6.05 with 8 splits, 5.94 with 2; MQA over an
// FP8 cache 4.45 TB/s with 16 splits, 2.98 with 8.
constexpr int kDecodeMinChunk = 1024;
constexpr long long kDecodeRoundBf16 = 512;
constexpr long long kDecodeRoundFp8 = 1024;
constexpr long long kDecodeResident = 1280;
void decode_split(const Shape& s, int batch, int cap, int* n_splits, int* chunk) {
  const long long streams = (long long)batch * s.Hkv;
  long long want = (4096 + streams - 1) / (streams > 0 ? streams : 1);
  long long max_splits = (cap + kDecodeMinChunk - 1) / kDecodeMinChunk;
  if (want > max_splits) want = max_splits;
  const long long round = s.kv_fp8 ? kDecodeRoundFp8 : kDecodeRoundBf16;
  const long long one_round = round / (streams > 0 ? streams : 1);
  if (one_round >= 8 && one_round < want) want = one_round;
  if (want < 1) want = 1;
  int ch = (int)((cap + want - 1) / want);
  ch = (ch + 31) / 32 * 32;
  if (ch < 32) ch = 32;
  *chunk = ch;
  *n_splits = (cap + ch - 1) / ch;
  if (*n_splits < 1) *n_splits = 1;
}

// Few tokens (decode): weight-streaming projections instead of 256x256 tiles.
constexpr long long kSkinnyMaxTokens = 256;
bool use_skinny(const Shape& s, long long tokens) { return s.bf16 && tokens <= kSkinnyMaxTokens; }

// The QKV GEMM's own epilogue (norm, RoPE, scatter) writes bf16 caches only;
// FP8 caches take the projection + norm/RoPE pass.
bool use_fused_qkv(const Shape& s, long long tokens) {
  return s.fused && !use_skinny(s, tokens) && !s.kv_fp8;
}

// FP8 caches are read by the split-KV decode kernel only.
gqa_status check_fp8_attn(const Shape& s, int q_len) {
  if (s.kv_fp8 && !use_decode(s, q_len))
    return fail(GQA_ERR_UNSUPPORTED_SHAPE,
                "kv_fp8: attention over an FP8 cache needs (num_heads/num_kv_heads) * q_len "
                "<= 32 (decode); got %d * %d", s.G, q_len);
  return GQA_OK;
}

// The vectorised bf16 norm/RoPE pass (head_dim 64, 128, 256; rotary width
// a multiple of 8) after the fp32 projection; FP8 caches take the general
// pass, which also encodes.
bool use_rows_normrope(const Shape& s) {
  return s.bf16 && !s.kv_fp8 && gqa::normrope_rows_ok(s.d, s.rot);
}

size_t rope_table_bytes(const Shape& s, size_t rows) {
  return align_up(rows * (s.rot / 2) * sizeof(float) * 2);
}

// Partial products of the few-token projections when their K is split
// over workgroups: the QKV projection's, and the layer's o_proj's, which
// reuse the same bytes once the projection has been normalised.
size_t skinny_part_bytes(const Shape& s, size_t T) {
  if (!use_skinny(s, (long long)T)) return 0;
  size_t b = 0;
  if (s.n_qkv % 4 == 0)
    b = (size_t)gqa::skinny_ksplit(s.n_qkv, s.H, (int)T) * T * s.n_qkv * sizeof(float);
  const int ko = s.Hq * s.d * (s.o_split ? 2 : 1);
  if (s.H % 4 == 0) {
    const size_t o = (size_t)gqa::skinny_ksplit(s.H, ko, (int)T) * T * s.H * sizeof(float);
    if (o > b) b = o;
  }
  return align_up(b);
}

// Offset of those partial products in the projection's workspace: after
// the fp32 projection and the RoPE table.
size_t skinny_part_offset(const Shape& s, size_t T) {
  const size_t y = align_up(T * (size_t)s.n_qkv * sizeof(float));  // fp32 projection output
  return use_rows_normrope(s) ? y + align_up(rope_table_bytes(s, T)) : y;
}

// The RoPE table of the separate norm/RoPE pass: after the fp32 projection.
float2* rope_table_at(const Shape& s, void* ws, size_t T) {
  return reinterpret_cast<float2*>(static_cast<char*>(ws) +
                                   align_up(T * (size_t)s.n_qkv * sizeof(float)));
}

size_t ws_qkv(const Shape& s, int batch, int q_len) {
  const size_t T = (size_t)batch * q_len;
  if (use_fused_qkv(s, (long long)T)) return rope_table_bytes(s, T);  // T rows max
  return skinny_part_offset(s, T) + skinny_part_bytes(s, T);
}

size_t ws_attn(const Shape& s, int batch, int q_len, int cap) {
  if (!use_decode(s, q_len)) return 0;
  int ns, ch;
  decode_split(s, batch, cap, &ns, &ch);
  const size_t parts = (size_t)batch * s.Hkv * ns * s.G * q_len;  // the group's real rows
  return align_up(parts * s.d * sizeof(float)) + align_up(parts * 2 * sizeof(float));
}

// o_proj of an fp16-carried attention output rounds W_o to fp16 inside the
// product for few tokens; otherwise it reads a converted copy.
bool oproj_rounds_w(const Shape& s, long long tokens) {
  return s.o_f16 && use_skinny(s, tokens) && gqa::skinny_lds_ok(s.Hq * s.d, 0);
}

// W_o converted to fp16 for an fp16-carried attention output
size_t wo16_bytes(const Shape& s, long long tokens) {
  return s.o_f16 && !oproj_rounds_w(s, tokens) ? align_up((size_t)s.H * s.Hq * s.d * 2) : 0;
}

size_t ws_layer(const Shape& s, int batch, int q_len, int cap) {
  const size_t T = (size_t)batch * q_len;
  return ws_qkv(s, batch, q_len) + align_up(T * s.Hq * s.d * esize(s)) /* q */ +
         align_up(T * s.Hq * s.d * esize(s) * (s.o_split ? 2 : 1)) /* attention output */ +
         ws_attn(s, batch, q_len, cap) + wo16_bytes(s, (long long)T);
}

gqa_status check_launch(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return GQA_OK;
}

gqa_status check_common(const Shape& s, int batch, int q_len, int cap) {
  if (batch < 0 || q_len < 0) return fail(GQA_ERR_INVALID_ARG, "batch and q_len must be >= 0");
  if (cap < q_len)
    return fail(GQA_ERR_CAPACITY, "kv_capacity %d is smaller than q_len %d", cap, q_len);
  if ((long long)batch * q_len > 65535LL * 64)
    return fail(GQA_ERR_UNSUPPORTED_SHAPE, "batch * q_len exceeds %lld tokens", 65535LL * 64);
  if (batch > 65535) return fail(GQA_ERR_UNSUPPORTED_SHAPE, "batch exceeds 65535");
  (void)s;
  return GQA_OK;
}

// y_raw (fused path only): also keep the fp32 projection before norm and RoPE.
gqa_status run_qkv(const gqa_config& c, const Shape& s, int batch, int q_len, const void* x,
                   const void* w_qkv, const void* qn, const void* kn, const int32_t* start_pos,
                   void* q, void* kc, void* vc, int cap, void* ws, hipStream_t st,
                   float* y_raw = nullptr) {
  const int T = batch * q_len;
  if (use_fused_qkv(s, T)) {
    float2* table = reinterpret_cast<float2*>(ws);
    const int rows = start_pos ? T : q_len;
    gqa_status r = check_launch(
        gqa::launch_rope_table(table, start_pos, rows, q_len, s.rot / 2, (double)c.rope_theta, st),
        "rope table");
    if (r != GQA_OK) return r;
    gqa::GemmArgs g{};
    g.W = static_cast<const __bf16*>(w_qkv);
    g.X = static_cast<const __bf16*>(x);
    g.N = s.n_qkv;
    g.M = T;
    g.K = s.H;
    g.q = static_cast<__bf16*>(q);
    g.k_cache = static_cast<__bf16*>(kc);
    g.v_cache = static_cast<__bf16*>(vc);
    g.q_norm_w = static_cast<const __bf16*>(qn);
    g.k_norm_w = static_cast<const __bf16*>(kn);
    g.rope = table;
    g.start_pos = start_pos;
    g.L = q_len;
    g.Hq = s.Hq;
    g.Hkv = s.Hkv;
    g.cap = cap;
    g.qk_norm = c.qk_norm;
    g.rot = s.rot;
    g.hd = s.d;
    g.eps = c.rms_eps;
    g.y_raw = y_raw;
    return check_launch(gqa::launch_gemm_qkv_bf16(g, st), "qkv projection");
  }
  float* y = reinterpret_cast<float*>(ws);
  gqa_status r;
  if (s.bf16) {  // fp32 projection, then norm + rope + scatter
    gqa::GemmArgs g{};
    g.W = static_cast<const __bf16*>(w_qkv);
    g.X = static_cast<const __bf16*>(x);
    g.N = s.n_qkv;
    g.M = T;
    g.K = s.H;
    g.out = y;
    g.out_f32 = 1;
    if (use_skinny(s, T) && s.n_qkv % 4 == 0) {
      g.ksplit = gqa::skinny_ksplit(s.n_qkv, s.H, T);
      g.part = reinterpret_cast<float*>(static_cast<char*>(ws) + skinny_part_offset(s, (size_t)T));
      // the norm + RoPE pass sums the partial products itself
      g.keep_parts = use_rows_normrope(s) ? 1 : 0;
    }
    if (use_skinny(s, T) && use_rows_normrope(s) && gqa::skinny_lds_ok(s.H, 0)) {
      // the projection also fills the RoPE table (no launch of its own)
      g.rope_table = rope_table_at(s, ws, (size_t)T);
      g.rope_start_pos = start_pos;
      g.rope_rows = start_pos ? T : q_len;
      g.rope_L = q_len;
      g.rope_half = s.rot / 2;
      g.rope_theta = (double)c.rope_theta;
    }
    r = use_skinny(s, T)
            ? check_launch(gqa::launch_gemm_skinny_bf16(g, st), "qkv projection (few tokens)")
            : check_launch(gqa::launch_gemm_plain_bf16(g, st), "qkv projection");
  } else {
    gqa::F32Args g{static_cast<const float*>(x), static_cast<const float*>(w_qkv), y, T, s.n_qkv,
                   s.H};
    r = check_launch(gqa::launch_gemm_f32(g, st), "qkv projection (f32)");
  }
  if (r != GQA_OK) return r;
  if (use_rows_normrope(s)) {
    gqa::NormRopeRowsArgs n{};
    const bool few = use_skinny(s, T);
    float2* table = rope_table_at(s, ws, (size_t)T);
    if (!(few && gqa::skinny_lds_ok(s.H, 0))) {
      const int rows = start_pos ? T : q_len;
      r = check_launch(
          gqa::launch_rope_table(table, start_pos, rows, q_len, s.rot / 2, (double)c.rope_theta, st),
          "rope table");
      if (r != GQA_OK) return r;
    }
    n.y = y;
    if (few && s.n_qkv % 4 == 0) {
      const int ks = gqa::skinny_ksplit(s.n_qkv, s.H, T);
      if (ks > 1) {
        n.part = reinterpret_cast<const float*>(static_cast<char*>(ws) + skinny_part_offset(s, (size_t)T));
        n.parts = ks;
      }
    }
    n.q_norm_w = static_cast<const __bf16*>(qn);
    n.k_norm_w = static_cast<const __bf16*>(kn);
    n.rope = table;
    n.start_pos = start_pos;
    n.q = static_cast<__bf16*>(q);
    n.k_cache = static_cast<__bf16*>(kc);
    n.v_cache = static_cast<__bf16*>(vc);
    n.B = batch;
    n.L = q_len;
    n.Hq = s.Hq;
    n.Hkv = s.Hkv;
    n.d = s.d;
    n.rot = s.rot;
    n.cap = cap;
    n.qk_norm = c.qk_norm;
    n.eps = c.rms_eps;
    return check_launch(gqa::launch_normrope_fwd_rows(n, st), "norm + rope");
  }
  gqa::NormRopeArgs n{};
  n.y = y;
  n.q_norm_w = qn;
  n.k_norm_w = kn;
  n.start_pos = start_pos;
  n.q = q;
  n.k_cache = kc;
  n.v_cache = vc;
  n.B = batch;
  n.L = q_len;
  n.Hq = s.Hq;
  n.Hkv = s.Hkv;
  n.d = s.d;
  n.rot = s.rot;
  n.cap = cap;
  n.qk_norm = c.qk_norm;
  n.bf16 = s.bf16;
  n.kv_fp8 = s.kv_fp8;
  n.inv_k_scale = 1.0f / s.k_scale;
  n.inv_v_scale = 1.0f / s.v_scale;
  n.eps = c.rms_eps;
  n.theta = (double)c.rope_theta;
  return check_launch(gqa::launch_normrope(n, st), "norm + rope");
}

// Prefill work split: a workgroup of 4 waves covers hpw query heads of one
// KV group x pb blocks of 32 positions (hpw * pb = 4).
gqa_status prefill_split(const Shape& s, int q_len, int* hpw, int* pb, int* n_hsub,
                         int* n_qtiles) {
  int h = 1;
  if (s.G % 4 == 0) h = 4;
  else if (s.G % 2 == 0) h = 2;
  *hpw = h;
  *pb = 4 / h;
  *n_hsub = s.G / h;
  *n_qtiles = (q_len + *pb * 32 - 1) / (*pb * 32);
  if (*n_qtiles > 65535)
    return fail(GQA_ERR_UNSUPPORTED_SHAPE, "q_len %d needs more than 65535 query tiles", q_len);
  return GQA_OK;
}

// lse (bf16 matrix-core path only): the prefill kernel also writes each
// query row's log-sum-exp, whatever q_len is.
gqa_status run_attn(const gqa_config& c, const Shape& s, int batch, int q_len, const void* q,
                    const void* kc, const void* vc, const int32_t* kv_base, int kv_add, int cap,
                    void* o, bool o_split, void* ws, hipStream_t st, float* lse = nullptr,
                    bool o_f16 = false) {
  const double scale = 1.0 / sqrt((double)s.d);
  if (!s.mfma) {  // fp32, or bf16 with a head_dim other than 64, 128, 256
    gqa::F32AttnArgs a{};
    a.q = q;
    a.k = kc;
    a.v = vc;
    a.o = o;
    a.bf16 = s.bf16;
    a.o_split = o_split && s.bf16;
    a.o_f16 = o_f16 && s.bf16;
    a.kv_base = kv_base;
    a.kv_add = kv_add;
    a.B = batch;
    a.Hq = s.Hq;
    a.Hkv = s.Hkv;
    a.Lq = q_len;
    a.cap = cap;
    a.d = s.d;
    a.causal = c.causal;
    a.scale = (float)scale;
    return check_launch(gqa::launch_attn_vec(a, st), "attention (vector path)");
  }
  gqa::AttnArgs a{};
  a.d = s.d;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(kc);
  a.v = static_cast<const __bf16*>(vc);
  a.o = static_cast<__bf16*>(o);
  a.o_split = o_split;
  a.o_f16 = o_f16;
  a.kv_base = kv_base;
  a.kv_add = kv_add;
  a.B = batch;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.Lq = q_len;
  a.cap = cap;
  a.causal = c.causal;
  // with FP8 caches the K scale multiplies every score and the V scale the
  // output: the kernels work on the codes' values
  a.scale_log2 = (float)(scale * 1.4426950408889634 * (double)s.k_scale);
  a.v_scale = s.v_scale;
  if (s.kv_fp8) {
    a.k = nullptr;
    a.v = nullptr;
    a.k8 = static_cast<const unsigned char*>(kc);
    a.v8 = static_cast<const unsigned char*>(vc);
  }
  a.lse = lse;
  if (!lse && use_decode(s, q_len)) {
    decode_split(s, batch, cap, &a.n_splits, &a.chunk);
    // Launches of more waves than the GPU holds at once (about 1280: five
    // per CU, by LDS) over a bf16 cache start each wave at its own tile:
    // 64 x 8 streams of 32768 keys 5.75 -> 5.88 TB/s.  One round of waves
    // (MQA) was 1-4% slower rotated, and the FP8 kernel did not gain.
    a.rotate = !s.kv_fp8 && (long long)batch * s.Hkv * a.n_splits > kDecodeResident;
    const size_t parts = (size_t)batch * s.Hkv * a.n_splits * s.G * q_len;
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_ml = reinterpret_cast<float2*>(static_cast<char*>(ws) + align_up(parts * s.d * sizeof(float)));
    return check_launch(gqa::launch_attn_decode_bf16(a, st), "decode attention");
  }
  gqa_status r = prefill_split(s, q_len, &a.hpw, &a.pb, &a.n_hsub, &a.n_qtiles);
  if (r != GQA_OK) return r;
  return check_launch(gqa::launch_attn_prefill_bf16(a, st), "prefill attention");
}

// part (few tokens, optional): skinny_part_bytes of scratch for a K split.
// w_o16 (optional): W_o as fp16, for an attention output o held as fp16.
// w_cvt (few tokens, o as fp16, skinny_lds_ok): W_o stays bf16 and is
// rounded to fp16 inside the product.
gqa_status run_oproj(const Shape& s, int tokens, const void* o, bool o_split, const void* w_o,
                     void* out, hipStream_t st, void* part = nullptr,
                     const void* w_o16 = nullptr, bool w_cvt = false) {
  if (s.bf16) {
    gqa::GemmArgs g{};
    g.W = static_cast<const __bf16*>(w_o16 ? w_o16 : w_o);
    g.f16 = w_o16 || w_cvt ? 1 : 0;
    g.w_bf16_to_f16 = w_cvt ? 1 : 0;
    g.X = static_cast<const __bf16*>(o);
    g.N = s.H;
    g.M = tokens;
    g.K = s.Hq * s.d * (o_split ? 2 : 1);
    g.w_kmod = o_split ? s.Hq * s.d : 0;
    g.out = out;
    g.out_f32 = s.out_f32;
    if (use_skinny(s, tokens)) {
      if (part && s.H % 4 == 0) {
        g.ksplit = gqa::skinny_ksplit(s.H, g.K, tokens);
        g.part = static_cast<float*>(part);
      }
      return check_launch(gqa::launch_gemm_skinny_bf16(g, st), "o_proj (few tokens)");
    }
    return check_launch(gqa::launch_gemm_plain_bf16(g, st), "o_proj");
  }
  gqa::F32Args g{static_cast<const float*>(o), static_cast<const float*>(w_o),
                 static_cast<float*>(out), tokens, s.H, s.Hq * s.d};
  return check_launch(gqa::launch_gemm_f32(g, st), "o_proj (f32)");
}

// ---------------------------------------------------------------------------
// Training (forward with saved activations, backward)
// ---------------------------------------------------------------------------

gqa_status check_train(const gqa_config& c, const Shape& s) {
  if (!s.bf16) return fail(GQA_ERR_UNSUPPORTED_DTYPE, "the training entry points need GQA_BF16");
  if (s.d != 64 && s.d != 128)
    return fail(GQA_ERR_UNSUPPORTED_HEAD_DIM,
                "Unsupported head_dim %d for training: the backward kernels take head_dim 64 "
                "and 128", s.d);
  if (c.o_split || s.kv_fp8)
    return fail(GQA_ERR_UNSUPPORTED_SHAPE, "the training entry points need o_split 0 and kv_fp8 0");
  if (!gqa::normrope_rows_ok(s.d, s.rot))
    return fail(GQA_ERR_UNSUPPORTED_SHAPE,
                "the training entry points need a rotary width that is a multiple of 8 (got %d)",
                s.rot);
  return GQA_OK;
}

// Split of the token axis for a weight-gradient GEMM with N x M outputs
// (256 x 256 tiles): enough batch members that their tiles cover the 256
// compute units, at least 512 tokens each, chunks of whole 64s.
struct TokSplit {
  int S, Rc;
};
TokSplit tok_split(long long T, int N, int M) {
  const long long tiles = (long long)((N + 255) / 256) * ((M + 255) / 256);
  long long S = (256 + tiles - 1) / tiles;
  const long long max_s = T / 512 > 1 ? T / 512 : 1;
  if (S > max_s) S = max_s;
  if (S < 1) S = 1;
  long long Rc = (T + S - 1) / S;
  Rc = (Rc + 63) / 64 * 64;
  TokSplit t;
  t.Rc = (int)Rc;
  t.S = (int)((T + Rc - 1) / Rc);
  return t;
}

// Workspace of the backward: byte offsets of its buffers.
struct BwdLayout {
  TokSplit so, sq;  // splits of the dW_o and dW_qkv products
  int gblocks;      // blocks of the norm/RoPE backward
  size_t doutT, oT, dwo_part, woT, dO, D, lse2, dq, dk, dv, rope, gpart, gstage, dy, dyT, xT, dwq_part, wqT;
  size_t total;
};

BwdLayout bwd_layout(const Shape& s, int batch, int L) {
  BwdLayout b{};
  const size_t T = (size_t)batch * L;
  const size_t qw = (size_t)s.Hq * s.d, kvw = (size_t)s.Hkv * s.d;
  b.so = tok_split((long long)T, s.H, (int)qw);
  b.sq = tok_split((long long)T, s.n_qkv, s.H);
  b.gblocks = gqa::normrope_bwd_blocks((long long)T, b.sq.Rc, s.Hq + 2 * s.Hkv);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  b.doutT = take((size_t)b.so.S * b.so.Rc * s.H * 2);
  b.oT = take((size_t)b.so.S * b.so.Rc * qw * 2);
  b.dwo_part = take(b.so.S > 1 ? (size_t)b.so.S * s.H * qw * 4 : 0);
  b.woT = take(qw * s.H * 2);
  b.dO = take(T * qw * 2);
  b.D = take(T * s.Hq * 4);
  b.lse2 = take(T * s.Hq * 4);
  b.dq = take(T * qw * 2);
  b.dk = take(T * kvw * 2);
  b.dv = take(T * kvw * 2);
  b.rope = take((size_t)L * (s.rot / 2) * 8);
  b.gpart = take((size_t)b.gblocks * 2 * s.d * 4);
  b.gstage = take(gqa::dgamma_stage_floats(s.d) * 4);
  b.dy = take(T * s.n_qkv * 2);
  b.dyT = take((size_t)b.sq.S * b.sq.Rc * s.n_qkv * 2);
  b.xT = take((size_t)b.sq.S * b.sq.Rc * s.H * 2);
  b.dwq_part = take(b.sq.S > 1 ? (size_t)b.sq.S * s.n_qkv * s.H * 4 : 0);
  b.wqT = take((size_t)s.H * s.n_qkv * 2);
  b.total = off;
  return b;
}

// out (fp32 [M, N]) = sum over the token chunks of X_s W_s^T, with X and W
// chunk-major ([S][M][Rc] and [S][N][Rc]); partial products go to `part`
// and are summed when there is more than one chunk.
gqa_status weight_grad(const __bf16* X, const __bf16* W, int M, int N, const TokSplit& t, float* part,
                       float* out, hipStream_t st, const char* what) {
  gqa::GemmArgs g{};
  g.X = X;
  g.W = W;
  g.M = M;
  g.N = N;
  g.K = t.Rc;
  g.batch = t.S;
  g.sX = (long long)M * t.Rc;
  g.sW = (long long)N * t.Rc;
  g.sOut = (long long)M * N;
  g.out = t.S > 1 ? part : out;
  g.out_f32 = 1;
  gqa_status r = check_launch(gqa::launch_gemm_plain_bf16(g, st), what);
  if (r != GQA_OK || t.S == 1) return r;
  return check_launch(gqa::launch_sum_partials(part, t.S, (long long)M * N, out, st), what);
}

// out (cfg dtype [M, N]) = X [M, K] W^T with W given as [N, K]
gqa_status plain_gemm(const __bf16* X, const __bf16* W, int M, int N, int K, void* out, int out_f32,
                      hipStream_t st, const char* what) {
  gqa::GemmArgs g{};
  g.X = X;
  g.W = W;
  g.M = M;
  g.N = N;
  g.K = K;
  g.out = out;
  g.out_f32 = out_f32;
  return check_launch(gqa::launch_gemm_plain_bf16(g, st), what);
}

// The checks every layer forward makes on the host before any launch.
gqa_status check_layer_call(const gqa_config* cfg, int batch, int q_len, const void* x,
                            const void* w_qkv, const void* q_norm_w, const void* k_norm_w,
                            const void* w_o, const void* k_cache, const void* v_cache,
                            int kv_capacity, const void* out, gqa_config* c, Shape* s) {
  gqa_status r = resolve(cfg, c, s);
  if (r != GQA_OK) return r;
  if ((r = check_common(*s, batch, q_len, kv_capacity)) != GQA_OK) return r;
  if (batch == 0 || q_len == 0) return ok();
  if (!x || !w_qkv || !w_o || !k_cache || !v_cache || !out)
    return fail(GQA_ERR_INVALID_ARG, "x, w_qkv, w_o, k_cache, v_cache and out must be non-null");
  if (c->qk_norm && (!q_norm_w || !k_norm_w))
    return fail(GQA_ERR_INVALID_ARG, "qk_norm is on but a norm weight is null");
  return check_fp8_attn(*s, q_len);
}

// The layer's kernels in order (workspace of ws_layer bytes, already checked).
gqa_status run_layer(const gqa_config& c, const Shape& s, int batch, int q_len, const void* x,
                     const void* w_qkv, const void* q_norm_w, const void* k_norm_w,
                     const void* w_o, void* k_cache, void* v_cache, int kv_capacity,
                     const int32_t* cache_len, void* out, void* workspace, hipStream_t st);

// Scratch of gqa_layer_forward_noalloc: a static device array, one copy per
// GPU, held until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: its device address is taken once per
// device with hipGetSymbolAddress (device current) and used from then on.

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

gqa_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GQA_ERR_UNSUPPORTED_SHAPE, "device %d: the static scratch covers devices 0..%d",
                dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(GQA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return GQA_OK;
}

}  // namespace

extern "C" {

gqa_status gqa_resolve(const gqa_config* in, gqa_config* out) {
  gqa_status r = resolve(in, out, nullptr);
  return r == GQA_OK ? ok() : r;
}

size_t gqa_workspace_bytes(const gqa_config* cfg, int32_t batch, int32_t q_len,
                           int32_t kv_capacity, int32_t kind) {
  Shape s;
  if (resolve(cfg, nullptr, &s) != GQA_OK || batch < 0 || q_len < 0) return 0;
  switch (kind) {
    case GQA_WS_QKV: return ws_qkv(s, batch, q_len);
    case GQA_WS_ATTN: return ws_attn(s, batch, q_len, kv_capacity);
    case GQA_WS_LAYER: return ws_layer(s, batch, q_len, kv_capacity);
    case GQA_WS_OPROJ: return 0;
    case GQA_WS_TRAIN_FORWARD: return rope_table_bytes(s, (size_t)q_len);
    case GQA_WS_BACKWARD: return bwd_layout(s, batch, q_len).total;
    default: return 0;
  }
}

gqa_status qkv_proj_normrope(const gqa_config* cfg, int32_t batch, int32_t q_len, const void* x,
                             const void* w_qkv, const void* q_norm_w, const void* k_norm_w,
                             const int32_t* start_pos, void* q, void* k_cache, void* v_cache,
                             int32_t kv_capacity, void* workspace, size_t workspace_bytes,
                             void* stream) {
  gqa_config c;
  Shape s;
  gqa_status r = resolve(cfg, &c, &s);
  if (r != GQA_OK) return r;
  if ((r = check_common(s, batch, q_len, kv_capacity)) != GQA_OK) return r;
  if (batch == 0 || q_len == 0) return ok();
  if (!x || !w_qkv || !q || !k_cache || !v_cache)
    return fail(GQA_ERR_INVALID_ARG, "x, w_qkv, q, k_cache and v_cache must be non-null");
  if (c.qk_norm && (!q_norm_w || !k_norm_w))
    return fail(GQA_ERR_INVALID_ARG, "qk_norm is on but a norm weight is null");
  const size_t need = ws_qkv(s, batch, q_len);
  if (need && (!workspace || workspace_bytes < need))
    return fail(GQA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                workspace_bytes);
  r = run_qkv(c, s, batch, q_len, x, w_qkv, q_norm_w, k_norm_w, start_pos, q, k_cache, v_cache,
              kv_capacity, workspace, (hipStream_t)stream);
  return r == GQA_OK ? ok() : r;
}

gqa_status gqa_attn_core(const gqa_config* cfg, int32_t batch, int32_t q_len, const void* q,
                         const void* k_cache, const void* v_cache, const int32_t* kv_len,
                         int32_t kv_capacity, void* o, void* workspace, size_t workspace_bytes,
                         void* stream) {
  gqa_config c;
  Shape s;
  gqa_status r = resolve(cfg, &c, &s);
  if (r != GQA_OK) return r;
  if ((r = check_common(s, batch, q_len, kv_capacity)) != GQA_OK) return r;
  if (batch == 0 || q_len == 0) return ok();
  if (!q || !k_cache || !v_cache || !o)
    return fail(GQA_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be non-null");
  if ((r = check_fp8_attn(s, q_len)) != GQA_OK) return r;
  const size_t need = ws_attn(s, batch, q_len, kv_capacity);
  if (need && (!workspace || workspace_bytes < need))
    return fail(GQA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                workspace_bytes);
  r = run_attn(c, s, batch, q_len, q, k_cache, v_cache, kv_len, kv_len ? 0 : q_len, kv_capacity, o,
               false, workspace, (hipStream_t)stream);
  return r == GQA_OK ? ok() : r;
}

gqa_status gqa_o_proj(const gqa_config* cfg, int32_t tokens, const void* o, const void* w_o,
                      void* out, void* stream) {
  gqa_config c;
  Shape s;
  gqa_status r = resolve(cfg, &c, &s);
  if (r != GQA_OK) return r;
  if (tokens < 0) return fail(GQA_ERR_INVALID_ARG, "tokens must be >= 0");
  if (tokens > 65535 * 64) return fail(GQA_ERR_UNSUPPORTED_SHAPE, "too many tokens");
  if (tokens == 0) return ok();
  if (!o || !w_o || !out) return fail(GQA_ERR_INVALID_ARG, "o, w_o and out must be non-null");
  r = run_oproj(s, tokens, o, false, w_o, out, (hipStream_t)stream);
  return r == GQA_OK ? ok() : r;
}

gqa_status gqa_layer_forward(const gqa_config* cfg, int32_t batch, int32_t q_len, const void* x,
                             const void* w_qkv, const void* q_norm_w, const void* k_norm_w,
                             const void* w_o, void* k_cache, void* v_cache, int32_t kv_capacity,
                             const int32_t* cache_len, void* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  gqa_config c;
  Shape s;
  gqa_status r = check_layer_call(cfg, batch, q_len, x, w_qkv, q_norm_w, k_norm_w, w_o, k_cache,
                                  v_cache, kv_capacity, out, &c, &s);
  if (r != GQA_OK || batch == 0 || q_len == 0) return r;
  const size_t need = ws_layer(s, batch, q_len, kv_capacity);
  if (!workspace || workspace_bytes < need)
    return fail(GQA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                workspace_bytes);
  r = run_layer(c, s, batch, q_len, x, w_qkv, q_norm_w, k_norm_w, w_o, k_cache, v_cache,
                kv_capacity, cache_len, out, workspace, (hipStream_t)stream);
  return r == GQA_OK ? ok() : r;
}

gqa_status gqa_layer_forward_noalloc(const gqa_config* cfg, int32_t batch, int32_t q_len,
                                     const void* x, const void* w_qkv, const void* q_norm_w,
                                     const void* k_norm_w, const void* w_o, void* k_cache,
                                     void* v_cache, int32_t kv_capacity, const int32_t* cache_len,
                                     void* out, void* stream) {
  gqa_config c;
  Shape s;
  gqa_status r = check_layer_call(cfg, batch, q_len, x, w_qkv, q_norm_w, k_norm_w, w_o, k_cache,
                                  v_cache, kv_capacity, out, &c, &s);
  if (r != GQA_OK || batch == 0 || q_len == 0) return r;
  const size_t need = ws_layer(s, batch, q_len, kv_capacity);
  if (need > kScratchBytes)
    return fail(GQA_ERR_WORKSPACE_TOO_SMALL,
                "gqa_layer_forward_noalloc: this call needs %zu bytes of scratch, more than the "
                "library's static %zu (use gqa_layer_forward with a workspace)",
                need, (size_t)kScratchBytes);
  void* scr = nullptr;
  if ((r = scratch_of_current_device(&scr)) != GQA_OK) return r;
  r = run_layer(c, s, batch, q_len, x, w_qkv, q_norm_w, k_norm_w, w_o, k_cache, v_cache,
                kv_capacity, cache_len, out, scr, (hipStream_t)stream);
  return r == GQA_OK ? ok() : r;
}

}  // extern "C"

namespace {

gqa_status run_layer(const gqa_config& c, const Shape& s, int batch, int q_len, const void* x,
                     const void* w_qkv, const void* q_norm_w, const void* k_norm_w,
                     const void* w_o, void* k_cache, void* v_cache, int kv_capacity,
                     const int32_t* cache_len, void* out, void* workspace, hipStream_t st) {
  gqa_status r;
  const size_t T = (size_t)batch * q_len;
  char* w = static_cast<char*>(workspace);
  void* ws_q = w;
  w += ws_qkv(s, batch, q_len);
  void* qbuf = w;
  w += align_up(T * s.Hq * s.d * esize(s));
  void* obuf = w;
  w += align_up(T * s.Hq * s.d * esize(s) * (s.o_split ? 2 : 1));
  void* ws_a = w;
  w += ws_attn(s, batch, q_len, kv_capacity);
  // o as fp16: W_o as fp16 too, converted once per call, or (few tokens)
  // rounded inside the product
  const bool w_cvt = oproj_rounds_w(s, (long long)T);
  void* wo16 = s.o_f16 && !w_cvt ? w : nullptr;
  r = run_qkv(c, s, batch, q_len, x, w_qkv, q_norm_w, k_norm_w, cache_len, qbuf, k_cache, v_cache,
              kv_capacity, ws_q, st);
  if (r != GQA_OK) return r;
  r = run_attn(c, s, batch, q_len, qbuf, k_cache, v_cache, cache_len, q_len, kv_capacity, obuf,
               s.o_split, ws_a, st, nullptr, s.o_f16);
  if (r != GQA_OK) return r;
  if (wo16) {
    r = check_launch(gqa::launch_cvt_bf16_f16(static_cast<const __bf16*>(w_o), wo16,
                                              (long long)s.H * s.Hq * s.d, st),
                     "W_o to fp16");
    if (r != GQA_OK) return r;
  }
  // few tokens: the projection's workspace, free again, holds o_proj's partial products
  return run_oproj(s, (int)T, obuf, s.o_split, w_o, out, st,
                   use_fused_qkv(s, (long long)T)
                       ? nullptr
                       : static_cast<char*>(ws_q) + skinny_part_offset(s, T),
                   wo16, w_cvt);
}

}  // namespace

extern "C" {

gqa_status gqa_layer_forward_train(const gqa_config* cfg, int32_t batch, int32_t q_len,
                                   const void* x, const void* w_qkv, const void* q_norm_w,
                                   const void* k_norm_w, const void* w_o, const gqa_saved* saved,
                                   void* out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  gqa_config c;
  Shape s;
  gqa_status r = resolve(cfg, &c, &s);
  if (r != GQA_OK) return r;
  if ((r = check_train(c, s)) != GQA_OK) return r;
  if ((r = check_common(s, batch, q_len, q_len)) != GQA_OK) return r;
  if (batch == 0 || q_len == 0) return ok();
  if (!x || !w_qkv || !w_o || !out || !saved)
    return fail(GQA_ERR_INVALID_ARG, "x, w_qkv, w_o, saved and out must be non-null");
  if (!saved->qkv || !saved->q || !saved->k || !saved->v || !saved->o || !saved->lse)
    return fail(GQA_ERR_INVALID_ARG, "every buffer of saved must be non-null");
  if (c.qk_norm && (!q_norm_w || !k_norm_w))
    return fail(GQA_ERR_INVALID_ARG, "qk_norm is on but a norm weight is null");
  const size_t need = rope_table_bytes(s, (size_t)q_len);
  if (!workspace || workspace_bytes < need)
    return fail(GQA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                workspace_bytes);
  const int T = batch * q_len;
  hipStream_t st = (hipStream_t)stream;
  if (use_fused_qkv(s, T)) {
    // projection with the norm + RoPE epilogue, which also keeps the fp32
    // projection for the backward
    r = run_qkv(c, s, batch, q_len, x, w_qkv, q_norm_w, k_norm_w, nullptr, saved->q, saved->k,
                saved->v, q_len, workspace, st, saved->qkv);
    if (r != GQA_OK) return r;
    r = run_attn(c, s, batch, q_len, saved->q, saved->k, saved->v, nullptr, q_len, q_len,
                 saved->o, false, nullptr, st, saved->lse);
    if (r != GQA_OK) return r;
    r = run_oproj(s, T, saved->o, false, w_o, out, st);
    return r == GQA_OK ? ok() : r;
  }
  // fused projection in fp32 (kept), then norm + RoPE + head-major scatter
  gqa::GemmArgs g{};
  g.W = static_cast<const __bf16*>(w_qkv);
  g.X = static_cast<const __bf16*>(x);
  g.N = s.n_qkv;
  g.M = T;
  g.K = s.H;
  g.out = saved->qkv;
  g.out_f32 = 1;
  r = use_skinny(s, T) ? check_launch(gqa::launch_gemm_skinny_bf16(g, st), "qkv projection")
                       : check_launch(gqa::launch_gemm_plain_bf16(g, st), "qkv projection");
  if (r != GQA_OK) return r;
  float2* table = static_cast<float2*>(workspace);
  r = check_launch(
      gqa::launch_rope_table(table, nullptr, q_len, q_len, s.rot / 2, (double)c.rope_theta, st),
      "rope table");
  if (r != GQA_OK) return r;
  gqa::NormRopeRowsArgs n{};
  n.y = saved->qkv;
  n.q_norm_w = static_cast<const __bf16*>(q_norm_w);
  n.k_norm_w = static_cast<const __bf16*>(k_norm_w);
  n.rope = table;
  n.q = static_cast<__bf16*>(saved->q);
  n.k_cache = static_cast<__bf16*>(saved->k);
  n.v_cache = static_cast<__bf16*>(saved->v);
  n.B = batch;
  n.L = q_len;
  n.Hq = s.Hq;
  n.Hkv = s.Hkv;
  n.d = s.d;
  n.rot = s.rot;
  n.cap = q_len;
  n.qk_norm = c.qk_norm;
  n.eps = c.rms_eps;
  if ((r = check_launch(gqa::launch_normrope_fwd_rows(n, st), "norm + rope")) != GQA_OK) return r;
  r = run_attn(c, s, batch, q_len, saved->q, saved->k, saved->v, nullptr, q_len, q_len, saved->o,
               false, nullptr, st, saved->lse);
  if (r != GQA_OK) return r;
  r = run_oproj(s, T, saved->o, false, w_o, out, st);
  return r == GQA_OK ? ok() : r;
}

gqa_status gqa_layer_backward(const gqa_config* cfg, int32_t batch, int32_t q_len, const void* x,
                              const void* w_qkv, const void* q_norm_w, const void* k_norm_w,
                              const void* w_o, const gqa_saved* saved, const void* dout,
                              const gqa_grads* grads, void* workspace, size_t workspace_bytes,
                              void* stream) {
  gqa_config c;
  Shape s;
  gqa_status r = resolve(cfg, &c, &s);
  if (r != GQA_OK) return r;
  if ((r = check_train(c, s)) != GQA_OK) return r;
  if ((r = check_common(s, batch, q_len, q_len)) != GQA_OK) return r;
  if (batch == 0 || q_len == 0) return ok();
  if (!x || !w_qkv || !w_o || !saved || !dout || !grads)
    return fail(GQA_ERR_INVALID_ARG, "x, w_qkv, w_o, saved, dout and grads must be non-null");
  if (!saved->qkv || !saved->q || !saved->k || !saved->v || !saved->o || !saved->lse)
    return fail(GQA_ERR_INVALID_ARG, "every buffer of saved must be non-null");
  if (!grads->dx || !grads->dw_qkv || !grads->dw_o)
    return fail(GQA_ERR_INVALID_ARG, "grads->dx, dw_qkv and dw_o must be non-null");
  if (c.qk_norm && (!q_norm_w || !k_norm_w || !grads->dq_norm_w || !grads->dk_norm_w))
    return fail(GQA_ERR_INVALID_ARG, "qk_norm is on but a norm weight or its gradient is null");
  const BwdLayout lay = bwd_layout(s, batch, q_len);
  if (!workspace || workspace_bytes < lay.total)
    return fail(GQA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", lay.total,
                workspace_bytes);
  char* w = static_cast<char*>(workspace);
  auto bfp = [&](size_t off) { return reinterpret_cast<__bf16*>(w + off); };
  auto f32p = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
  hipStream_t st = (hipStream_t)stream;
  const int T = batch * q_len;
  const int qw = s.Hq * s.d;
  const __bf16* dout_b = static_cast<const __bf16*>(dout);
  const __bf16* x_b = static_cast<const __bf16*>(x);

  // o_proj: dW_o = dout^T o (token-chunked), dO = dout W_o
  r = check_launch(gqa::launch_transpose_bf16(dout_b, T, s.H, lay.so.Rc, bfp(lay.doutT), st),
                   "transpose dout");
  if (r != GQA_OK) return r;
  r = check_launch(gqa::launch_transpose_bf16(static_cast<const __bf16*>(saved->o), T, qw, lay.so.Rc,
                                              bfp(lay.oT), st),
                   "transpose o");
  if (r != GQA_OK) return r;
  r = weight_grad(bfp(lay.doutT), bfp(lay.oT), s.H, qw, lay.so, f32p(lay.dwo_part), grads->dw_o,
                  st, "dW_o");
  if (r != GQA_OK) return r;
  r = check_launch(gqa::launch_transpose_bf16(static_cast<const __bf16*>(w_o), s.H, qw, s.H,
                                              bfp(lay.woT), st),
                   "transpose W_o");
  if (r != GQA_OK) return r;
  r = plain_gemm(dout_b, bfp(lay.woT), T, qw, s.H, bfp(lay.dO), 0, st, "dO");
  if (r != GQA_OK) return r;

  // attention: dq, dk, dv (bf16, head-major)
  gqa::AttnBwdArgs a{};
  a.d = s.d;
  a.q = static_cast<const __bf16*>(saved->q);
  a.k = static_cast<const __bf16*>(saved->k);
  a.v = static_cast<const __bf16*>(saved->v);
  a.o = static_cast<const __bf16*>(saved->o);
  a.dO = bfp(lay.dO);
  a.lse = saved->lse;
  a.D = f32p(lay.D);
  a.lse2 = f32p(lay.lse2);
  a.dq = bfp(lay.dq);
  a.dk = bfp(lay.dk);
  a.dv = bfp(lay.dv);
  a.B = batch;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.L = q_len;
  a.causal = c.causal;
  const double scale = 1.0 / sqrt((double)s.d);
  a.scale = (float)scale;
  a.scale_log2 = (float)(scale * 1.4426950408889634);
  if ((r = prefill_split(s, q_len, &a.hpw, &a.pb, &a.n_hsub, &a.n_qtiles)) != GQA_OK) return r;
  if ((r = check_launch(gqa::launch_attn_bwd_bf16(a, st), "attention backward")) != GQA_OK)
    return r;

  // RoPE and QK-norm: dy = gradient of the fused projection output
  float2* table = reinterpret_cast<float2*>(w + lay.rope);
  r = check_launch(gqa::launch_rope_table(table, nullptr, q_len, q_len, s.rot / 2,
                                          (double)c.rope_theta, st),
                   "rope table");
  if (r != GQA_OK) return r;
  gqa::NormRopeBwdArgs n{};
  n.dq = a.dq;
  n.dk = a.dk;
  n.dv = a.dv;
  n.y = saved->qkv;
  n.q_norm_w = static_cast<const __bf16*>(q_norm_w);
  n.k_norm_w = static_cast<const __bf16*>(k_norm_w);
  n.rope = table;
  n.dy = bfp(lay.dy);
  n.dyT = bfp(lay.dyT);
  n.Rc = lay.sq.Rc;
  n.dgamma_part = f32p(lay.gpart);
  n.B = batch;
  n.L = q_len;
  n.Hq = s.Hq;
  n.Hkv = s.Hkv;
  n.d = s.d;
  n.rot = s.rot;
  n.qk_norm = c.qk_norm;
  n.eps = c.rms_eps;
  if ((r = check_launch(gqa::launch_normrope_bwd(n, st), "norm + rope backward")) != GQA_OK)
    return r;
  if (c.qk_norm) {
    r = check_launch(gqa::launch_dgamma_reduce(f32p(lay.gpart), lay.gblocks, s.d,
                                               f32p(lay.gstage), grads->dq_norm_w,
                                               grads->dk_norm_w, st),
                     "norm weight gradients");
    if (r != GQA_OK) return r;
  }

  // fused projection: dW_qkv = dy^T x (token-chunked; dy^T came from the
  // norm/RoPE backward), dx = dy W_qkv
  r = check_launch(gqa::launch_transpose_bf16(x_b, T, s.H, lay.sq.Rc, bfp(lay.xT), st),
                   "transpose x");
  if (r != GQA_OK) return r;
  r = weight_grad(bfp(lay.dyT), bfp(lay.xT), s.n_qkv, s.H, lay.sq, f32p(lay.dwq_part),
                  grads->dw_qkv, st, "dW_qkv");
  if (r != GQA_OK) return r;
  r = check_launch(gqa::launch_transpose_bf16(static_cast<const __bf16*>(w_qkv), s.n_qkv, s.H,
                                              s.n_qkv, bfp(lay.wqT), st),
                   "transpose W_qkv");
  if (r != GQA_OK) return r;
  r = plain_gemm(bfp(lay.dy), bfp(lay.wqT), T, s.H, s.n_qkv, grads->dx, 0, st, "dx");
  return r == GQA_OK ? ok() : r;
}

const char* gqa_status_string(gqa_status s) {
  switch (s) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_INVALID_ARG: return "GQA_ERR_INVALID_ARG";
    case GQA_ERR_HEAD_DIM_INDIVISIBLE: return "GQA_ERR_HEAD_DIM_INDIVISIBLE";
    case GQA_ERR_GROUP_INDIVISIBLE: return "GQA_ERR_GROUP_INDIVISIBLE";
    case GQA_ERR_ODD_HEAD_DIM: return "GQA_ERR_ODD_HEAD_DIM";
    case GQA_ERR_UNSUPPORTED_HEAD_DIM: return "GQA_ERR_UNSUPPORTED_HEAD_DIM";
    case GQA_ERR_UNSUPPORTED_DTYPE: return "GQA_ERR_UNSUPPORTED_DTYPE";
    case GQA_ERR_UNSUPPORTED_SHAPE: return "GQA_ERR_UNSUPPORTED_SHAPE";
    case GQA_ERR_WORKSPACE_TOO_SMALL: return "GQA_ERR_WORKSPACE_TOO_SMALL";
    case GQA_ERR_CAPACITY: return "GQA_ERR_CAPACITY";
    case GQA_ERR_HIP: return "GQA_ERR_HIP";
  }
  return "GQA_ERR_UNKNOWN";
}

const char* gqa_last_error(void) { return g_err; }

#ifdef GQA_LDS_POISON
// Marks the LDS-poisoning debug build (its tests check that they run it).
int gqa_lds_poison_build(void) { return 1; }
#endif

}  // extern "C"
