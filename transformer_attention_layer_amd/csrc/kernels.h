// Internal launch interface between the C-ABI host code and the gfx950
// kernels.  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

// GEMM epilogue kinds: plain (bf16 or fp32 out), and the QKV projection's
// norm + RoPE + head-major scatter for head_dim 128, 64 and 256
enum { kEpiPlain = 0, kEpiQKV = 1, kEpiPlainF32 = 2, kEpiQKV64 = 3, kEpiQKV256 = 4 };
constexpr bool is_qkv_epi(int e) { return e == kEpiQKV || e == kEpiQKV64 || e == kEpiQKV256; }

// C^T[n, m] = sum_k W[n, k] X[m, k]  (bf16 in, fp32 accumulate)
struct GemmArgs {
  const __bf16* W;  // [N, K]
  const __bf16* X;  // [M, K]
  int N, M, K;
  // plain epilogues only: `batch` independent products (0 counts as 1), member z
  // at W + z sW, X + z sX, out + z sOut (elements)
  int batch;
  long long sW, sX, sOut;
  // plain epilogue: out[m, n], bf16 or (out_f32) fp32
  void* out;
  int out_f32;
  int w_kmod;       // > 0: W column k % w_kmod (W read twice along K for a hi | lo X)
  int f16;          // plain epilogues and few-token GEMM: W and X hold fp16 values
  // QKV epilogue (head_dim 128)
  __bf16* q;        // [B, Hq, L, 128]
  __bf16* k_cache;  // [B, Hkv, cap, 128]
  __bf16* v_cache;
  const __bf16* q_norm_w;
  const __bf16* k_norm_w;
  const float2* rope;     // [rows, rot / 2] (cos, sin); rows = T if start_pos else L
  const int* start_pos;   // [B] or null
  int L, Hq, Hkv, cap, qk_norm;
  int rot;                // rotary width: head_dim 128: 128 or 64; 64: 64 or 32; 256: 256
  int hd;                 // head_dim of the QKV epilogue: 128 (0 counts as 128), 64 or 256
  float eps;
  float* y_raw;           // optional: [M, N] fp32 projection before norm and RoPE (QKV
                          // epilogues: the columns of the normalised heads only)
  // few-token GEMM only: K split over ksplit workgroups (<= 1: none), whose
  // fp32 partial products go to part [ksplit][M][N] and are then summed into out
  int ksplit;
  float* part;
  int keep_parts;  // ksplit > 1: leave the partial products for the consumer to sum
  // few-token GEMM with f16 set and skinny_lds_ok: W holds bf16, rounded to
  // fp16 as its fragments are read (the same rounding as launch_cvt_bf16_f16)
  int w_bf16_to_f16;
  // few-token GEMM with skinny_lds_ok, optional: also fill the RoPE table
  // [rope_rows, rope_half] as launch_rope_table would (its workgroups'
  // first threads, while their first loads are in flight)
  float2* rope_table;
  const int* rope_start_pos;
  int rope_rows, rope_L, rope_half;
  double rope_theta;
};
// K splits for the few-token GEMM of M tokens that bring its workgroups to
// about one or two per CU
int skinny_ksplit(int N, int K, int M);
// the few-token GEMM's LDS-streamed kernel applies (K and a hi | lo X's W
// width multiples of 64)
bool skinny_lds_ok(int K, int w_kmod);

struct AttnArgs {
  int d;            // head_dim: 64, 128 or 256
  const __bf16* q;  // [B, Hq, Lq, d]
  const __bf16* k;  // [B, Hkv, cap, d]
  const __bf16* v;
  const unsigned char* k8;  // FP8 (E4M3) caches [B, Hkv, cap, d] (decode only), else null
  const unsigned char* v8;
  float v_scale;            // multiplies the output (FP8 V scale; 1 otherwise)
  __bf16* o;        // [B, Lq, Hq * d], or [B, Lq, 2, Hq * d] (hi | lo) when o_split
  int o_split;
  int o_f16;        // o holds fp16 values (rounded to nearest even) instead of bf16
  const int* kv_base;  // kv_len[b] = (kv_base ? kv_base[b] : 0) + kv_add, clamped to [0, cap]
  int kv_add;
  int B, Hq, Hkv, G, Lq, cap, causal;
  float scale_log2;    // d^-0.5 * log2(e)
  // prefill work split
  int hpw, pb, n_qtiles, n_hsub;
  // split-KV decode
  float* part_o;       // [B, Hkv, n_splits, G * Lq, d]
  float2* part_ml;     // [B, Hkv, n_splits, G * Lq] (running max in log2 units, sum)
  int n_splits, chunk;
  int rotate;          // bf16 decode: each wave starts its chunk at a tile of its own
  float* lse;          // prefill, optional: [B, Hq, Lq] natural log of each row's softmax denominator
};

hipError_t launch_rope_table(float2* table, const int* start_pos, int rows, int L, int half,
                             double theta, hipStream_t stream);
hipError_t launch_gemm_qkv_bf16(const GemmArgs& args, hipStream_t stream);
hipError_t launch_gemm_plain_bf16(const GemmArgs& args, hipStream_t stream);

hipError_t launch_attn_prefill_bf16(const AttnArgs& args, hipStream_t stream);

// Attention backward (bf16 matrix cores, head_dim 64 or 128, no cache:
// keys are the L tokens of each sequence).
struct AttnBwdArgs {
  int d;
  const __bf16* q;   // [B, Hq, L, d] after norm and RoPE
  const __bf16* k;   // [B, Hkv, L, d]
  const __bf16* v;   // [B, Hkv, L, d]
  const __bf16* o;   // [B, L, Hq * d] forward attention output
  const __bf16* dO;  // [B, L, Hq * d] its gradient
  const float* lse;  // [B, Hq, L] natural log of each row's softmax denominator
  float* D;          // [B, Hq, L] rowsum(dO * o): written by the dQ kernel
  float* lse2;       // [B, Hq, L] lse in log2 units (+inf: no visible key): written by the dQ kernel
  __bf16* dq;        // [B, Hq, L, d]
  __bf16* dk;        // [B, Hkv, L, d]
  __bf16* dv;        // [B, Hkv, L, d]
  int B, Hq, Hkv, G, L, causal;
  float scale;       // d^-0.5
  float scale_log2;  // scale * log2(e)
  int hpw, pb, n_qtiles, n_hsub;  // dQ kernel work split (as the forward prefill)
};
hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& args, hipStream_t stream);

// QK-norm + RoPE per (token, head) row of an fp32 projection output with
// bf16 outputs, head_dim 64, 128 or 256 and a rotary width that is a
// multiple of 8 (normrope_rows_ok); cos / sin from a rope_table.
struct NormRopeRowsArgs {
  const float* y;     // [T, n_qkv]
  const float* part;  // or, when set, `parts` partial products [parts][T][n_qkv] summed in order
  int parts;
  const __bf16* q_norm_w;
  const __bf16* k_norm_w;
  const float2* rope;    // [rows, rot / 2]: rows = T (indexed by token row) with start_pos, else L
  const int* start_pos;  // [B] or null
  __bf16* q;             // [B, Hq, L, d]
  __bf16* k_cache;       // [B, Hkv, cap, d]
  __bf16* v_cache;
  int B, L, Hq, Hkv, d, rot, cap, qk_norm;
  float eps;
};
bool normrope_rows_ok(int d, int rot);
hipError_t launch_normrope_fwd_rows(const NormRopeRowsArgs& args, hipStream_t stream);

// Backward through QK-norm and RoPE (same shapes and limits): per (token,
// head of the fused projection) the gradient of the projection output, bf16
// [T, n_qkv], and per-block partial sums of the norm-weight gradients.
struct NormRopeBwdArgs {
  const __bf16* dq;  // [B, Hq, L, d]
  const __bf16* dk;  // [B, Hkv, L, d]
  const __bf16* dv;  // [B, Hkv, L, d]
  const float* y;    // [T, n_qkv] projection output before norm and RoPE
  const __bf16* q_norm_w;
  const __bf16* k_norm_w;
  const float2* rope;  // [L, rot / 2] (cos, sin) of position t
  __bf16* dy;          // [T, n_qkv]
  __bf16* dyT;         // token chunks [ceil(T / Rc)][n_qkv][Rc] of dy^T, zero past T
  int Rc;              // tokens per chunk, a multiple of 64
  float* dgamma_part;  // [normrope_bwd_blocks][2][d]: q then k weight-gradient partial sums
  int B, L, Hq, Hkv, d, rot, qk_norm;
  float eps;
};
int normrope_bwd_blocks(long long T, int Rc, int nh);
hipError_t launch_normrope_bwd(const NormRopeBwdArgs& args, hipStream_t stream);
// dq_w[j] = sum over blocks of part[blk][0][j], dk_w[j] likewise with
// [blk][1][j] (fp32, fixed order); `stage` holds dgamma_stage_floats(d)
// floats of scratch.
size_t dgamma_stage_floats(int d);
hipError_t launch_dgamma_reduce(const float* part, int blocks, int d, float* stage, float* dq_w,
                                float* dk_w, hipStream_t stream);
// bf16 transpose into row chunks: in [R, C] (row-major) -> out[s][C][Rc] for
// s < ceil(R / Rc), out[s][c][r'] = in[s Rc + r'][c], zero where s Rc + r' >= R;
// Rc % 8 == 0 and C % 8 == 0.
hipError_t launch_transpose_bf16(const __bf16* in, int R, int C, int Rc, __bf16* out,
                                 hipStream_t stream);
// out[i] = sum_s part[s * n + i], fp32, n % 4 == 0
hipError_t launch_sum_partials(const float* part, int S, long long n, float* out,
                               hipStream_t stream);
hipError_t launch_attn_decode_bf16(const AttnArgs& args, hipStream_t stream);

// fp32 path (any even head_dim up to 256)
struct F32Args {
  const float* x; const float* w; float* y;  // y[M, N] = x[M, K] w[N, K]^T
  int M, N, K;
};
hipError_t launch_gemm_f32(const F32Args& args, hipStream_t stream);

// Per-(token, head) QK-norm + RoPE + scatter of an fp32 projection output;
// weights and outputs are fp32 or (bf16 != 0) bf16.
struct NormRopeArgs {
  const float* y;     // [T, (Hq + 2 Hkv) d] projection output
  const void* q_norm_w; const void* k_norm_w;
  const int* start_pos;
  void* q; void* k_cache; void* v_cache;
  int B, L, Hq, Hkv, d, rot, cap, qk_norm, bf16;
  int kv_fp8;                       // caches take E4M3 codes of x * inv_scale
  float inv_k_scale, inv_v_scale;
  float eps; double theta;
};
hipError_t launch_normrope(const NormRopeArgs& args, hipStream_t stream);

// few-token (decode) projections: out[m, n] = sum_k X[m, k] W[n, k], fp32 or bf16 out
hipError_t launch_gemm_skinny_bf16(const GemmArgs& args, hipStream_t stream);

// One-wave-per-query attention over fp32 or (bf16 != 0) bf16 q / caches / o,
// any even head_dim up to 256; o_split as in AttnArgs (bf16 only).
struct F32AttnArgs {
  const void* q; const void* k; const void* v; void* o;
  const int* kv_base; int kv_add;
  int B, Hq, Hkv, Lq, cap, d, causal, bf16, o_split, o_f16;
  float scale;
};

// out[i] = fp16(in[i]) (bf16 -> fp16, round to nearest even; n % 8 == 0)
hipError_t launch_cvt_bf16_f16(const __bf16* in, void* out, long long n, hipStream_t stream);
hipError_t launch_attn_vec(const F32AttnArgs& args, hipStream_t stream);

}  // namespace gqa
