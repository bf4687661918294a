// Internal launch interface between the C-ABI host code and the gfx950
// kernels.  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

enum { kEpiPlain = 0, kEpiQKV = 1, kEpiPlainF32 = 2 };  // GEMM epilogue kinds

// C^T[n, m] = sum_k W[n, k] X[m, k]  (bf16 in, fp32 accumulate)
struct GemmArgs {
  const __bf16* W;  // [N, K]
  const __bf16* X;  // [M, K]
  int N, M, K;
  // plain epilogue: out[m, n], bf16 or (out_f32) fp32
  void* out;
  int out_f32;
  int w_kmod;       // > 0: W column k % w_kmod (W read twice along K for a hi | lo X)
  // QKV epilogue (head_dim 128)
  __bf16* q;        // [B, Hq, L, 128]
  __bf16* k_cache;  // [B, Hkv, cap, 128]
  __bf16* v_cache;
  const __bf16* q_norm_w;
  const __bf16* k_norm_w;
  const float2* rope;     // [rows, rot / 2] (cos, sin); rows = T if start_pos else L
  const int* start_pos;   // [B] or null
  int L, Hq, Hkv, cap, qk_norm;
  int rot;                // rotary width: 128 (full) or 64 (first half of each head)
  float eps;
};

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
  const int* kv_base;  // kv_len[b] = (kv_base ? kv_base[b] : 0) + kv_add, clamped to [0, cap]
  int kv_add;
  int B, Hq, Hkv, G, Lq, cap, causal;
  float scale_log2;    // d^-0.5 * log2(e)
  // prefill work split
  int hpw, pb, n_qtiles, n_hsub;
  // split-KV decode
  float* part_o;       // [B, Hkv, n_splits, 32, d]
  float2* part_ml;     // [B, Hkv, n_splits, 32] (running max in log2 units, sum)
  int n_splits, chunk;
};

hipError_t launch_rope_table(float2* table, const int* start_pos, int rows, int L, int half,
                             double theta, hipStream_t stream);
hipError_t launch_gemm_qkv_bf16(const GemmArgs& args, hipStream_t stream);
hipError_t launch_gemm_plain_bf16(const GemmArgs& args, hipStream_t stream);

hipError_t launch_attn_prefill_bf16(const AttnArgs& args, hipStream_t stream);
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
  int B, Hq, Hkv, Lq, cap, d, causal, bf16, o_split;
  float scale;
};
hipError_t launch_attn_vec(const F32AttnArgs& args, hipStream_t stream);

}  // namespace gqa
