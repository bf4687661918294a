/*
 * gqa.h -- C ABI of the MI355X (gfx950) library for the forward pass of a
 * grouped-query attention layer whose head_dim is set explicitly, and for
 * its backward pass (gqa_layer_forward_train / gqa_layer_backward).
 *
 * The layer (tutorial "Multi-Head and Grouped-Query Attention (Full Layer)",
 * section 4, Attention.__call__ steps 1-7; GPT-NeoX issue "Support explicit
 * attention head_dim independent of hidden_size / num_attention_heads"):
 *
 *   y        = x W_qkv^T                 W_qkv rows: Q | K | V, (Hq+2Hkv)*d
 *   q, k     = RoPE(RMSNorm_head(q)), RoPE(RMSNorm_head(k))   (QK-norm optional)
 *   o        = softmax(q k^T * d^-0.5 + causal mask) v,  query head h -> KV head h / (Hq/Hkv)
 *   out      = flatten(o) W_o^T          flatten to Hq*d, W_o is [hidden, Hq*d]
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor arguments are DEVICE pointers owned by the caller; the
 *   library never allocates or frees device memory.  Scratch space comes
 *   from the caller's `workspace` (size from gqa_workspace_bytes, at least
 *   256-byte aligned), except for gqa_layer_forward_noalloc, which uses a
 *   static device array of the library's own.  Inputs are read-only;
 *   outputs must not alias inputs.
 * - One element type per call, cfg->dtype: GQA_BF16 (bf16 storage, fp32
 *   accumulation and fp32 norm/RoPE/softmax) or GQA_F32.
 * - All tensors are dense row-major with the shapes given below.  Rows of x,
 *   weights and outputs must start 16-byte aligned (hidden_size % 8 == 0).
 * - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *   enqueues work on it and never synchronizes.
 * - Validation runs on the host before any launch; on error nothing is
 *   launched and the status says why (gqa_last_error() gives detail, per
 *   thread).  A launch failure returns GQA_ERR_HIP.
 * - batch == 0 or q_len == 0 is a no-op returning GQA_OK.
 * - Supported head_dim: any even value from 2 to 256; others return
 *   GQA_ERR_UNSUPPORTED_HEAD_DIM.  With GQA_BF16, head_dim 64, 128 and 256
 *   run the matrix-core attention; 128 also fuses QK-norm and RoPE into the
 *   QKV GEMM (other sizes take a separate norm/RoPE pass); any other size
 *   runs a vector-unit attention (correct, much slower).  bf16 also needs num_heads*head_dim and
 *   (num_heads + 2*num_kv_heads)*head_dim to be multiples of 8, and o_split
 *   needs num_heads*head_dim to be a multiple of 32 (GQA_ERR_UNSUPPORTED_SHAPE).
 * - The training pair takes GQA_BF16 with head_dim 64 or 128 and a rotary
 *   width that is a multiple of 8; see its declarations below.
 */
#ifndef GQA_H_
#define GQA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARG = 1,          /* null pointer, negative size, bad flag */
  GQA_ERR_HEAD_DIM_INDIVISIBLE = 2, /* head_dim unset and hidden % Hq != 0 */
  GQA_ERR_GROUP_INDIVISIBLE = 3,    /* Hq % Hkv != 0 */
  GQA_ERR_ODD_HEAD_DIM = 4,         /* RoPE needs an even head_dim */
  GQA_ERR_UNSUPPORTED_HEAD_DIM = 5, /* no kernel tile for this head_dim */
  GQA_ERR_UNSUPPORTED_DTYPE = 6,
  GQA_ERR_UNSUPPORTED_SHAPE = 7,    /* e.g. hidden_size % 8 != 0 */
  GQA_ERR_WORKSPACE_TOO_SMALL = 8,
  GQA_ERR_CAPACITY = 9,             /* kv_capacity too small for the call */
  GQA_ERR_HIP = 10                  /* a HIP launch failed */
} gqa_status;

typedef enum { GQA_F32 = 0, GQA_BF16 = 1 } gqa_dtype;

/*
 * Layer configuration (GPT-NeoX issue, "Proposed configuration behavior" and
 * "Proposed implementation"; tutorial section 4 constructor arguments).
 *   num_kv_heads == 0  -> Hkv = Hq (plain multi-head attention)
 *   head_dim == 0      -> d = hidden_size / Hq, which then must divide evenly;
 *                         an explicit head_dim needs no divisibility.
 *   qk_norm            -> per-head RMSNorm of q and k before RoPE
 *                         (tutorial section 3), weights [d] each.
 *   causal             -> key j is visible to a query at position p iff j <= p.
 */
typedef struct {
  int32_t hidden_size;
  int32_t num_heads;     /* Hq */
  int32_t num_kv_heads;  /* Hkv, 0 = Hq */
  int32_t head_dim;      /* d, 0 = hidden_size / Hq */
  float rope_theta;
  float rms_eps;
  int32_t qk_norm;
  int32_t causal;
  int32_t dtype;         /* gqa_dtype */
  int32_t out_f32;       /* 1: the o_proj output (gqa_o_proj, gqa_layer_forward)
                            is written as fp32, straight from the fp32
                            accumulator; 0: in `dtype` */
  int32_t o_split;       /* bf16 only, gqa_layer_forward only.  1: the attention
                            output reaches o_proj as a bf16 pair hi + lo
                            (lo = bf16(o - hi)), about 16 significant bits, so
                            its rounding stays out of the output; costs one more
                            o_proj pass.  0: one bf16 value, the tutorial's cast
                            of the attention result to the input dtype. */
  int32_t rotary_dim;    /* r, 0 = head_dim.  Partial rotary (GPT-NeoX issue,
                            "Scaling and RoPE": RoPE is built at the effective
                            head_dim and keeps the rotary_pct option, which the
                            page does not define; read here as follows): the
                            first r entries of each q and k head rotate as
                            a width-r rotate-half RoPE (entry i < r/2 pairs with
                            i + r/2, angle pos * theta^(-2i/r)); entries r ..
                            head_dim-1 pass through.  Must be even and at most
                            head_dim, else GQA_ERR_INVALID_ARG. */
  int32_t kv_fp8;        /* 1: the K and V caches hold FP8 codes, one byte per
                            element ("Head Dimension" article, section 5.2:
                            K, V cached in FP8 precision).  Format: OCP E4M3
                            (sign, 4 exponent bits with bias 7, 3 mantissa
                            bits; largest finite 448; 0x7F/0xFF NaN).  An
                            entry stands for value(code) * k_scale (K) or
                            * v_scale (V).  Appending x (qkv_proj_normrope,
                            gqa_layer_forward) stores the code nearest to
                            x / scale, ties to even, magnitudes above 448
                            saturated; attention reads the stored values.
                            bf16 with head_dim 64 or 128 only
                            (GQA_ERR_UNSUPPORTED_DTYPE / _HEAD_DIM), and
                            gqa_attn_core / gqa_layer_forward
                            only for calls whose Hq/Hkv * q_len <= 32 (decode
                            and short chunks); else GQA_ERR_UNSUPPORTED_SHAPE.
                            0: the caches hold `dtype` values. */
  float k_scale;         /* kv_fp8 only: per-tensor scales, 0 = 1.0; positive */
  float v_scale;         /* and finite, else GQA_ERR_INVALID_ARG */
  int32_t o_fp16;        /* bf16 only (ignored for GQA_F32), gqa_layer_forward
                            and gqa_layer_forward_noalloc only.  1: the
                            attention output reaches o_proj as fp16 (11
                            significant bits, rounded to nearest even) and
                            o_proj runs on the fp16 matrix cores with W_o
                            converted to fp16 (exactly, for weights from 2^-17
                            to 65504 in magnitude) in the workspace: one
                            o_proj pass instead of o_split's two.  Values past
                            65504 in magnitude (o or W_o) become infinities, so
                            the output turns non-finite rather than wrong.
                            Cannot be combined with o_split
                            (GQA_ERR_INVALID_ARG). */
} gqa_config;

/* Host only (no device needed): copy *in to *out with num_kv_heads and
 * head_dim resolved, after every check above.  Returns the first violated
 * rule. */
gqa_status gqa_resolve(const gqa_config* in, gqa_config* out);

/* Which entry point a workspace is sized for. */
typedef enum {
  GQA_WS_QKV = 0, GQA_WS_ATTN = 1, GQA_WS_LAYER = 2, GQA_WS_OPROJ = 3,
  GQA_WS_TRAIN_FORWARD = 4, GQA_WS_BACKWARD = 5
} gqa_ws_kind;

/* Bytes of workspace the entry point `kind` needs for this call shape
 * (0 if the config is invalid).  Host only. */
size_t gqa_workspace_bytes(const gqa_config* cfg, int32_t batch, int32_t q_len,
                           int32_t kv_capacity, int32_t kind);

/*
 * Fused QKV projection + QK-norm + RoPE + head-major scatter (tutorial
 * section 4 steps 1-4; GPT-NeoX issue "Fused QKV projection").
 *   x        [batch, q_len, hidden]
 *   w_qkv    [(Hq + 2*Hkv) * d, hidden], rows Q | K | V
 *   q_norm_w, k_norm_w  [d] (ignored, may be NULL, when cfg->qk_norm == 0)
 *   start_pos [batch] int32 device array, or NULL for all zero: token t of
 *            sequence b sits at position start_pos[b] + t (RoPE angle) and
 *            its k, v go to cache row start_pos[b] + t.
 *   q        [batch, Hq, q_len, d]   (after norm and RoPE)
 *   k_cache, v_cache [batch, Hkv, kv_capacity, d]; only the rows above are
 *            written (k after norm and RoPE, v raw), as FP8 codes with
 *            cfg->kv_fp8.
 * The caller guarantees start_pos[b] + q_len <= kv_capacity.
 */
gqa_status qkv_proj_normrope(const gqa_config* cfg, int32_t batch, int32_t q_len,
                             const void* x, const void* w_qkv,
                             const void* q_norm_w, const void* k_norm_w,
                             const int32_t* start_pos, void* q, void* k_cache,
                             void* v_cache, int32_t kv_capacity,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Grouped attention core (tutorial section 4 step 6; GPT-NeoX issue
 * "Scaling and RoPE": scale = d^-0.5 of the effective head_dim).
 *   q        [batch, Hq, q_len, d]
 *   k_cache, v_cache [batch, Hkv, kv_capacity, d] (FP8 codes with
 *            cfg->kv_fp8)
 *   kv_len   [batch] int32 device array of valid key rows, or NULL for
 *            q_len.  Query i of sequence b sits at position
 *            kv_len[b] - q_len + i (bottom-right alignment) and, when
 *            causal, sees keys 0 .. that position.  Needs
 *            q_len <= kv_len[b] <= kv_capacity when causal.
 *   o        [batch, q_len, Hq * d]  (token-major: o_proj reads it directly)
 * Query head h reads KV head h / (Hq / Hkv).
 */
gqa_status gqa_attn_core(const gqa_config* cfg, int32_t batch, int32_t q_len,
                         const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* kv_len, int32_t kv_capacity, void* o,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Output projection (GPT-NeoX issue "Output projection"; tutorial section 4
 * step 7): out [tokens, hidden] = o [tokens, Hq*d] W_o^T, W_o [hidden, Hq*d].
 * out is fp32 when cfg->out_f32, else of cfg->dtype.
 */
gqa_status gqa_o_proj(const gqa_config* cfg, int32_t tokens, const void* o,
                      const void* w_o, void* out, void* stream);

/*
 * The whole layer forward: qkv_proj_normrope, then gqa_attn_core over the
 * cache, then gqa_o_proj.
 *   x        [batch, q_len, hidden]
 *   k_cache, v_cache [batch, Hkv, kv_capacity, d]: rows cache_len[b] ..
 *            cache_len[b] + q_len - 1 are written (tutorial step 5,
 *            update_and_fetch appends before attending); rows below are read.
 *   cache_len [batch] int32 device array or NULL (empty caches).
 *   out      [batch, q_len, hidden]  (the o_proj output; no residual add),
 *            fp32 when cfg->out_f32, else of cfg->dtype
 * Plain prefill: cache_len NULL and kv_capacity >= q_len.  Decode: q_len 1.
 */
gqa_status gqa_layer_forward(const gqa_config* cfg, int32_t batch, int32_t q_len,
                             const void* x, const void* w_qkv,
                             const void* q_norm_w, const void* k_norm_w,
                             const void* w_o, void* k_cache, void* v_cache,
                             int32_t kv_capacity, const int32_t* cache_len,
                             void* out, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * gqa_layer_forward without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): same arguments, outputs and errors as
 * gqa_layer_forward, and the same kernels, but the workspace is the
 * library's own static device array of 32 MiB (one per GPU, held until the
 * process ends).  The call allocates and frees nothing.  A call that needs
 * more than 32 MiB of workspace (gqa_workspace_bytes(..., GQA_WS_LAYER))
 * returns GQA_ERR_WORKSPACE_TOO_SMALL and launches nothing; a decode step
 * of 64 sequences against 32K-token caches needs about 14 MiB.  Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (two
 * streams, or two threads) race and give undefined results.  The array
 * keeps what the last call left; nothing in it needs to start at zero.
 */
gqa_status gqa_layer_forward_noalloc(const gqa_config* cfg, int32_t batch, int32_t q_len,
                                     const void* x, const void* w_qkv,
                                     const void* q_norm_w, const void* k_norm_w,
                                     const void* w_o, void* k_cache, void* v_cache,
                                     int32_t kv_capacity, const int32_t* cache_len,
                                     void* out, void* stream);

/*
 * Training: a forward that keeps what the backward reads, and the backward
 * (GPT-NeoX issue, "Tests and acceptance criteria": forward and backward
 * passes; "Attention head partitions: keep each head's dependencies
 * intact": gradients of the shared KV parameters).  No cache: the keys of
 * sequence b are its own q_len tokens at positions 0 .. q_len - 1.
 * Both need cfg->dtype GQA_BF16, head_dim 64 or 128, a rotary width that is
 * a multiple of 8, o_split 0 and kv_fp8 0 (else GQA_ERR_UNSUPPORTED_DTYPE /
 * _HEAD_DIM / _SHAPE).  All buffers are device memory owned by the caller;
 * every check runs on the host before any launch.
 */
typedef struct {
  float* qkv;  /* [batch, q_len, (Hq + 2*Hkv) * d]: the fused projection output
                  before QK-norm and RoPE, kept for the norm backward: only
                  the Q and K columns, and only with QK-norm on, are read,
                  and the other columns may be left unwritten */
  void* q;     /* [batch, Hq, q_len, d] after QK-norm and RoPE */
  void* k;     /* [batch, Hkv, q_len, d] after QK-norm and RoPE */
  void* v;     /* [batch, Hkv, q_len, d] */
  void* o;     /* [batch, q_len, Hq * d] attention output (the o_proj input) */
  float* lse;  /* [batch, Hq, q_len] natural log of each query row's softmax
                  denominator, sum_j exp(q . k_j * d^-0.5) over its visible keys */
} gqa_saved;

typedef struct {
  void* dx;          /* [batch, q_len, hidden], cfg->dtype */
  float* dw_qkv;     /* [(Hq + 2*Hkv) * d, hidden] */
  float* dq_norm_w;  /* [d]; not written (may be NULL) when cfg->qk_norm == 0 */
  float* dk_norm_w;  /* [d] */
  float* dw_o;       /* [hidden, Hq * d] */
} gqa_grads;

/*
 * The layer forward of gqa_layer_forward without a cache, writing every
 * buffer of *saved; out as there (fp32 when cfg->out_f32).  Needs
 * gqa_workspace_bytes(..., GQA_WS_TRAIN_FORWARD) bytes of workspace (the
 * RoPE table; GQA_ERR_WORKSPACE_TOO_SMALL otherwise).
 */
gqa_status gqa_layer_forward_train(const gqa_config* cfg, int32_t batch, int32_t q_len,
                                   const void* x, const void* w_qkv,
                                   const void* q_norm_w, const void* k_norm_w,
                                   const void* w_o, const gqa_saved* saved, void* out,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Gradients of the layer (the exact derivatives of the forward, taken
 * through o_proj, the grouped attention, RoPE, QK-norm and the fused
 * projection in reverse order) for the upstream gradient
 *   dout [batch, q_len, hidden] (cfg->dtype),
 * from the inputs of gqa_layer_forward_train and the *saved buffers it
 * wrote.  Every buffer of *grads is overwritten (not accumulated into).
 * A KV head's gradients sum over the Hq/Hkv query heads it serves; the norm
 * weights' over every token and head.  Needs
 * gqa_workspace_bytes(..., GQA_WS_BACKWARD) bytes of workspace; the
 * results do not depend on timing (no atomics).
 */
gqa_status gqa_layer_backward(const gqa_config* cfg, int32_t batch, int32_t q_len,
                              const void* x, const void* w_qkv, const void* q_norm_w,
                              const void* k_norm_w, const void* w_o, const gqa_saved* saved,
                              const void* dout, const gqa_grads* grads, void* workspace,
                              size_t workspace_bytes, void* stream);

const char* gqa_status_string(gqa_status s);
/* Detail of the last error on the calling thread ("" if none). */
const char* gqa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GQA_H_ */
